/*
 * vbm.h -- C ABI of the MI355X (gfx950) VoxelBlockManager stencil pipeline.
 *
 * An index grid maps each active voxel of a sparse set to an index 1..N
 * (0 = inactive).  A VoxelBlockManager (VBM) cuts the indices into blocks of
 * BlockWidth = 2^log2_width consecutive slots; per block it keeps the first
 * leaf and a jumpMap bit per slot that starts a new leaf.  On that structure
 * the library runs the stencil pipeline on the GPU:
 *   decode    slot -> (leafIndex, voxelOffset) by rank into the jumpMap and
 *             select into the leaf's value mask through its prefix directory
 *             (openvdb PR #2258, "VBM select-based inverse-map decode",
 *             "Summary" and "What changed");
 *   resolve   the 27-tap box, 7-tap cross and 19-tap axis stencils to indices, by a
 *             root-down tree walk per tap or through a per-block table of
 *             neighbour leaves staged in LDS (openvdb PR #2263, "Alternative
 *             stencil resolvers for VoxelBlockManager", "Summary");
 *   deliver   taps materialised into an array or streamed to the consumer in
 *             tap order t = (di+1)*9 + (dj+1)*3 + (dk+1)
 *             (openvdb PR #2262, "NanoVDB VBM: Streaming box-stencil",
 *             "What changed");
 *   gather    per channel, the fp32 sum over the active taps of
 *             sidecar[index*C + ch] (same section of PR #2262).
 *
 * Conventions for every entry point
 *   - Return 0 (VBM_OK) or a negative vbm_status.  Nothing throws.
 *   - Arguments are validated before any launch; on a validation error no
 *     work is enqueued and no output is touched.  Every buffer a kernel reads
 *     or writes (blob, sidecar, outputs) must be memory the GPU can reach:
 *     device, pinned host or managed memory (checked with
 *     hipPointerGetAttributes); anything else, such as pageable host memory,
 *     is refused with VBM_ERR_ARG instead of faulting the GPU.
 *   - GPU work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL = the default stream).  Nothing synchronises.  A failed
 *     launch is reported as VBM_ERR_HIP.
 *   - Device buffers are owned by the caller.  The library allocates no device
 *     memory and keeps no state between calls (the device-side build passes its
 *     state from plan to fill in the caller's workspace).  The one exception is
 *     vbm_build_device_static below, whose workspace is a static array of the
 *     library on each GPU it runs on.
 *   - Coordinates x -> di, y -> dj, z -> dk.  Leaves are 8^3; the voxel offset
 *     inside a leaf is o = (x&7)*64 + (y&7)*8 + (z&7).
 */
#ifndef VBM_H
#define VBM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vbm_status {
  VBM_OK = 0,
  VBM_ERR_ARG = -1,         /* null or host-only pointer, bad width / C / shape / flags, corrupt grid header */
  VBM_ERR_SIZE = -2,        /* grid too large for the library's index or memory limits          */
  VBM_ERR_ALIGN = -3,       /* float buffer not 4-byte aligned                                 */
  VBM_ERR_ALIAS = -4,       /* output overlaps the sidecar (neighbours are read while writing) */
  VBM_ERR_RANGE = -5,       /* coordinate with |c| >= 2^30                                      */
  VBM_ERR_HIP = -6,         /* a HIP launch failed                                              */
  VBM_ERR_UNSUPPORTED = -7, /* a combination the library does not offer (reserved)              */
  VBM_ERR_NOMEM = -8        /* host allocation in vbm_build failed                              */
} vbm_status;

/* flags */
#define VBM_CACHED 0x1        /* resolve through the LDS neighbour-leaf table (else tree walk)  */
#define VBM_STREAMING 0x2     /* stream taps to the consumer (else materialise them first)     */
#define VBM_OP_SUM 0x0        /* cross filter: sum of the 7 taps                                */
#define VBM_OP_LAPLACIAN 0x4  /* cross filter: (sum of active faces) - 6*centre                 */
#define VBM_WIDE_ROWS 0x8     /* filters: reach sidecar rows by 64-bit addresses even below 4 GiB
                                 (taken by itself when (N+1)*C*4 >= 0xFFFFFF00 bytes)           */

#define VBM_MAX_CACHED_LEAVES 16  /* openvdb PR #2263, "Notes": MaxCachedLeaves is 16           */
#define VBM_GRID_MAGIC 0x314D4256u /* "VBM1" */

/*
 * Host-side description of a built grid.  Filled by vbm_build and passed by
 * pointer to every GPU call together with the device copy of the blob.  All
 * offsets are byte offsets into the blob; every section starts 256-byte
 * aligned.  Blob sections:
 *   leaves            n_leaves records of 128 bytes:
 *                       u64 mask[8]   512-bit value mask, bit o = bit o%64 of word o/64
 *                       u64 prefix    7 fields of 9 bits: field k (bits 9k..9k+8) =
 *                                     active voxels in mask words 0..k
 *                       u64 first     index of the leaf's first active voxel
 *                       i32 origin[3] leaf min corner
 *                       u32 lower     parent lower node
 *                       u32 upper     parent upper node (its root tile)
 *                       28 bytes of zero padding
 *   root              n_root tiles of 16 bytes: i32 key[3] (= origin >> 12), u32 upper node;
 *                     sorted by key, lexicographic, signed
 *   upper             n_upper nodes of 32768 u32: lower-node id or 0xFFFFFFFF, slot
 *                     ((x>>7)&31)<<10 | ((y>>7)&31)<<5 | ((z>>7)&31)
 *   lower             n_lower nodes of 4096 u32: leaf id or 0xFFFFFFFF, slot
 *                     ((x>>3)&15)<<8 | ((y>>3)&15)<<4 | ((z>>3)&15)
 *   block_first_leaf  n_blocks u32: leaf owning slot 0 of the block
 *   block_jump        n_blocks * (W/64) u64: jumpMap; bit s set iff slot s >= 1 holds an
 *                     index that starts a leaf
 * Indices follow tree order: root tile, upper slot, lower slot, voxel offset.
 */
typedef struct vbm_grid {
  uint32_t magic;          /* VBM_GRID_MAGIC                                      */
  int32_t log2_width;      /* BlockWidth W = 1 << log2_width, 6..9                */
  uint64_t n_active;       /* N: active voxels; indices are 1..N, 0 = inactive    */
  uint32_t n_leaves;
  uint32_t n_blocks;       /* ceil(N / W)                                         */
  uint32_t n_root;
  uint32_t n_upper;
  uint32_t n_lower;
  uint32_t reserved;
  uint64_t blob_bytes;
  uint64_t off_leaves;
  uint64_t off_root;
  uint64_t off_upper;
  uint64_t off_lower;
  uint64_t off_block_first_leaf;
  uint64_t off_block_jump;
} vbm_grid;

/*
 * Build an index grid and its VBM metadata on the host (not on the timed path).
 *   ijk        host int32 [n][3] coordinates, any order; duplicates are collapsed
 *              (the input is a set).  May be NULL when n == 0.
 *   n          number of coordinates (>= 0)
 *   log2_width 6..9 (BlockWidth 64..512; openvdb PR #2258, "A/B" table)
 *   grid       out: header
 *   host_blob  out: *host_blob = a blob of grid->blob_bytes bytes allocated by the
 *              library; the caller copies it to the device and releases it with
 *              vbm_free_blob.
 * Errors: VBM_ERR_ARG (null pointers, bad width, n < 0), VBM_ERR_RANGE
 * (|coordinate| >= 2^30), VBM_ERR_SIZE (more than 2^32 - 2 active voxels),
 * VBM_ERR_NOMEM.  On error *host_blob is NULL.
 */
int vbm_build(const int32_t* ijk, int64_t n, int log2_width, vbm_grid* grid, void** host_blob);

/* Release a blob returned by vbm_build.  NULL is ignored. */
void vbm_free_blob(void* host_blob);

/*
 * Device-side VBM metadata build: from the leaf masks in d_blob, recompute on
 * the GPU every field the index grid and the VBM derive from them (openvdb PR
 * #2258, "What changed": the 9-bit prefix-sum directory; openvdb PR #2263,
 * "Built on the register-decode API": firstLeafID and the jumpMap of each
 * block):
 *   leaf prefix   field k = active voxels in mask words 0..k
 *   leaf first    1 + active voxels in all earlier leaves (tree order)
 *   block_first_leaf, block_jump   as vbm_build writes them
 * For a blob from vbm_build the result equals the host's bytes.  A caller may
 * edit leaf masks in place on the device and rebuild with this call as long as
 * every leaf keeps at least one active voxel and the total stays n_active (the
 * block sections are sized by it); the new total is written to *d_total (a
 * device u64; NULL to skip) so the caller can check, and *d_total is set to
 * UINT64_MAX instead if an edit left a leaf without any active voxel (the grid
 * is then unusable: a leaf index would no longer follow from the jumpMap rank).
 * The tree sections (root, upper, lower) and the leaf origins are read-only
 * here.  The jumpMap words hold the per-256-leaf partial sums of the leafFirst
 * scan until they are cleared for the block metadata, so the call needs no
 * workspace.  Asynchronous on
 * `stream`; the blob must not be in use by other work on other streams.
 * Errors: VBM_ERR_ARG, VBM_ERR_HIP.
 */
int vbm_build_metadata(const vbm_grid* grid, void* d_blob, uint64_t* d_total, void* stream);

/*
 * Inverse-map decode of every slot (openvdb PR #2258, "What changed": rank of
 * the slot into the block's jumpMap picks the leaf; the prefix directory picks
 * the 64-bit mask word; an in-word select recovers the voxel offset).
 *   d_blob          device copy of the blob
 *   d_leaf_index    device u32 [n_blocks * W]: leaf of slot s of block b at b*W + s
 *   d_voxel_offset  device u16 [n_blocks * W]: voxel offset o in that leaf
 * Slots past the last active index (the final partial block) receive the
 * sentinels 0xFFFFFFFF and 0xFFFF (openvdb PR #2258, "Validation").
 * Errors: VBM_ERR_ARG, VBM_ERR_HIP.
 */
int vbm_decode(const vbm_grid* grid, const void* d_blob, uint32_t* d_leaf_index, uint16_t* d_voxel_offset,
               void* stream);

/*
 * Inverse-map decode by the sweep that the select-based decode replaced
 * (openvdb PR #2258, "Summary": every thread of a block swept all 512 voxel
 * positions of every leaf overlapping the block, O(nLeaves x 512) per block).
 * Kept as the A/B baseline of the decode metric ("A/B" table of that page).
 * Arguments, outputs, sentinels and errors exactly as vbm_decode; the maps are
 * identical.
 */
int vbm_decode_sweep(const vbm_grid* grid, const void* d_blob, uint32_t* d_leaf_index, uint16_t* d_voxel_offset,
                     void* stream);

/*
 * Raw stencil taps of every slot (openvdb PR #2263, "Validation": all taps of
 * every thread written to global memory and compared bytewise).
 *   shape   27 (box, tap t = (di+1)*9 + (dj+1)*3 + (dk+1)),
 *           7 (cross: the box taps 4, 10, 12, 13, 14, 16, 22, i.e. -x, -y, -z,
 *           centre, +z, +y, +x), or
 *           19 (axis stencil, the reach of the 19-tap WENO consumer named in
 *           openvdb PR #2258, "A/B": the centre and +-1..+-3 along each axis, in
 *           ascending lexicographic (di, dj, dk) order; tap 9 = centre)
 *   flags   VBM_CACHED (box: the LDS brick; cross and axis: the per-tap table
 *           of the 7 leaf directions) and VBM_STREAMING (taps written from the
 *           streaming callback instead of a materialised array)
 *   d_taps  device u64 [n_blocks * W * shape]: row b*W + s = taps of slot s of block b;
 *           0 = inactive neighbour; rows of sentinel slots are all 0
 * Errors: VBM_ERR_ARG, VBM_ERR_HIP.
 */
int vbm_stencil_indices(const vbm_grid* grid, const void* d_blob, int shape, int flags, uint64_t* d_taps,
                        void* stream);

/*
 * 27-tap box filter (openvdb PR #2262, "What changed" and "A/B"):
 *   out[g*C + ch] = fp32 sum, in tap order from +0, of sidecar[tap*C + ch] over
 *   the active taps of voxel g (no division).  Row 0 of out is written as 0.
 *   d_sidecar  device f32 [(N+1) * C], row g = channels of index g (row 0 unused)
 *   d_out      device f32 [(N+1) * C]; must not overlap d_sidecar
 *   C          channels >= 1
 *   flags      VBM_CACHED | VBM_STREAMING in any combination (the four resolvers of
 *              openvdb PR #2263, "Summary" table)
 *              and VBM_WIDE_ROWS (below)
 * All four variants give bit-identical outputs.
 * Sidecar size: below 0xFFFFFF00 bytes ((N+1) * C * 4) the rows are read through
 * a bounds-checked buffer resource with 32-bit offsets, an inactive tap being an
 * offset past the end (reads zeros, no branch).  From that size on, or with
 * VBM_WIDE_ROWS, they are read by 64-bit addresses (an inactive tap loads
 * nothing) in chunks of 16, 8 or 4 channels (float4) or of one channel (buffers
 * not 16-byte aligned): somewhat slower, same bits.  A row (C * 4 bytes) must
 * fit in 32 bits.
 * Errors: VBM_ERR_ARG, VBM_ERR_ALIGN, VBM_ERR_ALIAS, VBM_ERR_HIP, and VBM_ERR_SIZE
 * when C * 4 exceeds 2^32 - 1.
 */
int vbm_box_filter(const vbm_grid* grid, const void* d_blob, const float* d_sidecar, float* d_out, int C,
                   int flags, void* stream);

/*
 * 7-tap cross filter (openvdb PR #2263, "Measurements": cross variants
 * accumulate their 7 taps; openvdb PR #2258, "A/B": the 7-point Laplacian):
 *   VBM_OP_SUM        out = fp32 sum, in cross order from +0, over the active taps
 *   VBM_OP_LAPLACIAN  out = (fp32 sum over the active face taps in cross order)
 *                           - fl(6 * centre)
 *   flags: VBM_CACHED, VBM_STREAMING, VBM_WIDE_ROWS and one op.  VBM_STREAMING streams the 7
 *   taps into the gather (the forEachCrossStencil that openvdb PR #2263,
 *   "Notes", leaves out as a wash on its hardware); without it the taps are
 *   materialised (7 entries) first.  All forms give identical bits.
 * Buffers as vbm_box_filter.  Errors: VBM_ERR_ARG, VBM_ERR_ALIGN,
 * VBM_ERR_ALIAS, VBM_ERR_HIP, VBM_ERR_SIZE (as vbm_box_filter).
 */
int vbm_cross_filter(const vbm_grid* grid, const void* d_blob, const float* d_sidecar, float* d_out, int C,
                     int flags, void* stream);

/*
 * 19-tap axis filter: the stencil of the 19-tap WENO consumer (openvdb PR
 * #2258, "A/B"), with its taps accumulated the way the pages' box and cross
 * consumers accumulate theirs (openvdb PR #2263, "Measurements"):
 *   out[g*C + ch] = fp32 sum, in axis tap order (see vbm_stencil_indices) from
 *   +0, of sidecar[tap*C + ch] over the active taps of voxel g.
 *   flags: VBM_CACHED (table of the 7 leaf directions: a reach of 3 < 8 leaves
 *   the leaf in at most one axis), VBM_STREAMING and VBM_WIDE_ROWS.  All forms
 *   give identical bits.
 * Buffers as vbm_box_filter.  Errors: VBM_ERR_ARG, VBM_ERR_ALIGN,
 * VBM_ERR_ALIAS, VBM_ERR_HIP, VBM_ERR_SIZE (as vbm_box_filter).
 */
int vbm_axis_filter(const vbm_grid* grid, const void* d_blob, const float* d_sidecar, float* d_out, int C,
                    int flags, void* stream);

/*
 * WENO consumer of the 19-tap axis stencil (openvdb PR #2258, "A/B", names a
 * 19-tap WENO consumer of the resolved taps; its arithmetic is not given there
 * and is taken as the fifth-order WENO scheme of Jiang and Shu, J. Comput.
 * Phys. 126 (1996), in its Hamilton-Jacobi form):
 *   out[g*C + ch] = |grad u|^2 of channel ch at voxel g by Godunov's upwind
 *   rule: per axis, the left- and right-biased fifth-order WENO derivatives
 *   from the seven values u[-3..3] along that axis (unit spacing); if the
 *   centre value is > 0, max(max(left, 0)^2, min(right, 0)^2), else
 *   max(min(left, 0)^2, max(right, 0)^2); summed over x, y, z.
 *   An inactive tap (index 0) reads sidecar row 0, the background value; this
 *   consumer, unlike the summing filters, therefore reads row 0.
 *   The fp32 evaluation order is fixed operation by operation (documented with
 *   the kernel); no contraction, correctly rounded division, denormals kept.
 *   flags: VBM_CACHED (the 7-direction table of the axis stencil) and
 *   VBM_STREAMING (taps resolved as their loads are issued instead of into an
 *   array first), and VBM_WIDE_ROWS (as vbm_box_filter; all channels in one
 *   launch).  All forms give identical bits.  Row 0 of out is written as 0.
 * Buffers as vbm_box_filter.  Errors: VBM_ERR_ARG, VBM_ERR_ALIGN,
 * VBM_ERR_ALIAS, VBM_ERR_HIP, VBM_ERR_SIZE (as vbm_box_filter).
 */
int vbm_weno_filter(const vbm_grid* grid, const void* d_blob, const float* d_sidecar, float* d_out, int C,
                    int flags, void* stream);

/*
 * Device-side build of the same grid from coordinates already on the GPU: the
 * blob is byte for byte the one vbm_build writes for the same coordinates and
 * width (openvdb PR #2258, "What changed": leaf masks and the 9-bit prefix-sum
 * directory; openvdb PR #2263, "Built on the register-decode API": firstLeafID
 * and the jumpMap of each block).  Three calls:
 *
 * vbm_build_device_workspace(n, &bytes)
 *   Bytes of device workspace the build of n coordinates needs (about 40 B per
 *   coordinate plus the sort's temporary storage).  Needs the GPU (the sort's
 *   storage depends on the device).  Errors: VBM_ERR_ARG, VBM_ERR_SIZE
 *   (n >= 2^32 - 1), VBM_ERR_HIP.
 *
 * vbm_build_device_plan(d_ijk, n, log2_width, d_workspace, workspace_bytes, grid, stream)
 *   d_ijk         device int32 [n][3] coordinates, any order, duplicates allowed
 *   d_workspace   caller-owned device memory of at least the queried bytes
 *   grid          out: the header, including blob_bytes
 *   Sorts the tree-order keys and counts voxels, leaves and tree nodes on
 *   `stream`, then WAITS for the stream (the blob's size depends on the data:
 *   this is the one entry point of the library that synchronises).  The
 *   workspace keeps the sorted keys for vbm_build_device_fill.
 *   Errors: VBM_ERR_ARG, VBM_ERR_SIZE (workspace too small, more than 2^32 - 2
 *   voxels), VBM_ERR_RANGE (|coordinate| >= 2^30), VBM_ERR_UNSUPPORTED (the
 *   bounding box of the 4096^3 root tiles holds more than 2^28 tiles),
 *   VBM_ERR_HIP.
 *
 * vbm_build_device_fill(grid, n, d_workspace, workspace_bytes, d_blob, stream)
 *   grid, n, d_workspace, workspace_bytes: as returned by / given to the plan,
 *   with the workspace untouched since; d_blob: caller-owned device memory of
 *   grid->blob_bytes bytes.  Writes the whole blob asynchronously on `stream`.
 *   Errors: VBM_ERR_ARG (including a header the plan did not write),
 *   VBM_ERR_SIZE, VBM_ERR_HIP.
 */
int vbm_build_device_workspace(int64_t n, uint64_t* workspace_bytes);
int vbm_build_device_plan(const int32_t* d_ijk, int64_t n, int log2_width, void* d_workspace,
                          uint64_t workspace_bytes, vbm_grid* grid, void* stream);
int vbm_build_device_fill(const vbm_grid* grid, int64_t n, void* d_workspace, uint64_t workspace_bytes,
                          void* d_blob, void* stream);

/*
 * The device-side build without any allocation, for callers that cannot
 * allocate device memory (tight loops, harnesses that forbid hipMalloc): plan
 * and fill in one call, with the workspace in a static array of the library on
 * the current GPU instead of a caller workspace.
 *   d_ijk, n, log2_width, grid, stream: as vbm_build_device_plan (this call
 *              waits for the stream once, as the plan does)
 *   d_blob     caller-owned device memory of blob_capacity bytes; filled when
 *              blob_capacity >= grid->blob_bytes
 * Limit: n <= 1,048,576 coordinates (a 48 MiB array that every GPU the library
 * runs on holds until the process ends).  Calls on one GPU share that array:
 * calls that overlap in time on the same GPU (other host threads, other
 * streams) race and must not be issued.
 * Errors: as the plan and fill; VBM_ERR_SIZE also for n above the limit, and
 * for d_blob NULL or blob_capacity below grid->blob_bytes (grid then holds the
 * header, so the caller knows the size; nothing is written to d_blob).
 * Calls no hipMalloc, hipFree or allocating library routine.
 */
int vbm_build_device_static(const int32_t* d_ijk, int64_t n, int log2_width, void* d_blob, uint64_t blob_capacity,
                            vbm_grid* grid, void* stream);

/* Static English text for a status code. */
const char* vbm_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* VBM_H */

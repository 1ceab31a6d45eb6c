// Device-side build of the index grid and its VoxelBlockManager metadata from
// a set of coordinates already on the GPU (the same blob, byte for byte, as
// the host builder in vbm_build.cpp).
//
// The blob is what every stage of the pipeline reads: per leaf the 512-bit
// value mask, the 9-bit prefix-sum directory and the first index (openvdb PR
// #2258, "What changed"), the tree the resolvers walk (openvdb PR #2263,
// "Summary"), and per block firstLeafID and the jumpMap (openvdb PR #2263,
// "Built on the register-decode API": the first leaf, spanned leaves =
// 1 + popcount(jumpMap)).
//
// Plan (vbm_build_device_plan), on the caller's stream and workspace:
//   1. bounding box of the root tiles (x >> 12, ...) and the range check;
//   2. one 64-bit key per coordinate: the root tile's position in that box,
//      linearised x-major (so keys order root tiles lexicographically, as the
//      host's dense root ranks do), above the 36-bit position in the tile
//      (upper slot, lower slot, voxel offset, each x-major) -- tree order;
//   3. radix sort of the keys over the bits in use, then duplicates removed;
//   4. counts of voxels, leaves (key >> 9), lower nodes (key >> 21) and root
//      tiles (key >> 36), read back by the host, which lays out the blob.
// Fill (vbm_build_device_fill), asynchronous:
//   leaf ids, lower-node ids and root ranks by scans over start flags; one
//   work-item per leaf builds its mask from its run of sorted keys and writes
//   its record (prefix directory from the mask) and its entries in the lower,
//   upper and root sections; the block metadata by scatter: each leaf sets the jumpMap
//   bit of its first index and writes firstLeafID of every block whose first
//   index it holds (no search).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <vector>

#include <rocprim/device/device_radix_sort.hpp>

#include "vbm.h"
#include "vbm_host_checks.hpp"
#include "vbm_layout.hpp"

namespace {

constexpr int32_t kCoordLimit = int32_t(1) << 30;
constexpr uint32_t kNone = 0xFFFFFFFFu;

// First 256 bytes of the workspace.
struct BuildHeader {
  int32_t lo[3];         // root-tile bounding box (inclusive), x >> 12 etc.
  int32_t hi[3];
  uint32_t status;       // bit 0: a coordinate with |c| >= 2^30
  uint32_t pad;
  uint64_t n_unique;     // N after removing duplicates
  unsigned long long n_leaves, n_lower, n_root;
};
static_assert(sizeof(BuildHeader) <= 256, "workspace header");

// Workspace sections for n coordinates (256-byte aligned offsets).
struct WorkspaceLayout {
  uint64_t keys_a, keys_b, leaf_of_voxel, leaf_key, leaf_first, lower_id, root_rank, temp, temp_bytes, total;
};

WorkspaceLayout workspace_layout(uint64_t n, uint64_t temp_bytes) {
  using vbm_layout::align_up;
  WorkspaceLayout w;
  uint64_t off = 256;
  w.keys_a = off;        off = align_up(off + 8 * n);
  w.keys_b = off;        off = align_up(off + 8 * n);
  w.leaf_of_voxel = off; off = align_up(off + 4 * n);
  w.leaf_key = off;      off = align_up(off + 8 * n);
  w.leaf_first = off;    off = align_up(off + 4 * n);
  w.lower_id = off;      off = align_up(off + 4 * n);
  w.root_rank = off;     off = align_up(off + 4 * n);
  w.temp = off;          off = align_up(off + temp_bytes);
  w.temp_bytes = temp_bytes;
  w.total = off;
  return w;
}

// ---------------------------------------------------------------------------
// scans of start flags (duplicate removal and the leaf / lower-node / root ids)
// ---------------------------------------------------------------------------
// Inclusive scan of flag(i), i < count, in three launches: per tile of
// kScanTile elements the number of set flags; one workgroup turns the tile
// totals into exclusive offsets (and writes the grand total); per tile again
// a block scan in index order, each element handed to sink(i, inclusive, flag).
// Tiles are read 256 consecutive elements at a time (coalesced).
constexpr uint32_t kScanThreads = 256;
constexpr uint32_t kScanItems = 16;
constexpr uint64_t kScanTile = uint64_t(kScanThreads) * kScanItems;

uint64_t scan_tiles(uint64_t count) { return (count + kScanTile - 1) / kScanTile; }

// Inclusive prefix sum over the 256 work-items of the workgroup; *total gets
// the workgroup's sum.  All work-items must call it.
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* total) {
  __shared__ uint32_t wave_sum[kScanThreads / 64];
  const uint32_t lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_up(v, d);
    if (lane >= uint32_t(d)) v += t;
  }
  if (lane == 63) wave_sum[wave] = v;
  __syncthreads();
  uint32_t before = 0, sum = 0;
#pragma unroll
  for (uint32_t k = 0; k < kScanThreads / 64; ++k) {
    before += k < wave ? wave_sum[k] : 0u;
    sum += wave_sum[k];
  }
  __syncthreads();  // wave_sum is reused by the next call
  *total = sum;
  return before + v;
}

template <class Flag>
__global__ void __launch_bounds__(kScanThreads) k_scan_tile_counts(Flag flag, uint64_t count, uint32_t* tile_sum) {
  const uint64_t base = blockIdx.x * kScanTile;
  uint32_t c = 0;
#pragma unroll
  for (uint32_t j = 0; j < kScanItems; ++j) {
    const uint64_t i = base + j * kScanThreads + threadIdx.x;
    c += i < count ? flag(i) : 0u;
  }
  uint32_t total;
  block_inclusive_scan(c, &total);
  if (threadIdx.x == 0) tile_sum[blockIdx.x] = total;
}

// One workgroup: tile_sum[0 .. T) becomes exclusive offsets; *grand = the sum.
__global__ void __launch_bounds__(1024) k_scan_tile_offsets(uint32_t* tile_sum, uint64_t T, uint64_t* grand) {
  __shared__ uint64_t part[1024];
  const uint64_t t = threadIdx.x, per = (T + blockDim.x - 1) / blockDim.x;
  const uint64_t a = t * per < T ? t * per : T, e = a + per < T ? a + per : T;
  uint64_t sum = 0;
  for (uint64_t k = a; k < e; ++k) sum += tile_sum[k];
  part[t] = sum;
  __syncthreads();
  for (uint32_t d = 1; d < blockDim.x; d <<= 1) {
    const uint64_t v = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  uint64_t run = t ? part[t - 1] : 0;
  for (uint64_t k = a; k < e; ++k) {
    const uint32_t c = tile_sum[k];
    tile_sum[k] = uint32_t(run);
    run += c;
  }
  if (t == blockDim.x - 1 && grand) *grand = part[t];
}

template <class Flag, class Sink>
__global__ void __launch_bounds__(kScanThreads) k_scan_apply(Flag flag, uint64_t count, const uint32_t* tile_off,
                                                             Sink sink) {
  const uint64_t base = blockIdx.x * kScanTile;
  uint32_t running = tile_off[blockIdx.x];
  for (uint32_t j = 0; j < kScanItems; ++j) {  // block-uniform trip count: every barrier is reached by all
    const uint64_t i = base + j * kScanThreads + threadIdx.x;
    const uint32_t f = i < count ? flag(i) : 0u;
    uint32_t total;
    const uint32_t incl = block_inclusive_scan(f, &total);
    if (i < count) sink(i, running + incl, f);
    running += total;
  }
}

// Start flags over sorted keys: element i starts a new group of key >> shift,
// i.e. keys i - 1 and i differ in a bit at or above `shift` (tested with a
// mask, so no shift by a run-time count is emitted).
struct KeyGroupStart {
  const uint64_t* keys;
  uint64_t high;  // ~((1 << shift) - 1): all ones for shift 0 (any difference starts a group)
  __host__ __device__ uint32_t operator()(uint64_t i) const {
    return i == 0 || ((keys[i] ^ keys[i - 1]) & high) != 0 ? 1u : 0u;
  }
};
KeyGroupStart group_start(const uint64_t* keys, uint32_t shift) {
  return KeyGroupStart{keys, shift >= 64 ? uint64_t(0) : ~((uint64_t(1) << shift) - 1)};
}

// Sinks: the inclusive count itself, or (duplicate removal) the key moved to
// its place among the distinct keys.
struct WriteCount {
  uint32_t* out;
  __device__ void operator()(uint64_t i, uint32_t incl, uint32_t) const { out[i] = incl; }
};
struct CompactKey {
  const uint64_t* in;
  uint64_t* out;
  __device__ void operator()(uint64_t i, uint32_t incl, uint32_t f) const {
    if (f) out[incl - 1] = in[i];
  }
};

// Inclusive scan of flag over count elements with sink; the tile totals live
// in `tile_sum` (scan_tiles(count) entries).
template <class Flag, class Sink>
void flag_scan(Flag flag, uint64_t count, uint32_t* tile_sum, uint64_t* grand, Sink sink, hipStream_t st) {
  const uint64_t T = scan_tiles(count);
  if (T == 0) return;
  hipLaunchKernelGGL(k_scan_tile_counts<Flag>, dim3(uint32_t(T)), dim3(kScanThreads), 0, st, flag, count, tile_sum);
  hipLaunchKernelGGL(k_scan_tile_offsets, dim3(1), dim3(1024), 0, st, tile_sum, T, grand);
  hipLaunchKernelGGL((k_scan_apply<Flag, Sink>), dim3(uint32_t(T)), dim3(kScanThreads), 0, st, flag, count, tile_sum,
                     sink);
}

// Temporary storage of the plan and fill for n keys: the radix sort's (from
// rocPRIM's size query) or the scans' tile totals, whichever is larger.
hipError_t temp_storage_bytes(uint64_t n, hipStream_t st, uint64_t* bytes) {
  size_t sort = 0;
  uint64_t* k = nullptr;
  hipError_t e = rocprim::radix_sort_keys(nullptr, sort, k, k, n, 0, 64, st);
  if (e != hipSuccess) return e;
  const uint64_t tiles = 4 * scan_tiles(n);
  *bytes = sort > tiles ? sort : tiles;
  return hipSuccess;
}

__global__ void k_build_init(BuildHeader* h) {
  if (threadIdx.x == 0) {
    for (int a = 0; a < 3; ++a) {
      h->lo[a] = INT32_MAX;
      h->hi[a] = INT32_MIN;
    }
    h->status = 0;
    h->n_unique = 0;
    h->n_leaves = h->n_lower = h->n_root = 0;
  }
}

__device__ __forceinline__ int32_t wave_min(int32_t v) {
  for (int d = 32; d > 0; d >>= 1) v = min(v, __shfl_xor(v, d));
  return v;
}
__device__ __forceinline__ int32_t wave_max(int32_t v) {
  for (int d = 32; d > 0; d >>= 1) v = max(v, __shfl_xor(v, d));
  return v;
}

// Root-tile bounding box and the coordinate range check: per work-item, then
// per wave (shuffles), then per workgroup (LDS), then one set of atomics per
// workgroup (the grid is capped, so there are few).
__global__ void __launch_bounds__(256) k_build_bounds(const int32_t* __restrict__ ijk, uint64_t n, BuildHeader* h) {
  __shared__ int32_t wlo[4][3], whi[4][3];
  __shared__ uint32_t wbad[4];
  int32_t lo[3] = {INT32_MAX, INT32_MAX, INT32_MAX}, hi[3] = {INT32_MIN, INT32_MIN, INT32_MIN};
  bool bad = false;
  for (uint64_t i = blockIdx.x * uint64_t(blockDim.x) + threadIdx.x; i < n; i += uint64_t(gridDim.x) * blockDim.x) {
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const int32_t c = ijk[3 * i + a];
      bad |= c <= -kCoordLimit || c >= kCoordLimit;
      lo[a] = min(lo[a], c >> 12);
      hi[a] = max(hi[a], c >> 12);
    }
  }
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    lo[a] = wave_min(lo[a]);
    hi[a] = wave_max(hi[a]);
  }
  const bool any_bad = __any(bad);
  const uint32_t w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    for (int a = 0; a < 3; ++a) {
      wlo[w][a] = lo[a];
      whi[w][a] = hi[a];
    }
    wbad[w] = any_bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t waves = blockDim.x >> 6;
    for (uint32_t k = 1; k < waves; ++k)
      for (int a = 0; a < 3; ++a) {
        wlo[0][a] = min(wlo[0][a], wlo[k][a]);
        whi[0][a] = max(whi[0][a], whi[k][a]);
        wbad[0] |= wbad[k];
      }
    for (int a = 0; a < 3; ++a) {
      atomicMin(&h->lo[a], wlo[0][a]);
      atomicMax(&h->hi[a], whi[0][a]);
    }
    if (wbad[0]) atomicOr(&h->status, 1u);
  }
}

// Position of a voxel inside its root tile, in tree order: upper slot, lower
// slot, voxel offset, each x-major (bits 35..0).
__device__ __forceinline__ uint64_t in_tile_position(int32_t x, int32_t y, int32_t z) {
  const uint64_t ux = (uint32_t(x) >> 7) & 31, uy = (uint32_t(y) >> 7) & 31, uz = (uint32_t(z) >> 7) & 31;
  const uint64_t lx = (uint32_t(x) >> 3) & 15, ly = (uint32_t(y) >> 3) & 15, lz = (uint32_t(z) >> 3) & 15;
  const uint64_t vx = uint32_t(x) & 7, vy = uint32_t(y) & 7, vz = uint32_t(z) & 7;
  return (ux << 31) | (uy << 26) | (uz << 21) | (lx << 17) | (ly << 13) | (lz << 9) | (vx << 6) | (vy << 3) | vz;
}

struct TileBox {
  int32_t lo[3];
  uint64_t span_y, span_z;  // tiles along y and z
};

__device__ __forceinline__ TileBox tile_box(const BuildHeader* h) {
  TileBox b;
  for (int a = 0; a < 3; ++a) b.lo[a] = h->lo[a];
  b.span_y = uint64_t(int64_t(h->hi[1]) - h->lo[1] + 1);
  b.span_z = uint64_t(int64_t(h->hi[2]) - h->lo[2] + 1);
  return b;
}

__global__ void __launch_bounds__(256) k_build_keys(const int32_t* __restrict__ ijk, uint64_t n, const BuildHeader* h,
                                                    uint64_t* __restrict__ keys) {
  const TileBox box = tile_box(h);
  for (uint64_t i = blockIdx.x * uint64_t(blockDim.x) + threadIdx.x; i < n; i += uint64_t(gridDim.x) * blockDim.x) {
    const int32_t x = ijk[3 * i], y = ijk[3 * i + 1], z = ijk[3 * i + 2];
    const uint64_t tile = (uint64_t(int64_t(x >> 12) - box.lo[0]) * box.span_y + uint64_t(int64_t(y >> 12) - box.lo[1])) *
                              box.span_z +
                          uint64_t(int64_t(z >> 12) - box.lo[2]);
    keys[i] = (tile << 36) | in_tile_position(x, y, z);
  }
}

// Counts of leaves, lower nodes and root tiles among the N sorted unique keys:
// per wave (shuffles), per workgroup (LDS), one set of atomics per workgroup.
__global__ void __launch_bounds__(256) k_build_counts(const uint64_t* __restrict__ keys, BuildHeader* h) {
  __shared__ uint32_t part[4][3];
  const uint64_t N = h->n_unique;
  uint32_t leaves = 0, lowers = 0, roots = 0;
  for (uint64_t i = blockIdx.x * uint64_t(blockDim.x) + threadIdx.x; i < N; i += uint64_t(gridDim.x) * blockDim.x) {
    const uint64_t k = keys[i], p = i ? keys[i - 1] : ~k;
    leaves += (k >> 9) != (p >> 9);
    lowers += (k >> 21) != (p >> 21);
    roots += (k >> 36) != (p >> 36);
  }
  for (int d = 32; d > 0; d >>= 1) {
    leaves += __shfl_xor(leaves, d);
    lowers += __shfl_xor(lowers, d);
    roots += __shfl_xor(roots, d);
  }
  const uint32_t w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    part[w][0] = leaves;
    part[w][1] = lowers;
    part[w][2] = roots;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long sum[3] = {0, 0, 0};
    for (uint32_t k = 0; k < (blockDim.x >> 6); ++k)
      for (int a = 0; a < 3; ++a) sum[a] += part[k][a];
    atomicAdd(&h->n_leaves, sum[0]);
    atomicAdd(&h->n_lower, sum[1]);
    atomicAdd(&h->n_root, sum[2]);
  }
}

// Blob initialisation: zero everywhere except the upper and lower node
// sections, whose entries start as kNone (no child).  16-byte stores.
__global__ void __launch_bounds__(256) k_fill_init(uint4* __restrict__ blob, uint64_t pieces, uint64_t none_a0,
                                                   uint64_t none_a1, uint64_t none_b0, uint64_t none_b1) {
  for (uint64_t i = blockIdx.x * uint64_t(blockDim.x) + threadIdx.x; i < pieces; i += uint64_t(gridDim.x) * blockDim.x) {
    const bool none = (i >= none_a0 && i < none_a1) || (i >= none_b0 && i < none_b1);
    blob[i] = none ? make_uint4(kNone, kNone, kNone, kNone) : make_uint4(0u, 0u, 0u, 0u);
  }
}

// Record of each leaf start: its key >> 9 and the index of its first voxel.
// (Every id below is checked against the header's counts, so a header that
// does not belong to the workspace can give a wrong blob but no access outside
// the buffers.)
__global__ void __launch_bounds__(256) k_fill_leaf_starts(const uint64_t* __restrict__ keys, uint64_t N, uint64_t L,
                                                          const uint32_t* __restrict__ leaf_of_voxel,
                                                          uint64_t* __restrict__ leaf_key,
                                                          uint32_t* __restrict__ leaf_first) {
  for (uint64_t i = blockIdx.x * uint64_t(blockDim.x) + threadIdx.x; i < N; i += uint64_t(gridDim.x) * blockDim.x) {
    if (i == 0 || (keys[i] >> 9) != (keys[i - 1] >> 9)) {
      const uint32_t l = leaf_of_voxel[i] - 1;  // inclusive count of starts
      if (l >= L) continue;
      leaf_key[l] = keys[i] >> 9;
      leaf_first[l] = uint32_t(i + 1);
    }
  }
}

struct BlobLeaf {  // the 128-byte leaf record of include/vbm.h
  uint64_t mask[8];
  uint64_t prefix;
  uint64_t first;
  int32_t origin[3];
  uint32_t lower;
  uint32_t upper;
  uint32_t pad[7];
};
static_assert(sizeof(BlobLeaf) == 128, "leaf record");

struct BlobSections {
  BlobLeaf* leaves;
  int32_t* root;       // 4 ints per tile: key x, y, z, upper node
  uint32_t* upper;     // n_root * 32768
  uint32_t* lower;     // n_lower * 4096
  uint32_t n_root, n_lower;
};

// One work-item per leaf: the value mask from the leaf's run of sorted keys
// (voxels first .. next leaf's first - 1), prefix directory, first index,
// origin, parents; the leaf's entry in its lower node, and (for the first leaf
// of a lower node / root tile) the entries of the upper node and the root table.
__global__ void __launch_bounds__(256) k_fill_leaves(uint64_t L, uint64_t N, const uint64_t* __restrict__ keys,
                                                     const uint64_t* __restrict__ leaf_key,
                                                     const uint32_t* __restrict__ leaf_first,
                                                     const uint32_t* __restrict__ lower_id,
                                                     const uint32_t* __restrict__ root_rank, const BuildHeader* h,
                                                     BlobSections blob) {
  const TileBox box = tile_box(h);
  for (uint64_t l = blockIdx.x * uint64_t(blockDim.x) + threadIdx.x; l < L; l += uint64_t(gridDim.x) * blockDim.x) {
    BlobLeaf& rec = blob.leaves[l];
    const uint64_t end = l + 1 < L ? uint64_t(leaf_first[l + 1]) - 1 : N;  // one past the leaf's last voxel
    uint32_t half[16] = {};  // the mask as 32-bit halves (32-bit shifts only)
    for (uint64_t i = uint64_t(leaf_first[l]) - 1; i < end && i < N; ++i) {
      const uint32_t o = uint32_t(keys[i] & 511);
#pragma unroll
      for (int k = 0; k < 16; ++k) half[k] |= (o >> 5) == uint32_t(k) ? 1u << (o & 31) : 0u;
    }
    uint64_t count = 0, dir = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      rec.mask[w] = uint64_t(half[2 * w]) | (uint64_t(half[2 * w + 1]) << 32);
      count += __popc(half[2 * w]) + __popc(half[2 * w + 1]);
      if (w < 7) dir |= count << (9 * w);
    }
    const uint64_t lk = leaf_key[l];
    const uint64_t tile = lk >> 27;  // position of the root tile in the bounding box
    const int32_t rx = box.lo[0] + int32_t(tile / (box.span_y * box.span_z));
    const int32_t ry = box.lo[1] + int32_t((tile / box.span_z) % box.span_y);
    const int32_t rz = box.lo[2] + int32_t(tile % box.span_z);
    const uint32_t t = uint32_t(lk & ((uint64_t(1) << 27) - 1));  // upper slot (15 bits) | lower slot (12 bits)
    const uint32_t low = lower_id[l] - 1, up = root_rank[l] - 1;
    if (low >= blob.n_lower || up >= blob.n_root) continue;
    rec.prefix = dir;
    rec.first = leaf_first[l];
    rec.origin[0] = rx * 4096 + int32_t((t >> 22) & 31) * 128 + int32_t((t >> 8) & 15) * 8;
    rec.origin[1] = ry * 4096 + int32_t((t >> 17) & 31) * 128 + int32_t((t >> 4) & 15) * 8;
    rec.origin[2] = rz * 4096 + int32_t((t >> 12) & 31) * 128 + int32_t(t & 15) * 8;
    rec.lower = low;
    rec.upper = up;
    blob.lower[uint64_t(low) * 4096 + (t & 4095)] = uint32_t(l);
    const uint64_t plk = l ? leaf_key[l - 1] : ~lk;
    if ((lk >> 12) != (plk >> 12)) blob.upper[uint64_t(up) * 32768 + (t >> 12)] = low;
    if ((lk >> 27) != (plk >> 27)) {
      int32_t* r = blob.root + 4 * uint64_t(up);
      r[0] = rx;
      r[1] = ry;
      r[2] = rz;
      r[3] = int32_t(up);
    }
  }
}

// Block metadata by scatter: leaf l (first index f, c voxels) sets the jumpMap
// bit of slot (f - 1) % W of block (f - 1) / W unless it starts the block, and
// is firstLeafID of every block whose first index 1 + bW lies in [f, f + c).
__global__ void __launch_bounds__(256) k_fill_blocks(uint64_t L, uint64_t N, int log2w,
                                                     const uint32_t* __restrict__ leaf_first,
                                                     uint32_t* __restrict__ block_first_leaf,
                                                     uint64_t* block_jump) {
  const uint64_t W = uint64_t(1) << log2w, words = W / 64;
  for (uint64_t l = blockIdx.x * uint64_t(blockDim.x) + threadIdx.x; l < L; l += uint64_t(gridDim.x) * blockDim.x) {
    const uint64_t f = leaf_first[l];
    const uint64_t end = l + 1 < L ? uint64_t(leaf_first[l + 1]) : N + 1;  // one past the leaf's last index
    const uint64_t s = (f - 1) & (W - 1), b = (f - 1) >> log2w;
    if (s != 0)  // the bit's 32-bit half of the jumpMap word (32-bit shifts only)
      atomicOr(reinterpret_cast<uint32_t*>(&block_jump[b * words + s / 64]) + ((s >> 5) & 1), 1u << (s & 31));
    for (uint64_t bb = (f - 1 + W - 1) >> log2w; 1 + (bb << log2w) < end; ++bb) block_first_leaf[bb] = uint32_t(l);
  }
}

// Workspace of vbm_build_device_static, for callers that cannot allocate: a
// static array on every GPU the library runs on (held until the process
// ends), reached from host code only through the address hipGetSymbolAddress
// returns for the current device.
constexpr uint64_t kStaticMaxCoords = uint64_t(1) << 20;
constexpr uint64_t kStaticScratchBytes = uint64_t(48) << 20;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// Address of `scratch` on the current device, looked up once per device.
int static_scratch(void** ptr) {
  static std::mutex lock;
  static std::vector<void*> per_device;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return VBM_ERR_HIP;
  std::lock_guard<std::mutex> guard(lock);
  if (per_device.size() <= size_t(dev)) per_device.resize(size_t(dev) + 1, nullptr);
  if (!per_device[size_t(dev)]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return VBM_ERR_HIP;
    }
    per_device[size_t(dev)] = p;
  }
  *ptr = per_device[size_t(dev)];
  return VBM_OK;
}

uint32_t grid_for(uint64_t items) {
  const uint64_t g = (items + 255) / 256;
  return uint32_t(g < 1 ? 1 : (g > 8192 ? 8192 : g));
}

// Runs a rocPRIM call f(temp, bytes) after checking, with a size query
// f(nullptr, bytes), that its temporary storage fits the workspace's.
// Grid of the reduction kernels: at most 1024 workgroups of 256, so the
// per-workgroup atomics stay few.
uint32_t reduce_grid(uint64_t items) {
  const uint64_t g = (items + 255) / 256;
  return uint32_t(g < 1 ? 1 : (g > 1024 ? 1024 : g));
}

template <class F>
int run_with_temp(void* temp, uint64_t temp_bytes, F&& f) {
  size_t need = 0;
  if (f(nullptr, need) != hipSuccess) return VBM_ERR_HIP;
  if (need > temp_bytes) return VBM_ERR_SIZE;
  size_t have = size_t(temp_bytes);
  return f(temp, have) == hipSuccess ? VBM_OK : VBM_ERR_HIP;
}

}  // namespace

extern "C" int vbm_build_device_workspace(int64_t n, uint64_t* workspace_bytes) {
  if (!workspace_bytes || n < 0) return VBM_ERR_ARG;
  if (uint64_t(n) >= 0xFFFFFFFFull) return VBM_ERR_SIZE;
  uint64_t temp = 0;
  if (temp_storage_bytes(uint64_t(n), nullptr, &temp) != hipSuccess) {
    (void)hipGetLastError();
    return VBM_ERR_HIP;
  }
  *workspace_bytes = workspace_layout(uint64_t(n), temp).total;
  return VBM_OK;
}

extern "C" int vbm_build_device_plan(const int32_t* d_ijk, int64_t n, int log2_width, void* d_workspace,
                                     uint64_t workspace_bytes, vbm_grid* grid, void* stream) {
  if (!grid || !d_workspace || n < 0 || (n > 0 && !d_ijk)) return VBM_ERR_ARG;
  if (log2_width < 6 || log2_width > 9) return VBM_ERR_ARG;
  if (uint64_t(n) >= 0xFFFFFFFFull) return VBM_ERR_SIZE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint64_t temp = 0;
  if (temp_storage_bytes(uint64_t(n), st, &temp) != hipSuccess) {
    (void)hipGetLastError();
    return VBM_ERR_HIP;
  }
  const WorkspaceLayout w = workspace_layout(uint64_t(n), temp);
  if (workspace_bytes < w.total) return VBM_ERR_SIZE;
  int rc = n > 0 ? vbm_host::check_kernel_memory({d_ijk, d_workspace}) : vbm_host::check_kernel_memory({d_workspace});
  if (rc) return rc;
  uint8_t* ws = static_cast<uint8_t*>(d_workspace);
  BuildHeader* h = reinterpret_cast<BuildHeader*>(ws);
  uint64_t* keys_a = reinterpret_cast<uint64_t*>(ws + w.keys_a);
  uint64_t* keys_b = reinterpret_cast<uint64_t*>(ws + w.keys_b);
  hipLaunchKernelGGL(k_build_init, dim3(1), dim3(64), 0, st, h);
  if (n > 0) hipLaunchKernelGGL(k_build_bounds, dim3(reduce_grid(uint64_t(n))), dim3(256), 0, st, d_ijk, uint64_t(n), h);
  BuildHeader host;
  if (hipMemcpyAsync(&host, h, sizeof(host), hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return VBM_ERR_HIP;
  if (host.status & 1u) return VBM_ERR_RANGE;
  unsigned key_bits = 36;
  if (n > 0) {
    const uint64_t tiles = uint64_t(int64_t(host.hi[0]) - host.lo[0] + 1) * uint64_t(int64_t(host.hi[1]) - host.lo[1] + 1) *
                           uint64_t(int64_t(host.hi[2]) - host.lo[2] + 1);
    unsigned tile_bits = 0;
    while (tile_bits < 64 && (uint64_t(1) << tile_bits) < tiles) ++tile_bits;
    if (tile_bits > 28) return VBM_ERR_UNSUPPORTED;  // the key keeps 28 bits for the root tile
    key_bits += tile_bits;
    hipLaunchKernelGGL(k_build_keys, dim3(grid_for(uint64_t(n))), dim3(256), 0, st, d_ijk, uint64_t(n), h, keys_a);
    void* temp = ws + w.temp;
    const uint64_t nn = uint64_t(n);
    if ((rc = run_with_temp(temp, w.temp_bytes, [&](void* t, size_t& b) {
           return rocprim::radix_sort_keys(t, b, keys_a, keys_b, nn, 0, key_bits, st);
         })))
      return rc;
    // duplicates removed: every key that differs from its predecessor moves to its place
    flag_scan(group_start(keys_b, 0), nn, static_cast<uint32_t*>(temp), &h->n_unique, CompactKey{keys_b, keys_a}, st);
    hipLaunchKernelGGL(k_build_counts, dim3(reduce_grid(uint64_t(n))), dim3(256), 0, st, keys_a, h);
    if (hipMemcpyAsync(&host, h, sizeof(host), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return VBM_ERR_HIP;
  }
  if ((rc = vbm_host::launch_status())) return rc;
  return vbm_layout::layout(host.n_unique, host.n_leaves, host.n_root, host.n_lower, log2_width, grid);
}

extern "C" int vbm_build_device_fill(const vbm_grid* grid, int64_t n, void* d_workspace, uint64_t workspace_bytes,
                                     void* d_blob, void* stream) {
  if (!grid || grid->magic != VBM_GRID_MAGIC || !d_workspace || !d_blob || n < 0) return VBM_ERR_ARG;
  if (grid->log2_width < 6 || grid->log2_width > 9 || grid->n_active > uint64_t(n) || grid->n_leaves > grid->n_active)
    return VBM_ERR_ARG;
  if (uint64_t(n) >= 0xFFFFFFFFull) return VBM_ERR_SIZE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint64_t temp = 0;
  if (temp_storage_bytes(uint64_t(n), st, &temp) != hipSuccess) {
    (void)hipGetLastError();
    return VBM_ERR_HIP;
  }
  const WorkspaceLayout w = workspace_layout(uint64_t(n), temp);
  if (workspace_bytes < w.total) return VBM_ERR_SIZE;
  vbm_grid check;
  if (vbm_layout::layout(grid->n_active, grid->n_leaves, grid->n_root, grid->n_lower, grid->log2_width, &check) ||
      std::memcmp(&check, grid, sizeof(check)) != 0)
    return VBM_ERR_ARG;  // not a header that vbm_build_device_plan wrote
  int rc = vbm_host::check_kernel_memory({d_workspace, d_blob});
  if (rc) return rc;
  uint8_t* ws = static_cast<uint8_t*>(d_workspace);
  uint8_t* blob = static_cast<uint8_t*>(d_blob);
  const BuildHeader* h = reinterpret_cast<const BuildHeader*>(ws);
  const uint64_t* keys = reinterpret_cast<const uint64_t*>(ws + w.keys_a);
  uint32_t* leaf_of_voxel = reinterpret_cast<uint32_t*>(ws + w.leaf_of_voxel);
  uint64_t* leaf_key = reinterpret_cast<uint64_t*>(ws + w.leaf_key);
  uint32_t* leaf_first = reinterpret_cast<uint32_t*>(ws + w.leaf_first);
  uint32_t* lower_id = reinterpret_cast<uint32_t*>(ws + w.lower_id);
  uint32_t* root_rank = reinterpret_cast<uint32_t*>(ws + w.root_rank);
  const uint64_t N = grid->n_active, L = grid->n_leaves;
  const uint64_t pieces = grid->blob_bytes / 16;
  hipLaunchKernelGGL(k_fill_init, dim3(grid_for(pieces)), dim3(256), 0, st, reinterpret_cast<uint4*>(blob), pieces,
                     grid->off_upper / 16, (grid->off_upper + uint64_t(grid->n_upper) * 32768 * 4) / 16,
                     grid->off_lower / 16, (grid->off_lower + uint64_t(grid->n_lower) * 4096 * 4) / 16);
  if (N > 0) {
    // inclusive scans of start flags: leaf of each voxel, lower node and root rank of each leaf
    uint32_t* tiles = reinterpret_cast<uint32_t*>(ws + w.temp);
    flag_scan(group_start(keys, 9), N, tiles, nullptr, WriteCount{leaf_of_voxel}, st);
    hipLaunchKernelGGL(k_fill_leaf_starts, dim3(grid_for(N)), dim3(256), 0, st, keys, N, L, leaf_of_voxel, leaf_key,
                       leaf_first);
    flag_scan(group_start(leaf_key, 12), L, tiles, nullptr, WriteCount{lower_id}, st);
    flag_scan(group_start(leaf_key, 27), L, tiles, nullptr, WriteCount{root_rank}, st);
    BlobLeaf* leaves = reinterpret_cast<BlobLeaf*>(blob + grid->off_leaves);
    BlobSections sec{leaves, reinterpret_cast<int32_t*>(blob + grid->off_root),
                     reinterpret_cast<uint32_t*>(blob + grid->off_upper),
                     reinterpret_cast<uint32_t*>(blob + grid->off_lower), grid->n_root, grid->n_lower};
    hipLaunchKernelGGL(k_fill_leaves, dim3(grid_for(L)), dim3(256), 0, st, L, N, keys, leaf_key, leaf_first,
                       lower_id, root_rank, h, sec);
    hipLaunchKernelGGL(k_fill_blocks, dim3(grid_for(L)), dim3(256), 0, st, L, N, grid->log2_width, leaf_first,
                       reinterpret_cast<uint32_t*>(blob + grid->off_block_first_leaf),
                       reinterpret_cast<uint64_t*>(blob + grid->off_block_jump));
  }
  return vbm_host::launch_status();
}

extern "C" int vbm_build_device_static(const int32_t* d_ijk, int64_t n, int log2_width, void* d_blob,
                                       uint64_t blob_capacity, vbm_grid* grid, void* stream) {
  if (!grid || n < 0 || (n > 0 && !d_ijk)) return VBM_ERR_ARG;
  if (log2_width < 6 || log2_width > 9) return VBM_ERR_ARG;
  if (uint64_t(n) > kStaticMaxCoords) return VBM_ERR_SIZE;
  void* ws = nullptr;
  int rc = static_scratch(&ws);
  if (rc) return rc;
  uint64_t temp = 0;
  if (temp_storage_bytes(uint64_t(n), static_cast<hipStream_t>(stream), &temp) != hipSuccess) {
    (void)hipGetLastError();
    return VBM_ERR_HIP;
  }
  if (workspace_layout(uint64_t(n), temp).total > kStaticScratchBytes) return VBM_ERR_SIZE;
  if ((rc = vbm_build_device_plan(d_ijk, n, log2_width, ws, kStaticScratchBytes, grid, stream))) return rc;
  if (!d_blob || blob_capacity < grid->blob_bytes) return VBM_ERR_SIZE;  // grid tells the size needed
  return vbm_build_device_fill(grid, n, ws, kStaticScratchBytes, d_blob, stream);
}

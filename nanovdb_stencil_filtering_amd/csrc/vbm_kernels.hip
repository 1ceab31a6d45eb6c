// gfx950 kernels of the VBM stencil pipeline and the C-ABI entry points that
// launch them.
//
// One workgroup per VBM block, one work-item per slot (W = 64..512 work-items,
// 1..8 wave64s).  Each work-item decodes its own slot in registers, resolves
// its taps (tree walk, or the LDS neighbour table staged by the whole
// workgroup), and accumulates C fp32 sidecar channels in tap order.
//
// fp32 semantics: every accumulation is a separate IEEE add (no contraction,
// denormals kept), in tap order from +0.  An inactive tap reads a row of
// zeros instead of branching: the accumulator starts at +0 and a sum of
// nonzero terms that cancels exactly is +0 under round-to-nearest, so it is
// never -0, and adding +0 to anything other than -0 returns it unchanged.
// Skipping the tap (openvdb PR #2262, "What changed": `if (index)`) and
// adding +0 therefore give identical bits.
#pragma clang fp contract(off)

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <initializer_list>
#include <type_traits>

#include "vbm.h"
#include "vbm_device.hpp"
#include "vbm_division.hpp"
#include "vbm_host_checks.hpp"

using namespace vbm;

namespace {

// ---------------------------------------------------------------------------
// sidecar access
// ---------------------------------------------------------------------------
// A kernel reaches sidecar rows through one of two access types, both handing
// out a 32-bit handle per row:
//   Sidecar      (sidecars below 4 GiB) a bounds-checked buffer resource; the
//                handle is the row's byte offset.  Raw buffer loads whose offset
//                is at or beyond num_records return zeros, so an inactive tap
//                carries the offset kInactive and adds +0 without a branch or
//                a pointer select.  Rows must end below kInactive bytes.
//   WideSidecar  (any size) 64-bit addresses; the handle is the row's index,
//                and an inactive tap's handle kNoRow loads nothing and reads
//                zeros.  Buffer resources cannot replace it: their offsets are
//                32-bit, and so is the address of an indexed (strided) load.
// tap(idx): handle of a tap (index 0 = inactive, reads zeros); row(idx): handle
// of row idx itself (row 0 included); load4 / load1: 16 / 4 bytes at byte
// offset in_row of a row.
constexpr uint32_t kInactive = 0xFFFFFF00u;
constexpr uint32_t kBufferFlags = 0x00020000u;  // gfx9 buffer resource word 3

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef const f32x4 __attribute__((address_space(1))) global_f32x4;
typedef const float __attribute__((address_space(1))) global_f32;

struct Sidecar {
  static constexpr bool kWide = false;
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t row_bytes;  // C * 4
  static __device__ __forceinline__ Sidecar make(const float* sc, uint32_t bytes, uint32_t C, uint32_t ch0) {
    Sidecar s;
    s.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(sc + ch0), short(0), int(bytes - 4 * ch0),
                                               int(kBufferFlags));
    s.row_bytes = 4 * C;
    return s;
  }
  __device__ __forceinline__ uint32_t tap(uint32_t idx) const { return idx ? idx * row_bytes : kInactive; }
  __device__ __forceinline__ uint32_t row(uint32_t idx) const { return idx * row_bytes; }
  __device__ __forceinline__ uint32_t inactive() const { return kInactive; }
  __device__ __forceinline__ uint32_t brick_scale() const { return row_bytes; }  // brick cells hold handles
  __device__ __forceinline__ f32x4 load4(uint32_t h, uint32_t in_row) const {
    // whole-vector bit cast: indexing the u32 vector element by element made
    // clang emit a single dword load for all four channels
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, h + in_row, 0, 0));
  }
  __device__ __forceinline__ float load1(uint32_t h, uint32_t in_row) const {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsrc, h + in_row, 0, 0));
  }
};

struct WideSidecar {
  static constexpr bool kWide = true;
  static constexpr uint32_t kNoRow = 0xFFFFFFFFu;  // never an index (N < 2^32 - 1)
  const char* base;    // channel ch0 of row 0
  uint32_t row_bytes;  // C * 4
  static __device__ __forceinline__ WideSidecar make(const float* sc, uint32_t, uint32_t C, uint32_t ch0) {
    return WideSidecar{reinterpret_cast<const char*>(sc + ch0), 4 * C};
  }
  __device__ __forceinline__ uint32_t tap(uint32_t idx) const { return idx ? idx : kNoRow; }
  __device__ __forceinline__ uint32_t row(uint32_t idx) const { return idx; }
  __device__ __forceinline__ uint32_t inactive() const { return kNoRow; }
  __device__ __forceinline__ uint32_t brick_scale() const { return 1u; }
  __device__ __forceinline__ const char* at(uint32_t h, uint32_t in_row) const {
    return base + (uint64_t(h) * row_bytes + in_row);
  }
  __device__ __forceinline__ f32x4 load4(uint32_t h, uint32_t in_row) const {
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (h != kNoRow) v = *(const global_f32x4*)(at(h, in_row));  // a global-memory load
    return v;
  }
  __device__ __forceinline__ float load1(uint32_t h, uint32_t in_row) const {
    float v = 0.0f;
    if (h != kNoRow) v = *(const global_f32*)(at(h, in_row));
    return v;
  }
};

// acc[c] += row[c] for the CH channels of handle h (an inactive tap: zeros),
// from byte in_row of the row on.
template <int CH, bool VEC, class SC>
__device__ __forceinline__ void add_row(float (&acc)[CH], const SC& s, uint32_t h, uint32_t in_row = 0) {
  if constexpr (VEC && CH % 4 == 0) {
#pragma unroll
    for (int q = 0; q < CH / 4; ++q) {
      const f32x4 v = s.load4(h, in_row + 16 * q);
      acc[4 * q + 0] = acc[4 * q + 0] + v.x;
      acc[4 * q + 1] = acc[4 * q + 1] + v.y;
      acc[4 * q + 2] = acc[4 * q + 2] + v.z;
      acc[4 * q + 3] = acc[4 * q + 3] + v.w;
    }
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = acc[c] + s.load1(h, in_row + 4 * c);
  }
}

// The CH channels of handle h, loaded into registers (no use yet).
template <int CH, bool VEC>
struct Row {
  static constexpr int kVec = (VEC && CH % 4 == 0) ? CH / 4 : 0;
  f32x4 v[kVec ? kVec : 1];
  float f[kVec ? 1 : CH];
  template <class SC>
  __device__ __forceinline__ void load(const SC& s, uint32_t h, uint32_t in_row = 0) {
    if constexpr (kVec) {
#pragma unroll
      for (int q = 0; q < kVec; ++q) v[q] = s.load4(h, in_row + 16 * q);
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c) f[c] = s.load1(h, in_row + 4 * c);
    }
  }
  __device__ __forceinline__ void add_to(float (&acc)[CH]) const {
    if constexpr (kVec) {
#pragma unroll
      for (int q = 0; q < kVec; ++q) {
        acc[4 * q + 0] = acc[4 * q + 0] + v[q].x;
        acc[4 * q + 1] = acc[4 * q + 1] + v[q].y;
        acc[4 * q + 2] = acc[4 * q + 2] + v[q].z;
        acc[4 * q + 3] = acc[4 * q + 3] + v[q].w;
      }
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c) acc[c] = acc[c] + f[c];
    }
  }
};

// Gather-accumulate of NT taps (default: the 27 box taps) in tap order, software pipelined:
// the rows of taps t+1..t+D are in flight while tap t is added, and the
// scheduler is fenced between steps so it cannot hoist all 27 rows at once
// (which costs more registers than a wave can hold).  off(t) gives the handle
// of tap t (s.tap(index): an inactive tap reads zeros); the channels are read
// from byte in_row of each row on.
template <int CH, bool VEC, int D, int NT = kBoxTaps, class SC, class Off>
__device__ __forceinline__ void gather_box_pipelined(float (&acc)[CH], const SC& s, Off&& off, uint32_t in_row = 0) {
  Row<CH, VEC> buf[D];
#pragma unroll
  for (int t = 0; t < D; ++t) buf[t].load(s, off(t), in_row);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    __builtin_amdgcn_sched_barrier(0);
    buf[t % D].add_to(acc);
    // Keep tap t's adds here: without this the compiler sinks every add below
    // the tree walks of later taps and keeps all the rows live.  Emits nothing.
#pragma unroll
    for (int c = 0; c < CH; ++c) asm volatile("" : "+v"(acc[c]));
    if (t + D < NT) buf[t % D].load(s, off(t + D), in_row);
  }
}

template <int CH, bool VEC>
__device__ __forceinline__ void store_row(float* __restrict__ p, const float (&acc)[CH]) {
  if constexpr (VEC && CH % 4 == 0) {
#pragma unroll
    for (int q = 0; q < CH / 4; ++q)
      reinterpret_cast<float4*>(p)[q] = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) p[c] = acc[c];
  }
}

// The taps of one slot shared by its LANES work-items of a split kernel (LANES
// adjacent lanes of one quad, 2 or 4; task = LANES slot + q with 64-lane waves
// of consecutive tasks): lane q resolves taps q, q + LANES, ... once, and tap t
// is read from lane t % LANES of the slot by a quad-permute DPP move, instead
// of every lane resolving every tap.  Every lane a move reads must be active:
// callers keep a slot's lanes active or idle together.
template <int LANES, class S>
struct SlotTaps {
  static_assert(LANES == 2 || LANES == 4, "taps are shared within pairs or quads");
  static constexpr int kPer = (S::kTaps + LANES - 1) / LANES;
  uint32_t mine[kPer];
  // res(t, di, dj, dk): index of tap t (< S::kTaps) at offset (di, dj, dk)
  template <class Resolve>
  __device__ __forceinline__ void resolve(uint32_t q, Resolve&& res) {
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      auto pick = [&](auto f) {  // the offset of tap LANES r + q, chosen among LANES constants
        const int a = f(LANES * r), b = f(LANES * r + 1);
        if constexpr (LANES == 2) {
          return q == 0 ? a : b;
        } else {
          const int c = f(LANES * r + 2), d = f(LANES * r + 3);
          return q == 0 ? a : q == 1 ? b : q == 2 ? c : d;
        }
      };
      const int di = pick([](int t) { return t < S::kTaps ? S::di(t) : 0; });
      const int dj = pick([](int t) { return t < S::kTaps ? S::dj(t) : 0; });
      const int dk = pick([](int t) { return t < S::kTaps ? S::dk(t) : 0; });
      const int t = LANES * r + int(q);
      mine[r] = t < S::kTaps ? res(t, di, dj, dk) : 0u;
    }
  }
  // tap t (a constant once the caller's loop is unrolled)
  __device__ __forceinline__ uint32_t operator()(int t) const {
    const int v = int(mine[t / LANES]);
    if constexpr (LANES == 2) {  // lane t % 2 of each pair: quad_perm [0,0,2,2] or [1,1,3,3]
      if (t % 2 == 0) return uint32_t(__builtin_amdgcn_mov_dpp(v, 0xA0, 0xF, 0xF, false));
      return uint32_t(__builtin_amdgcn_mov_dpp(v, 0xF5, 0xF, 0xF, false));
    } else {
      switch (t % 4) {  // lane t % 4 of the quad
        case 0: return uint32_t(__builtin_amdgcn_mov_dpp(v, 0x00, 0xF, 0xF, false));
        case 1: return uint32_t(__builtin_amdgcn_mov_dpp(v, 0x55, 0xF, 0xF, false));
        case 2: return uint32_t(__builtin_amdgcn_mov_dpp(v, 0xAA, 0xF, 0xF, false));
        default: return uint32_t(__builtin_amdgcn_mov_dpp(v, 0xFF, 0xF, 0xF, false));
      }
    }
  }
};

template <int CH>
__device__ __forceinline__ void zero_index_row(float* __restrict__ out, uint32_t ch0) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) out[ch0 + c] = 0.0f;
  }
}

// Prefetch of block bn's rows (indices 1 + bn*W .. (bn+1)*W, one contiguous byte
// range of the sidecar) into the L2, so that a later block finds them there: one
// dword of each 128-byte line of the range (the L2 fetches whole lines), line
// threadIdx.x + k * blockDim.x in v[k], so the first N * blockDim.x lines.  A
// dword per line takes a small fraction of the address cycles that loading the
// rows themselves took, and leaves the L1 to the gather.  The caller consumes v
// only at its very end (consume_touch), so no wave waits for these loads.
// bn = 0xFFFFFFFF (or a block past the grid) loads nothing.
template <int N, class SC>
__device__ __forceinline__ void touch_block_lines(const DeviceGrid& g, const SC& side, uint32_t bn, float (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) v[k] = 0.0f;
  if constexpr (!SC::kWide) {  // the wide path does not prefetch
    const bool has = bn < g.n_blocks;
    const uint64_t row0 = 1 + (uint64_t(has ? bn : 0u) << g.log2w);
    const uint64_t rows = has ? min(uint64_t(1) << g.log2w, uint64_t(g.n_active) + 1 - row0) : 0;
    const uint64_t begin = row0 * side.row_bytes & ~uint64_t(127);  // the line holding the first row
    const uint64_t end = (row0 + rows) * side.row_bytes;
    const uint32_t lines = rows ? uint32_t((end - begin + 127) / 128) : 0u;
#pragma unroll
    for (int k = 0; k < N; ++k) {
      if (k == 0 || k * blockDim.x < lines) {  // workgroup-uniform
        const uint32_t line = threadIdx.x + k * blockDim.x;
        v[k] = side.load1(line < lines ? uint32_t(begin + uint64_t(line) * 128) : kInactive, 0);
      }
    }
  }
}
template <int N>
__device__ __forceinline__ void consume_touch(const float (&v)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) asm volatile("" :: "v"(v[k]));
}

// Tunables of the brick-cached box kernel (defaults measured on MI355X).
#ifndef VBM_PIPE_WIDE
#define VBM_PIPE_WIDE 2   // taps in flight per work-item for CH >= 8
#endif
#ifndef VBM_PIPE_NARROW
// taps in flight per work-item for CH < 8: 6 is 1-3 % faster than 4 on the
// one- to four-channel box, cross, Laplacian and axis kernels (8: about the
// same as 6, slower at 3 channels W512)
#define VBM_PIPE_NARROW 6
#endif
#ifndef VBM_XCD_REMAP
#define VBM_XCD_REMAP 1    // 1: give each of the 8 XCDs a contiguous range of blocks
#endif
#ifndef VBM_NT_STORE
#define VBM_NT_STORE 1  // 1: output rows written with non-temporal stores
#endif
#ifndef VBM_SPLIT_MAX
#define VBM_SPLIT_MAX 256  // work-items per workgroup of the split-row kernel (at least W)
#endif
#ifndef VBM_PIPE_SPLIT
#define VBM_PIPE_SPLIT 8   // taps in flight per work-item in the split-row kernel
#endif
#ifndef VBM_DECODE_THREADS
#define VBM_DECODE_THREADS 512  // work-items per workgroup of k_decode (W or more)
#endif
#ifndef VBM_STENCIL_SPLIT
#define VBM_STENCIL_SPLIT 1  // 1: cross / Laplacian / axis filters split 16-channel rows over 4 work-items
#endif
#ifndef VBM_PREFETCH_AHEAD
#define VBM_PREFETCH_AHEAD 64  // split box, split cross, 8-channel stencils: blocks ahead (per XCD) whose rows each workgroup prefetches; 0 = off
#endif
#ifndef VBM_PLAIN_SPLIT
#define VBM_PLAIN_SPLIT 1  // 16-channel tree-walk box: rows split over quads, taps walked once per slot
#endif
#ifndef VBM_STAGE_LEAVES
#define VBM_STAGE_LEAVES 1  // 1: the split-row kernel stages neighbour leaf records in LDS for the brick build
#endif

// Checking build (VBM_POISON_LDS=1, a separate library used by the tests only):
// before every brick pass all cells of the bricks are overwritten with a
// poison value, so a voxel that reads a plane the pass did not build (the
// build resolves only the x planes the block reaches), or a cell left from an
// earlier pass or an earlier workgroup, gives a wrong tap or a wrong sum --
// a deterministic mismatch against the oracle, never an access outside a
// buffer (raw taps copy the value out; filter offsets go through the
// bounds-checked sidecar loads).  The x ranges, tables, staged records and
// slot corners are written in full before their barrier and are not poisoned.
#ifndef VBM_POISON_LDS
#define VBM_POISON_LDS 0
#endif

__device__ __forceinline__ void poison_bricks(uint32_t* brick, uint32_t count, uint32_t value) {
#if VBM_POISON_LDS
  for (uint32_t c = threadIdx.x; c < count * kBrickCells; c += blockDim.x) brick[c] = value;
  __syncthreads();
#else
  (void)brick; (void)count; (void)value;
#endif
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  With VBM_XCD_REMAP the workgroup id is mapped so that XCD k works on
// the contiguous block range [k * per, (k + 1) * per): neighbouring blocks
// share halo rows through one L2.  Returns n_blocks or more for padding
// workgroups (they exit).
__device__ __forceinline__ uint32_t block_of_workgroup(uint32_t wg, uint32_t n_blocks) {
#if VBM_XCD_REMAP
  const uint32_t per = (n_blocks + 7) / 8;
  return (wg % 8) * per + wg / 8;
#else
  (void)n_blocks;
  return wg;
#endif
}

__host__ __device__ constexpr uint32_t box_grid_size(uint32_t n_blocks) {
#if VBM_XCD_REMAP
  return ((n_blocks + 7) / 8) * 8;
#else
  return n_blocks;
#endif
}

// Dynamic LDS of the brick-cached kernels: the neighbour table of up to `cap`
// spanned leaves, then their bricks.
__host__ __device__ constexpr uint32_t brick_lds_bytes(uint32_t cap) { return cap * 27 * 4 + cap * kBrickCells * 4; }

// Dynamic LDS of the split-row kernel: staged leaf records (or the neighbour
// table), the per-slot brick corners and the bricks.
__host__ __device__ constexpr uint32_t split_lds_bytes(uint32_t cap, uint32_t W) {
  return VBM_STAGE_LEAVES ? cap * 27 * uint32_t(sizeof(StagedLeaf)) + W * 4 + cap * kBrickCells * 4
                          : brick_lds_bytes(cap) + W * 4;
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

// A workgroup of blockDim.x >= W work-items decodes blockDim.x / W consecutive
// blocks (fewer, larger workgroups: the kernel is short and dispatch-bound).
__global__ void __launch_bounds__(512) k_decode(DeviceGrid g, uint32_t* __restrict__ leaf_index,
                                                uint16_t* __restrict__ voxel_offset) {
  const uint32_t b = blockIdx.x * (blockDim.x >> g.log2w) + (threadIdx.x >> g.log2w);
  if (b >= g.n_blocks) return;  // whole waves (W >= 64)
  const uint32_t slot = threadIdx.x & ((1u << g.log2w) - 1);
  const Slot s = decode_own_slot(g, b, slot);
  const uint64_t row = (uint64_t(b) << g.log2w) + slot;
  leaf_index[row] = s.leaf;
  voxel_offset[row] = uint16_t(s.offset);
}

// Inverse maps by the sweep that the select-based decode replaced
// (openvdb PR #2258, "Summary"): the workgroup of block b walks every voxel
// position of every leaf the block spans, O(span x 512) per block; a set bit
// whose index falls inside the block writes its slot.  Slots past the last
// active index receive the sentinels.  Same maps as k_decode.
__global__ void __launch_bounds__(512) k_decode_sweep(DeviceGrid g, uint32_t* __restrict__ leaf_index,
                                                      uint16_t* __restrict__ voxel_offset) {
  const uint32_t b = blockIdx.x;
  const uint32_t W = 1u << g.log2w;
  const uint64_t g0 = 1 + (uint64_t(b) << g.log2w);
  uint32_t* li = leaf_index + (uint64_t(b) << g.log2w);
  uint16_t* vo = voxel_offset + (uint64_t(b) << g.log2w);
  if (g0 + threadIdx.x > g.n_active) {
    li[threadIdx.x] = kSentinelLeaf;
    vo[threadIdx.x] = uint16_t(kSentinelOffset);
  }
  const uint32_t first = g.block_first_leaf[b];
  const uint32_t span = block_span(g, b);
  for (uint32_t j = 0; j < span; ++j) {
    const Leaf& L = g.leaves[first + j];
    for (uint32_t o = threadIdx.x; o < 512; o += blockDim.x) {
      const uint32_t idx = index_in_leaf(L, o);  // 0 if the position is inactive
      const uint64_t slot = uint64_t(idx) - g0;
      if (idx != 0 && slot < W) {
        li[slot] = first + j;
        vo[slot] = uint16_t(o);
      }
    }
  }
}

// Raw box taps through the brick cache (materialised or streamed), block by
// block in passes of at most `cap` spanned leaves; blocks spanning more than
// kMaxCachedLeaves walk the tree per tap.
template <bool STREAM>
__global__ void __launch_bounds__(512) k_taps_box_cached(DeviceGrid g, uint64_t* __restrict__ taps, uint32_t cap) {
  extern __shared__ uint32_t lds[];
  __shared__ uint32_t xr[2 * kMaxCachedLeaves];
  uint32_t* table = lds;
  uint32_t* brick = lds + cap * 27;
  const uint32_t b = blockIdx.x;
  const Slot s = decode_own_slot(g, b);
  const bool valid = s.leaf != kSentinelLeaf;
  uint64_t* out = taps + ((uint64_t(b) << g.log2w) + threadIdx.x) * kBoxTaps;
  const uint32_t first = g.block_first_leaf[b];
  const uint32_t span = block_span(g, b);  // block-uniform: every barrier below is uniform
  if (span > kMaxCachedLeaves) {
    if (valid) for_each_box(g, s, [&](int t, uint32_t idx) { out[t] = idx; });
  } else {
    record_leaf_xrange(g, b, s, first, xr);
    const uint32_t j = valid ? s.leaf - first : 0xFFFFFFFFu;
    for (uint32_t j0 = 0; j0 < span; j0 += cap) {
      const uint32_t count = min(cap, span - j0);
      if (j0) __syncthreads();
      stage_table_range(g, first + j0, count, table);
      poison_bricks(brick, count, 0xFFFFFFFEu);  // never an index
      build_bricks(g, table, count, xr + j0, 1u, 0u, brick);
      if (j - j0 < count) {
        const uint32_t* corner = brick_corner(brick, j - j0, s.offset);
        if constexpr (STREAM) {
          for_each_box_brick(corner, [&](int t, uint32_t idx) { out[t] = idx; });
        } else {
          uint32_t st[kBoxTaps];
          for_each_box_brick(corner, [&](int t, uint32_t idx) { st[t] = idx; });
#pragma unroll
          for (int t = 0; t < kBoxTaps; ++t) out[t] = st[t];
        }
      }
    }
  }
  if (!valid) {
#pragma unroll
    for (int t = 0; t < kBoxTaps; ++t) out[t] = 0;
  }
}

// Raw taps of any shape by tree walks, or of the 7-direction shapes (cross,
// 19-tap axis) through the per-tap cached table of neighbour leaves; streamed
// straight to the output row or materialised into an array first.
template <class S, bool CACHED, bool STREAM>
__global__ void __launch_bounds__(512) k_taps(DeviceGrid g, uint64_t* __restrict__ taps) {
  __shared__ StagedLeaf staged[CACHED ? kMaxCachedLeaves * S::kDirs : 1];  // neighbour leaf records
  __shared__ RootTile root_lds[CACHED ? 1 : kLdsRootTiles];                // the plain resolver's root table
  const uint32_t b = blockIdx.x;
  const Slot s = decode_own_slot(g, b);
  const bool valid = s.leaf != kSentinelLeaf;
  uint64_t* out = taps + ((uint64_t(b) << g.log2w) + threadIdx.x) * S::kTaps;
  bool cached = false;
  uint32_t first = 0;
  if constexpr (CACHED) {
    first = g.block_first_leaf[b];
    const uint32_t span = block_span(g, b);  // block-uniform: the barrier below is uniform
    if (span <= kMaxCachedLeaves) {
      stage_neighbour_records<S::kDirs>(g, first, span, staged);
      cached = true;
    }
  }
  // the plain resolver's walks search the root table in LDS; the cached one's
  // fallback walks (blocks spanning more than kMaxCachedLeaves) the global table
  const LdsRoot root = CACHED ? LdsRoot{root_lds, false} : stage_root_table(g, root_lds);
  if (!valid) {
#pragma unroll
    for (int j = 0; j < S::kTaps; ++j) out[j] = 0;
    return;
  }
  if constexpr (STREAM) {
    auto put = [&](int t, uint32_t idx) { out[t] = idx; };
    if (cached) for_each_tap_staged<S>(staged, first, s, put);
    else for_each_tap<S>(g, root, s, put);
  } else {
    uint64_t st[S::kTaps];
    auto keep = [&](int t, uint32_t idx) { st[t] = idx; };
    if (cached) for_each_tap_staged<S>(staged, first, s, keep);
    else for_each_tap<S>(g, root, s, keep);
#pragma unroll
    for (int j = 0; j < S::kTaps; ++j) out[j] = st[j];
  }
}

// Value bricks, for a sidecar of one channel (rows 4 bytes apart): the cells
// of build_bricks hold the bits of the voxel's value instead of a row handle,
// and +0.0f for an inactive position, so a voxel's 27 taps are LDS reads with no
// gather left.  The active voxels of a leaf column (z = 0..7) have consecutive
// indices, so their values are one run of at most eight consecutive floats:
// two 16-byte loads from the column's first index (values past the run are not
// used; past the sidecar's end the bounds-checked loads read zeros, dword by
// dword), then each active z takes the next value of the run.  The -z and +z
// neighbours' cells take one load each.  All threads of the block; ends with a
// barrier.
__device__ __forceinline__ void build_value_bricks(const DeviceGrid& g, const uint32_t* table, uint32_t count,
                                                   const uint32_t* xr, const Sidecar& side, uint32_t* brick) {
  uint32_t total = 0;
  for (uint32_t jj = 0; jj < count; ++jj) total += (xr[kMaxCachedLeaves + jj] - xr[jj] + 3) * 10;
  for (uint32_t c = threadIdx.x; c < total; c += blockDim.x) {
    // column c -> (brick jj, plane xp, row yp), as in build_bricks
    uint32_t jj = 0, rem = c, xp0 = xr[0];
    for (;;) {
      const uint32_t n = (xr[kMaxCachedLeaves + jj] - xp0 + 3) * 10;
      if (rem < n) break;
      rem -= n;
      xp0 = xr[++jj];
    }
    const uint32_t xp = xp0 + rem / 10, yp = rem % 10;  // plane xp holds x = xp - 1
    const int x = int(xp) - 1, y = int(yp) - 1;
    const int dxl = x >> 3, dyl = y >> 3;  // -1, 0, +1
    const uint32_t wx = uint32_t(x) & 7, y8 = (uint32_t(y) & 7) << 3;
    const uint32_t* trow = table + jj * 27 + (dxl + 1) * 9 + (dyl + 1) * 3;
    const ColumnBits zm = column_bits(g, trow[0], wx, y8);  // -z neighbour, its z = 7
    const ColumnBits zc = column_bits(g, trow[1], wx, y8);  // the leaf column, z = 0..7
    const ColumnBits zp = column_bits(g, trow[2], wx, y8);  // +z neighbour, its z = 0
    const float vm = side.load1(side.tap(((zm.bits >> 7) & 1u) ? zm.base + __popc(zm.bits & 0x7Fu) : 0u), 0u);
    const float vp = side.load1(side.tap((zp.bits & 1u) ? zp.base : 0u), 0u);
    const uint32_t h = side.tap(zc.bits ? zc.base : 0u);  // an empty column loads nothing
    const f32x4 r0 = side.load4(h, 0u), r1 = side.load4(h, 16u);
    float run[8] = {r0.x, r0.y, r0.z, r0.w, r1.x, r1.y, r1.z, r1.w};
    uint32_t* out = brick + jj * kBrickCells + xp * 100 + yp * 10;
    out[0] = __float_as_uint(vm);
#pragma unroll
    for (uint32_t z = 0; z < 8; ++z) {
      const bool on = (zc.bits >> z) & 1u;
      out[1 + z] = on ? __float_as_uint(run[0]) : 0u;
      if (z < 7) {
#pragma unroll
        for (uint32_t i = 0; i + 1 < 8 - z; ++i) run[i] = on ? run[i + 1] : run[i];  // drop the value taken
      }
    }
    out[9] = __float_as_uint(vp);
  }
  __syncthreads();
}

// 27-tap box filter, tree-walk resolution, over channels [ch0, ch0 + CH).
template <int CH, bool VEC, bool STREAM, class SC = Sidecar>
__global__ void __launch_bounds__(512) k_box_plain(DeviceGrid g, const float* __restrict__ sc, uint32_t sc_bytes,
                                                   float* __restrict__ out, uint32_t C, uint32_t ch0) {
  // taps in flight per work-item; the materialised form holds all 27 taps as
  // well, and at 3-4 channels six in flight would take it past 64 VGPRs (8 waves
  // per SIMD): measured 2-7 % slower than four, so it keeps four
  constexpr int kPipe = CH >= 8 ? VBM_PIPE_WIDE : (STREAM || CH < 3 ? VBM_PIPE_NARROW : 4);
  __shared__ RootTile root_lds[kLdsRootTiles];
  const uint32_t b = blockIdx.x;
  zero_index_row<CH>(out, ch0);
  const LdsRoot root = stage_root_table(g, root_lds);
  const Slot s = decode_own_slot(g, b);
  if (s.leaf == kSentinelLeaf) return;
  const SC side = SC::make(sc, sc_bytes, C, ch0);
  float acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = 0.0f;
  if constexpr (STREAM) {
    // taps streamed to the gather in three groups of nine (one x offset of the
    // stencil each): the nine tree walks of a group are independent chains of
    // dependent loads that overlap one another, and the group's offsets are
    // consumed in tap order; at most nine are held, never the whole stencil
    const VoxelCoord p = voxel_coord(g, s);
#pragma unroll
    for (int grp = 0; grp < 3; ++grp) {
      uint32_t off[9];
#pragma unroll
      for (int k = 0; k < 9; ++k) {
        const int t = 9 * grp + k;
        off[k] = side.tap(resolve_tree(g, root, p.x + box_di(t), p.y + box_dj(t), p.z + box_dk(t)));
      }
      gather_box_pipelined<CH, VEC, kPipe, 9>(acc, side, [&](int k) { return off[k]; });
    }
  } else {
    uint64_t st[kBoxTaps];
    compute_box(g, root, s, st);
    gather_box_pipelined<CH, VEC, kPipe>(acc, side, [&](int t) { return side.tap(uint32_t(st[t])); });
  }
  const uint64_t idx = 1 + (uint64_t(b) << g.log2w) + threadIdx.x;
  store_row<CH, VEC>(out + idx * C + ch0, acc);
}

// 27-tap box filter through the brick cache (materialised or streamed taps).
// VALUES (one-channel sidecars only): value bricks, so the taps are LDS reads.
template <int CH, bool VEC, bool STREAM, class SC = Sidecar, bool VALUES = false>
__global__ void __launch_bounds__(512) k_box_cached(DeviceGrid g, const float* __restrict__ sc, uint32_t sc_bytes,
                                                    float* __restrict__ out, uint32_t C, uint32_t ch0, uint32_t cap) {
  static_assert(!VALUES || (CH == 1 && !SC::kWide), "value bricks: one channel through the buffer resource");
  constexpr int kPipe = CH >= 8 ? VBM_PIPE_WIDE : VBM_PIPE_NARROW;  // taps in flight per work-item
  extern __shared__ uint32_t lds[];
  __shared__ uint32_t xr[2 * kMaxCachedLeaves];
  uint32_t* table = lds;
  uint32_t* brick = lds + cap * 27;
  const uint32_t b = block_of_workgroup(blockIdx.x, g.n_blocks);
  if (b >= g.n_blocks) return;  // padding workgroup
  zero_index_row<CH>(out, ch0);
  const Slot s = decode_own_slot(g, b);
  const bool valid = s.leaf != kSentinelLeaf;
  const SC side = SC::make(sc, sc_bytes, C, ch0);
  float acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = 0.0f;
  const uint32_t first = g.block_first_leaf[b];
  const uint32_t span = block_span(g, b);  // block-uniform: every barrier below is uniform
  if (span > kMaxCachedLeaves) {
    if (valid) {  // per-tap tree walk
      const VoxelCoord p = voxel_coord(g, s);
      gather_box_pipelined<CH, VEC, kPipe>(acc, side, [&](int t) {
        return side.tap(resolve_tree(g, p.x + box_di(t), p.y + box_dj(t), p.z + box_dk(t)));
      });
    }
  } else {
    record_leaf_xrange(g, b, s, first, xr);
    const uint32_t j = valid ? s.leaf - first : 0xFFFFFFFFu;
    for (uint32_t j0 = 0; j0 < span; j0 += cap) {
      const uint32_t count = min(cap, span - j0);
      if (j0) __syncthreads();
      stage_table_range(g, first + j0, count, table);
      if constexpr (VALUES) {
        poison_bricks(brick, count, 0x3F800000u);  // 1.0f: a wrong value
        build_value_bricks(g, table, count, xr + j0, side, brick);
      } else {
        poison_bricks(brick, count, side.row(1));  // handle of row 1: a wrong, in-bounds row
        build_bricks(g, table, count, xr + j0, side.brick_scale(), side.inactive(), brick);
      }
      if (j - j0 < count) {
        const uint32_t* corner = brick_corner(brick, j - j0, s.offset);
        if constexpr (VALUES) {
          // the values themselves, added in tap order (streamed as read, or
          // read into an array first)
          if constexpr (STREAM) {
#pragma unroll
            for (int t = 0; t < kBoxTaps; ++t) acc[0] = acc[0] + __uint_as_float(corner[box_brick_offset(t)]);
          } else {
            float v[kBoxTaps];
#pragma unroll
            for (int t = 0; t < kBoxTaps; ++t) v[t] = __uint_as_float(corner[box_brick_offset(t)]);
#pragma unroll
            for (int t = 0; t < kBoxTaps; ++t) acc[0] = acc[0] + v[t];
          }
        } else if constexpr (STREAM) {
          // taps streamed from the brick as the pipeline consumes them
          gather_box_pipelined<CH, VEC, kPipe>(acc, side, [&](int t) { return corner[box_brick_offset(t)]; });
        } else {
          uint32_t st[kBoxTaps];
          for_each_box_brick(corner, [&](int t, uint32_t off) { st[t] = off; });
          gather_box_pipelined<CH, VEC, kPipe>(acc, side, [&](int t) { return st[t]; });
        }
      }
    }
  }
  if (!valid) return;
  const uint64_t idx = 1 + (uint64_t(b) << g.log2w) + threadIdx.x;
  store_row<CH, VEC>(out + idx * C + ch0, acc);
}

// 27-tap box filter through the brick cache with each sidecar row split over
// LANES = CH / 4 work-items (one float4 of channels each): a wave gathers
// 64 / LANES whole rows per load instead of one 16-byte piece of 64 rows, and
// writes whole output rows.  Slots are decoded once into LDS; the workgroup
// has min(W * LANES, max(W, VBM_SPLIT_MAX)) work-items, each handling one or
// more (slot, quarter) tasks.  STREAM: taps are streamed from the brick in tap
// order; else the 27 taps are materialised into an array first.
template <int CH, bool STREAM, class SC = Sidecar>
__global__ void __launch_bounds__(1024) k_box_cached_split(DeviceGrid g, const float* __restrict__ sc,
                                                           uint32_t sc_bytes, float* __restrict__ out, uint32_t C,
                                                           uint32_t ch0, uint32_t cap) {
  static_assert(CH % 4 == 0 && CH >= 8, "split rows need whole float4 groups");
  constexpr uint32_t LANES = CH / 4;
  constexpr int kPipe = VBM_PIPE_SPLIT;
  extern __shared__ uint4 lds4[];
  __shared__ uint32_t xr[2 * kMaxCachedLeaves];
  const uint32_t W = 1u << g.log2w;
#if VBM_STAGE_LEAVES
  StagedLeaf* staged = reinterpret_cast<StagedLeaf*>(lds4);  // leaf records of the neighbour table
  uint32_t* slot_corner = reinterpret_cast<uint32_t*>(staged + cap * 27);
  uint32_t* brick = slot_corner + W;
#else
  uint32_t* slot_corner = reinterpret_cast<uint32_t*>(lds4);  // per slot: brick corner | leaf-in-block << 16
  uint32_t* table = slot_corner + W;
  uint32_t* brick = table + cap * 27;
#endif
  const uint32_t b = block_of_workgroup(blockIdx.x, g.n_blocks);
  if (b >= g.n_blocks) return;  // padding workgroup
  if (blockIdx.x == 0 && threadIdx.x < CH) out[ch0 + threadIdx.x] = 0.0f;
  const SC side = SC::make(sc, sc_bytes, C, ch0);
  const uint32_t first = g.block_first_leaf[b];
  const uint32_t span = block_span(g, b);  // block-uniform: every barrier below is uniform
  const uint32_t tasks = W * LANES;
  // one (slot, quarter) task: gather its 27 taps through off(t) and store
  auto run = [&](uint32_t task, auto&& off) {
    const uint32_t slot = task / LANES, q = task % LANES;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // bytes 16 q .. 16 q + 15 of each tap's row; an inactive tap's buffer offset
    // kInactive + 16 q (at most 0xFFFFFF30) is still at or beyond the buffer's
    // size (checked on the host), so it reads zeros too
    gather_box_pipelined<4, true, kPipe>(acc, side, off, 16 * q);
    const uint64_t idx = 1 + (uint64_t(b) << g.log2w) + slot;
#if VBM_NT_STORE
    f32x4* dst = reinterpret_cast<f32x4*>(out + idx * C + ch0) + q;
    __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]}, dst);
#else
    reinterpret_cast<float4*>(out + idx * C + ch0)[q] = make_float4(acc[0], acc[1], acc[2], acc[3]);
#endif
  };
  // Phase 1: the waves holding slots decode them (lane-rank decode; a slot
  // past the last index is marked 0xFFFFFFFF) while the other waves stage the
  // neighbour table of the first pass, so the two chains of dependent loads
  // overlap.
  const bool cached = span <= kMaxCachedLeaves;
  const uint32_t count0 = cached ? min(cap, span) : 0u;
  if (threadIdx.x < W) {
    const Slot s = decode_own_slot(g, b);
    slot_corner[threadIdx.x] =
        s.leaf == kSentinelLeaf
            ? 0xFFFFFFFFu
            : ((s.leaf - first) << 16) | ((s.offset >> 6) * 100 + ((s.offset >> 3) & 7) * 10 + (s.offset & 7));
    if (cached) record_leaf_xrange(g, b, s, first, xr);
  }
  const uint32_t stagers = blockDim.x > W ? blockDim.x - W : blockDim.x;
  const uint32_t stager = blockDim.x > W ? threadIdx.x - W : threadIdx.x;  // wraps for decoders when blockDim > W
#if VBM_STAGE_LEAVES
  if (blockDim.x == W || threadIdx.x >= W) fill_table_range_staged(g, first, count0, staged, stager, stagers);
#else
  if (blockDim.x == W || threadIdx.x >= W) fill_table_range(g, first, count0, table, stager, stagers);
#endif
  __syncthreads();
  // Prefetch the rows of the block this XCD starts VBM_PREFETCH_AHEAD blocks
  // later (about two per CU), so that block finds them in the L2 instead of HBM;
  // near enough that they are still in the 4 MB L2 when it starts, far enough
  // that the loads have landed.  Issued after the decode and the table: vector
  // loads retire in order, so a prefetch issued earlier would hold up the waits
  // of the decode's own loads behind its trip to HBM.
  float ahead[1];  // one line per work-item: the whole block at up to 32 channels
  {
    const uint32_t per = (g.n_blocks + 7) / 8;
    const uint32_t in_xcd = b - (blockIdx.x % 8) * per;
    const bool has = VBM_PREFETCH_AHEAD > 0 && in_xcd + VBM_PREFETCH_AHEAD < per;
    touch_block_lines(g, side, has ? b + VBM_PREFETCH_AHEAD : 0xFFFFFFFFu, ahead);
  }
  if (!cached) {  // per-tap tree walk
    for (uint32_t task = threadIdx.x; task < tasks; task += blockDim.x) {
      const uint32_t info = slot_corner[task / LANES];
      if (info == 0xFFFFFFFFu) continue;
      const Leaf& L = g.leaves[first + (info >> 16)];
      const uint32_t cell = info & 0xFFFF;
      const int x = L.origin[0] + int(cell / 100), y = L.origin[1] + int((cell / 10) % 10);
      const int z = L.origin[2] + int(cell % 10);
      SlotTaps<LANES, BoxShape> taps;  // each tap walked once per slot, shared by its LANES work-items
      taps.resolve(task % LANES, [&](int, int di, int dj, int dk) { return resolve_tree(g, x + di, y + dj, z + dk); });
      run(task, [&](int t) { return side.tap(taps(t)); });
    }
    return;
  }
  for (uint32_t j0 = 0; j0 < span; j0 += cap) {
    const uint32_t count = min(cap, span - j0);
#if VBM_STAGE_LEAVES
    if (j0) {  // later passes: the whole block restages
      __syncthreads();  // the previous pass is done with the LDS
      fill_table_range_staged(g, first + j0, count, staged, threadIdx.x, blockDim.x);
      __syncthreads();
    }
    poison_bricks(brick, count, side.row(1));
    build_bricks_staged(staged, count, xr + j0, side.brick_scale(), side.inactive(), brick);
#else
    if (j0) {  // later passes: the whole block restages
      __syncthreads();  // the previous pass is done with the LDS
      fill_table_range(g, first + j0, count, table, threadIdx.x, blockDim.x);
      __syncthreads();
    }
    poison_bricks(brick, count, side.row(1));
    build_bricks(g, table, count, xr + j0, side.brick_scale(), side.inactive(), brick);
#endif
    for (uint32_t task = threadIdx.x; task < tasks; task += blockDim.x) {
      const uint32_t info = slot_corner[task / LANES];
      const uint32_t j = info >> 16;
      if (info == 0xFFFFFFFFu || j - j0 >= count) continue;
      const uint32_t* corner = brick + (j - j0) * kBrickCells + (info & 0xFFFF);
      if constexpr (STREAM) {
        run(task, [&](int t) { return corner[box_brick_offset(t)]; });
      } else {  // the 27 taps materialised into an array first
        uint32_t st[kBoxTaps];
#pragma unroll
        for (int t = 0; t < kBoxTaps; ++t) st[t] = corner[box_brick_offset(t)];
        run(task, [&](int t) { return st[t]; });
      }
    }
  }
  consume_touch(ahead);
}

// Filters of the 7-direction shapes: the cross (sum, or 7-point Laplacian =
// faces in cross order - fl(6 c)) and the 19-tap axis stencil (sum).  Taps by
// tree walks or through the per-tap cached table; streamed into the gather
// pipeline (STREAM) or materialised into an array first.  CAPL: spanned
// leaves whose records are staged at a time; below kMaxCachedLeaves a block is
// processed in passes of CAPL leaves (each voxel gathers in the pass holding
// its leaf), so that LDS does not limit how many single-wave workgroups (W64)
// are resident.
template <class S, int CH, bool VEC, bool CACHED, bool LAP, bool STREAM, class SC = Sidecar,
          int CAPL = kMaxCachedLeaves>
__global__ void __launch_bounds__(512) k_stencil(DeviceGrid g, const float* __restrict__ sc, uint32_t sc_bytes,
                                                 float* __restrict__ out, uint32_t C, uint32_t ch0) {
  static_assert(CAPL >= 1 && CAPL <= kMaxCachedLeaves, "records staged per pass");
  constexpr bool kPasses = CAPL < kMaxCachedLeaves;
  // taps in flight per work-item; the streamed form at eight or more channels
  // takes a deeper pipeline than the box's two (measured on the shell, cached
  // streamed C=8: cross 1-2 % faster with three, 19-tap axis 1-7 % with four)
  constexpr int kPipe =
      CH >= 8 ? (STREAM ? (S::kTaps > 7 ? 4 : 3) : VBM_PIPE_WIDE) : VBM_PIPE_NARROW;
  __shared__ StagedLeaf staged[CACHED ? CAPL * S::kDirs : 1];  // neighbour leaf records
  __shared__ RootTile root_lds[CACHED ? 1 : kLdsRootTiles];    // the plain resolver's root table
  const uint32_t b = blockIdx.x;
  zero_index_row<CH>(out, ch0);
  const Slot s = decode_own_slot(g, b);
  const bool valid = s.leaf != kSentinelLeaf;
  bool cached = false;
  uint32_t first = 0, span = 0;
  if constexpr (CACHED) {
    first = g.block_first_leaf[b];
    span = block_span(g, b);  // block-uniform: the barriers below are uniform
    if (span <= kMaxCachedLeaves) {
      if constexpr (!kPasses) stage_neighbour_records<S::kDirs>(g, first, span, staged);
      cached = true;
    }
  }
  // the plain resolver's walks search the root table in LDS; the cached one's
  // fallback walks (blocks spanning more than kMaxCachedLeaves) the global table
  const LdsRoot root = CACHED ? LdsRoot{root_lds, false} : stage_root_table(g, root_lds);
  const SC side = SC::make(sc, sc_bytes, C, ch0);
  // Rows of the block this XCD starts VBM_PREFETCH_AHEAD blocks later (blocks go
  // round-robin over the 8 XCDs here, hence the factor 8).  Measured on MI355X:
  // 3-6 % faster at 8 channels a work-item, 2-3 % slower at 1, so only the wide form.
  constexpr bool kTouch = CH >= 8;
  float ahead[1];  // one line per work-item: the whole block at up to 32 channels
  if constexpr (kTouch)
    touch_block_lines(g, side, VBM_PREFETCH_AHEAD && b + 8 * VBM_PREFETCH_AHEAD < g.n_blocks
                                   ? b + 8 * VBM_PREFETCH_AHEAD : 0xFFFFFFFFu, ahead);
  float acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = 0.0f;
  if constexpr (CACHED && kPasses) {
    // passes of CAPL spanned leaves: the records of leaves j0 .. j0 + count - 1
    // in LDS, then the voxels of those leaves gather (the same taps, the same
    // order as in one pass)
    if (cached) {
      const uint32_t j = valid ? s.leaf - first : 0xFFFFFFFFu;
      const int x = int(s.offset >> 6), y = int((s.offset >> 3) & 7), z = int(s.offset & 7);
      for (uint32_t j0 = 0; j0 < span; j0 += CAPL) {
        const uint32_t count = min(uint32_t(CAPL), span - j0);
        if (j0) __syncthreads();  // the previous pass's records are no longer read
        stage_neighbour_records<S::kDirs>(g, first + j0, count, staged);
        if (j - j0 < count) {
          if constexpr (STREAM) {
            gather_box_pipelined<CH, VEC, kPipe, S::kTaps>(acc, side, [&](int t) {
              if (LAP && t == S::kCentre) return side.inactive();
              return side.tap(resolve_staged<S::kDirs>(staged, j - j0, x, y, z, S::di(t), S::dj(t), S::dk(t)));
            });
          } else {
            uint64_t st[S::kTaps];
            for_each_tap_staged<S>(staged, first + j0, s, [&](int t, uint32_t idx) { st[t] = idx; });
#pragma unroll
            for (int t = 0; t < S::kTaps; ++t) {
              if (LAP && t == S::kCentre) continue;
              add_row<CH, VEC>(acc, side, side.tap(uint32_t(st[t])));
            }
          }
        }
      }
    }
  }
  if (!valid) {
    if constexpr (kTouch) consume_touch(ahead);
    return;
  }
  // the Laplacian's centre enters only as -6 * centre: it reads as an inactive tap here
  if constexpr (STREAM) {
    if (cached) {
      if constexpr (!kPasses) {
        const uint32_t j = s.leaf - first;
        const int x = int(s.offset >> 6), y = int((s.offset >> 3) & 7), z = int(s.offset & 7);
        gather_box_pipelined<CH, VEC, kPipe, S::kTaps>(acc, side, [&](int t) {
          if (LAP && t == S::kCentre) return side.inactive();
          return side.tap(resolve_staged<S::kDirs>(staged, j, x, y, z, S::di(t), S::dj(t), S::dk(t)));
        });
      }
    } else {
      // tree walks streamed in three groups (as in the plain box): a group's walks
      // are independent chains of dependent loads that overlap one another, and
      // no walk waits behind a sidecar row load (vector loads retire in order)
      // except at a group's start; at most a third of the taps are held
      const VoxelCoord p = voxel_coord(g, s);
      constexpr int kG = (S::kTaps + 2) / 3;
      auto group = [&](auto first_c, auto n_c) {
        constexpr int F = decltype(first_c)::value, N = decltype(n_c)::value;
        uint32_t off[N];
#pragma unroll
        for (int k = 0; k < N; ++k) {
          const int t = F + k;
          off[k] = (LAP && t == S::kCentre) ? side.inactive()
                                            : side.tap(resolve_tree(g, root, p.x + S::di(t), p.y + S::dj(t),
                                                                    p.z + S::dk(t)));
        }
        gather_box_pipelined<CH, VEC, (kPipe < N ? kPipe : N), N>(acc, side, [&](int k) { return off[k]; });
      };
      group(std::integral_constant<int, 0>{}, std::integral_constant<int, kG>{});
      group(std::integral_constant<int, kG>{}, std::integral_constant<int, kG>{});
      group(std::integral_constant<int, 2 * kG>{}, std::integral_constant<int, S::kTaps - 2 * kG>{});
    }
  } else if (!kPasses || !cached) {
    uint64_t st[S::kTaps];
    auto keep = [&](int t, uint32_t idx) { st[t] = idx; };
    if (cached) for_each_tap_staged<S>(staged, first, s, keep);
    else for_each_tap<S>(g, root, s, keep);
#pragma unroll
    for (int j = 0; j < S::kTaps; ++j) {
      if (LAP && j == S::kCentre) continue;
      add_row<CH, VEC>(acc, side, side.tap(uint32_t(st[j])));
    }
  }
  const uint64_t idx = 1 + (uint64_t(b) << g.log2w) + threadIdx.x;
  if constexpr (LAP) {
    float centre[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) centre[c] = 0.0f;
    add_row<CH, VEC>(centre, side, side.row(uint32_t(idx)));
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const float six_c = 6.0f * centre[c];
      acc[c] = acc[c] - six_c;
    }
  }
  store_row<CH, VEC>(out + idx * C + ch0, acc);
  if constexpr (kTouch) consume_touch(ahead);
}

// The 7-direction filters with each sidecar row split over LANES = CH / 4
// work-items (one float4 of channels each; used for CH = 16), as in
// k_box_cached_split: the slots are decoded once into LDS (threads < W), the
// neighbour records staged (Cached), then every (slot, quarter) task resolves
// its taps and gathers its 16 bytes per tap in tap order.  The workgroup has at
// least W work-items.  Same taps, same order, same result as k_stencil.
template <class S, int CH, bool CACHED, bool LAP, bool STREAM, class SC = Sidecar>
__global__ void __launch_bounds__(512) k_stencil_split(DeviceGrid g, const float* __restrict__ sc, uint32_t sc_bytes,
                                                       float* __restrict__ out, uint32_t C, uint32_t ch0) {
  static_assert(CH % 4 == 0 && CH >= 8, "split rows need whole float4 groups");
  constexpr uint32_t LANES = CH / 4;
  constexpr int kPipe = VBM_PIPE_SPLIT < S::kTaps ? VBM_PIPE_SPLIT : S::kTaps;
  __shared__ StagedLeaf staged[CACHED ? kMaxCachedLeaves * S::kDirs : 1];  // neighbour leaf records
  __shared__ RootTile root_lds[CACHED ? 1 : kLdsRootTiles];                // the plain resolver's root table
  __shared__ uint32_t slot_info[512];  // per slot: leaf-in-block << 16 | voxel offset, or 0xFFFFFFFF
  const uint32_t W = 1u << g.log2w;
  const uint32_t b = block_of_workgroup(blockIdx.x, g.n_blocks);
  if (b >= g.n_blocks) return;  // padding workgroup
  if (blockIdx.x == 0 && threadIdx.x < CH) out[ch0 + threadIdx.x] = 0.0f;
  const SC side = SC::make(sc, sc_bytes, C, ch0);
  const uint32_t first = g.block_first_leaf[b];
  const uint32_t span = block_span(g, b);  // block-uniform: the barriers below are uniform
  const bool cached = CACHED && span <= kMaxCachedLeaves;
  if (threadIdx.x < W) {
    const Slot s = decode_own_slot(g, b);
    slot_info[threadIdx.x] = s.leaf == kSentinelLeaf ? 0xFFFFFFFFu : ((s.leaf - first) << 16) | s.offset;
  }
  // either ends with a barrier (the slot table is read across the workgroup);
  // the cached resolver's fallback walks search the global root table
  LdsRoot root{root_lds, false};
  if (!CACHED) root = stage_root_table(g, root_lds);
  else if (cached) stage_neighbour_records<S::kDirs>(g, first, span, staged);
  else __syncthreads();
  // The rows of the block this XCD starts VBM_PREFETCH_AHEAD blocks later, into
  // the L2 (as in the split box kernel).  Measured on MI355X: 7-9 % faster for
  // the 7-tap cross, within 2 % either way for the 19-tap axis stencil, which
  // therefore does without.
  constexpr bool kTouch = S::kTaps == 7;
  float ahead[1] = {0.0f};
  if constexpr (kTouch) {
    const uint32_t per = (g.n_blocks + 7) / 8;
    const uint32_t in_xcd = b - (blockIdx.x % 8) * per;
    const bool has = VBM_PREFETCH_AHEAD > 0 && in_xcd + VBM_PREFETCH_AHEAD < per;
    touch_block_lines(g, side, has ? b + VBM_PREFETCH_AHEAD : 0xFFFFFFFFu, ahead);
  }
  for (uint32_t task = threadIdx.x; task < W * LANES; task += blockDim.x) {
    const uint32_t info = slot_info[task / LANES];
    if (info == 0xFFFFFFFFu) continue;
    const uint32_t q = task % LANES, j = info >> 16, o = info & 0xFFFF;
    const int x = int(o >> 6), y = int((o >> 3) & 7), z = int(o & 7);
    // each tap resolved once per slot and shared in the quad ((LAP) the centre
    // reads as inactive: it enters only as -6 * centre)
    SlotTaps<LANES, S> taps;
    taps.resolve(q, [&](int t, int di, int dj, int dk) -> uint32_t {
      if (LAP && t == S::kCentre) return 0u;
      if (cached) return resolve_staged<S::kDirs>(staged, j, x, y, z, di, dj, dk);
      const Leaf& L = g.leaves[first + j];
      return resolve_tree(g, root, L.origin[0] + x + di, L.origin[1] + y + dj, L.origin[2] + z + dk);
    });
    auto tap = [&](int t) -> uint32_t { return taps(t); };
    // bytes 16 q .. 16 q + 15 of each tap's row
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (STREAM) {
      gather_box_pipelined<4, true, kPipe, S::kTaps>(acc, side, [&](int t) { return side.tap(tap(t)); }, 16 * q);
    } else {
      uint32_t st[S::kTaps];
#pragma unroll
      for (int t = 0; t < S::kTaps; ++t) st[t] = tap(t);
      gather_box_pipelined<4, true, kPipe, S::kTaps>(acc, side, [&](int t) { return side.tap(st[t]); }, 16 * q);
    }
    const uint64_t idx = 1 + (uint64_t(b) << g.log2w) + task / LANES;
    if constexpr (LAP) {
      float centre[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      add_row<4, true>(centre, side, side.row(uint32_t(idx)), 16 * q);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float six_c = 6.0f * centre[c];
        acc[c] = acc[c] - six_c;
      }
    }
    reinterpret_cast<float4*>(out + idx * C + ch0)[q] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  }
  if constexpr (kTouch) consume_touch(ahead);
}

// ---------------------------------------------------------------------------
// WENO consumer on the 19 axis taps
// ---------------------------------------------------------------------------
//
// openvdb PR #2258 ("A/B") times a 19-tap WENO consumer of the resolved
// taps without giving its arithmetic.  Here it is the fifth-order WENO scheme
// of Jiang and Shu (J. Comput. Phys. 126, 1996) in its Hamilton-Jacobi form:
// along each axis the left- and right-biased derivatives of the field from
// its seven values u[-3..3] (unit spacing), combined by Godunov's upwind rule
// into |grad u|^2 per channel.  An inactive tap (index 0) reads sidecar row 0,
// the background.  Every fp32 operation below is one IEEE rounding in the
// order written (no contraction, correctly rounded division), which fixes the
// result bit for bit:
//   differences  d[j] = u[j+1] - u[j], j = 0..5
//   left         weno5(d0, d1, d2, d3, d4), right weno5(d5, d4, d3, d2, d1)
//   weno5(a..e)  candidates ((2a - 7b) + 11c)/6, ((-b + 5c) + 2d)/6, ((2c + 5d) - e)/6;
//                indicators (13 q^2)/12 + (r^2)*0.25 with q, r =
//                ((a - 2b) + c, (a - 4b) + 3c), ((b - 2c) + d, b - d),
//                ((c - 2d) + e, (3c - 4d) + e); t = indicator + 1e-6;
//                weights 1/(t1 t1), 6/(t2 t2), 3/(t3 t3);
//                result ((w1 p1 + w2 p2) + w3 p3) / ((w1 + w2) + w3)
//   Godunov      centre > 0: max(max(left, 0)^2, min(right, 0)^2), else
//                max(min(left, 0)^2, max(right, 0)^2); axes summed (x + y) + z.

// FAST divides by 6 and 12 and forms the three weights n / t^2 with the
// shortcuts of vbm_division.hpp, which the caller may choose only when
// weno_fast_ok holds for the tap values; otherwise every division is the IEEE
// one.  Both give the same bits on that range.
template <bool FAST>
__device__ __forceinline__ float weno5_derivative(float a, float b, float c, float d, float e) {
  auto by6 = [](float x) { return FAST ? vbm_div::div_const(x, 6.0f, 1.0f / 6.0f) : x / 6.0f; };
  auto by12 = [](float x) { return FAST ? vbm_div::div_const(x, 12.0f, 1.0f / 12.0f) : x / 12.0f; };
  const float p1 = by6((2.0f * a - 7.0f * b) + 11.0f * c);
  const float p2 = by6((-b + 5.0f * c) + 2.0f * d);
  const float p3 = by6((2.0f * c + 5.0f * d) - e);
  const float qa = (a - 2.0f * b) + c, ra = (a - 4.0f * b) + 3.0f * c;
  const float qb = (b - 2.0f * c) + d, rb = b - d;
  const float qc = (c - 2.0f * d) + e, rc = (3.0f * c - 4.0f * d) + e;
  const float ta = (by12(13.0f * (qa * qa)) + (ra * ra) * 0.25f) + 1.0e-6f;
  const float tb = (by12(13.0f * (qb * qb)) + (rb * rb) * 0.25f) + 1.0e-6f;
  const float tc = (by12(13.0f * (qc * qc)) + (rc * rc) * 0.25f) + 1.0e-6f;
  const float ya = ta * ta, yb = tb * tb, yc = tc * tc;
  float wa, wb, wc;
  if constexpr (FAST) {
    wa = vbm_div::recip(ya);
    wb = vbm_div::div_by_recip(6.0f, yb, vbm_div::recip(yb));
    wc = vbm_div::div_by_recip(3.0f, yc, vbm_div::recip(yc));
  } else {
    wa = 1.0f / ya, wb = 6.0f / yb, wc = 3.0f / yc;
  }
  return ((wa * p1 + wb * p2) + wc * p3) / ((wa + wb) + wc);
}

// |grad u|^2 contribution of one axis from its seven values u[0..6] = u[-3..3].
template <bool FAST>
__device__ __forceinline__ float weno_axis_sq(const float (&u)[7], bool outside) {
  float d[6];
#pragma unroll
  for (int j = 0; j < 6; ++j) d[j] = u[j + 1] - u[j];
  const float left = weno5_derivative<FAST>(d[0], d[1], d[2], d[3], d[4]);
  const float right = weno5_derivative<FAST>(d[5], d[4], d[3], d[2], d[1]);
  const float lo = outside ? (left > 0.0f ? left : 0.0f) : (left < 0.0f ? left : 0.0f);
  const float hi = outside ? (right < 0.0f ? right : 0.0f) : (right > 0.0f ? right : 0.0f);
  const float l2 = lo * lo, h2 = hi * hi;
  return l2 > h2 ? l2 : h2;
}

// Axis-stencil tap holding u[k - 3] of axis a (0 = x, 1 = y, 2 = z), k = 0..6;
// AxisShape orders its taps x-3..x-1, y-3..y-1, z-3..z-1, centre, z+1..z+3,
// y+1..y+3, x+1..x+3.
__host__ __device__ constexpr int weno_tap(int a, int k) {
  return k == 3 ? 9 : k < 3 ? 3 * a + k : (a == 2 ? 10 + (k - 4) : a == 1 ? 13 + (k - 4) : 16 + (k - 4));
}

// The WENO consumer per channel from the 19 tap values v[0..18] of one channel.
template <bool FAST>
__device__ __forceinline__ float weno_norm_sq(const float (&v)[kAxisTaps]) {
  const bool outside = v[9] > 0.0f;
  float sum = 0.0f;
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    float u[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) u[k] = v[weno_tap(a, k)];
    const float g2 = weno_axis_sq<FAST>(u, outside);
    sum = a == 0 ? g2 : sum + g2;
  }
  return sum;
}

// Whether one channel's tap values allow the FAST divisions: each value zero
// or of magnitude in [2^-40, 2^27] (the sum of magnitudes bounds them above
// and is NaN or infinite when a value is; twice the magnitude bits less two,
// wrapping for zero, bounds the nonzero ones below).  Every value is then a
// multiple of 2^-63, and so is every difference, numerator and second
// difference q formed from them by fp32 additions and small integer multiples:
// a nonzero numerator or 13 q^2 is at least 2^-63 resp. 13 * 2^-126 (above
// 2^-124) and all stay below 2^70, inside the range of div_const.  A
// difference is at most 2^28, so q and r are at most 2^30 and 2^31, an
// indicator (13 q^2) / 12 + r^2 / 4 below 2^61.1, and t^2 lies in
// [1e-12, 2^123): inside [2^-40, 2^126), the range of recip and div_by_recip.
// The one way the shortcuts part from IEEE division there, a candidate of -0
// coming out +0, does not reach the output: a zero candidate adds nothing to
// the nonzero sums it enters, and a zero derivative of either sign becomes +0
// in Godunov's rule before it is squared.
__device__ __forceinline__ bool weno_fast_ok(const float (&v)[kAxisTaps]) {
  constexpr uint32_t kLow = 0x2B800000u;  // bits of 2^-40
  float mag = 0.0f;
  uint32_t low = 0xFFFFFFFFu;
#pragma unroll
  for (int t = 0; t < kAxisTaps; ++t) {
    mag += __builtin_fabsf(v[t]);
    low = min(low, (__builtin_bit_cast(uint32_t, v[t]) << 1) - 2u);
  }
  return mag <= 0x1p27f && low >= 2u * kLow - 2u;
}

// One channel: with the FAST divisions where the range check allows them.  The
// values enter the IEEE path through an empty register constraint, so that the
// compiler cannot share its subexpressions with the FAST path and hoist them
// above the branch (which held both paths' values live: 82 VGPRs against 60).
__device__ __forceinline__ float weno_channel(const float (&v)[kAxisTaps]) {
  if (weno_fast_ok(v)) return weno_norm_sq<true>(v);
  float w[kAxisTaps];
#pragma unroll
  for (int t = 0; t < kAxisTaps; ++t) {
    w[t] = v[t];
    asm volatile("" : "+v"(w[t]));
  }
  return weno_norm_sq<false>(w);
}

// The WENO consumer kernel: one work-item per slot.  The 19 axis taps are
// resolved by tree walks or through the staged neighbour records (CACHED),
// either each as its value load is issued (STREAM) or all into an array first;
// then the channels are processed four at a time (VEC: 16-byte loads and
// stores) or one at a time, reusing the resolved taps.
template <bool VEC, bool CACHED, bool STREAM, class SC = Sidecar>
__global__ void __launch_bounds__(512) k_weno(DeviceGrid g, const float* __restrict__ sc, uint32_t sc_bytes,
                                              float* __restrict__ out, uint32_t C) {
  using S = AxisShape;
  __shared__ StagedLeaf staged[CACHED ? kMaxCachedLeaves * S::kDirs : 1];  // neighbour leaf records
  __shared__ RootTile root_lds[CACHED ? 1 : kLdsRootTiles];                // the plain resolver's root table
  const uint32_t b = blockIdx.x;
  if (blockIdx.x == 0)
    for (uint32_t c = threadIdx.x; c < C; c += blockDim.x) out[c] = 0.0f;  // row 0
  const Slot s = decode_own_slot(g, b);
  const bool valid = s.leaf != kSentinelLeaf;
  bool cached = false;
  uint32_t first = 0;
  if constexpr (CACHED) {
    first = g.block_first_leaf[b];
    const uint32_t span = block_span(g, b);  // block-uniform: the barrier below is uniform
    if (span <= kMaxCachedLeaves) {
      stage_neighbour_records<S::kDirs>(g, first, span, staged);
      cached = true;
    }
  }
  // the plain resolver's walks search the root table in LDS; the cached one's
  // fallback walks (blocks spanning more than kMaxCachedLeaves) the global table
  const LdsRoot root = CACHED ? LdsRoot{root_lds, false} : stage_root_table(g, root_lds);
  if (!valid) return;
  const SC side = SC::make(sc, sc_bytes, C, 0);
  const int x = int(s.offset >> 6), y = int((s.offset >> 3) & 7), z = int(s.offset & 7);
  const uint32_t j = s.leaf - first;
  VoxelCoord p{0, 0, 0};
  if (!cached) p = voxel_coord(g, s);
  auto resolve = [&](int t) -> uint32_t {
    if (cached) return resolve_staged<S::kDirs>(staged, j, x, y, z, S::di(t), S::dj(t), S::dk(t));
    return resolve_tree(g, root, p.x + S::di(t), p.y + S::dj(t), p.z + S::dk(t));
  };
  uint32_t row[S::kTaps];  // handle of each tap's row (index 0: row 0, the background)
  const uint64_t idx = 1 + (uint64_t(b) << g.log2w) + threadIdx.x;
  if constexpr (VEC) {
    // one chunk of four channels: q-th float4 of every tap row, then the four
    // channels one after another (fenced, so their arithmetic is not interleaved)
    f32x4 v4[S::kTaps];
    auto finish = [&](uint32_t q) {
      float r[4];
      bool fast = true;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        __builtin_amdgcn_sched_barrier(0);
        float v[S::kTaps];
#pragma unroll
        for (int t = 0; t < S::kTaps; ++t) v[t] = v4[t][c];
        fast = fast && weno_fast_ok(v);
        r[c] = weno_norm_sq<true>(v);
      }
      if (!fast) {  // a value outside that range: the four channels again with IEEE divisions
#pragma unroll 1
        for (int c = 0; c < 4; ++c) {  // channel c sits in component 0 after c rotations
          float v[S::kTaps];
#pragma unroll
          for (int t = 0; t < S::kTaps; ++t) {
            v[t] = v4[t][0];
            v4[t] = f32x4{v4[t][1], v4[t][2], v4[t][3], v4[t][0]};
          }
          const float exact = weno_norm_sq<false>(v);
          r[0] = r[1], r[1] = r[2], r[2] = r[3], r[3] = exact;
        }
      }
      reinterpret_cast<float4*>(out + idx * C)[q] = make_float4(r[0], r[1], r[2], r[3]);
    };
    auto load = [&](uint32_t q) {
#pragma unroll
      for (int t = 0; t < S::kTaps; ++t)
        v4[t] = side.load4(row[t], 16 * q);
    };
    if constexpr (STREAM) {  // first chunk: taps resolved and loaded in three groups (see k_stencil)
#pragma unroll
      for (int grp = 0; grp < 3; ++grp) {
        constexpr int kG = (S::kTaps + 2) / 3;
#pragma unroll
        for (int t = grp * kG; t < (grp + 1) * kG && t < S::kTaps; ++t) row[t] = side.row(resolve(t));
#pragma unroll
        for (int t = grp * kG; t < (grp + 1) * kG && t < S::kTaps; ++t) v4[t] = side.load4(row[t], 0);
      }
    } else {
#pragma unroll
      for (int t = 0; t < S::kTaps; ++t) row[t] = side.row(resolve(t));
      load(0);
    }
    finish(0);
    for (uint32_t q = 1; q < C / 4; ++q) {
      load(q);
      finish(q);
    }
  } else {
    float v[S::kTaps];
    if constexpr (STREAM) {  // taps resolved and loaded in three groups (see k_stencil)
#pragma unroll
      for (int grp = 0; grp < 3; ++grp) {
        constexpr int kG = (S::kTaps + 2) / 3;
#pragma unroll
        for (int t = grp * kG; t < (grp + 1) * kG && t < S::kTaps; ++t) row[t] = side.row(resolve(t));
#pragma unroll
        for (int t = grp * kG; t < (grp + 1) * kG && t < S::kTaps; ++t) v[t] = side.load1(row[t], 0);
      }
    } else {
#pragma unroll
      for (int t = 0; t < S::kTaps; ++t) row[t] = side.row(resolve(t));
#pragma unroll
      for (int t = 0; t < S::kTaps; ++t)
        v[t] = side.load1(row[t], 0);
    }
    out[idx * C] = weno_channel(v);
    for (uint32_t ch = 1; ch < C; ++ch) {
#pragma unroll
      for (int t = 0; t < S::kTaps; ++t)
        v[t] = side.load1(row[t], 4 * ch);
      out[idx * C + ch] = weno_channel(v);
    }
  }
}

// ---------------------------------------------------------------------------
// device-side VBM metadata build
// ---------------------------------------------------------------------------
//
// From the leaf masks in the blob, the device recomputes what the index grid
// and the VBM derive from them (openvdb PR #2258, "What changed"; openvdb PR
// #2263, "Built on the register-decode API"):
//   * per leaf the 9-bit prefix directory (field k = active voxels in mask
//     words 0..k) and leafFirst (1 + active voxels in all earlier leaves);
//   * per block the leaf owning its first index and the jumpMap bits of the
//     slots >= 1 whose index starts a leaf.
// Five launches: per-leaf counts and directories (with per-256-leaf sums), one
// workgroup scanning the sums, every leaf's leafFirst, the jumpMap words
// cleared, and the block metadata scattered by the leaves.

struct MutableGrid {
  Leaf* leaves;
  uint32_t* block_first_leaf;
  uint64_t* block_jump;
  uint32_t n_leaves;
  uint32_t n_blocks;
  int32_t log2w;
};

// Per leaf: prefix directory, and the active count parked in `first` for the
// scan; per workgroup of 256 leaves the sum of their counts, parked in
// block_jump[workgroup] (the jumpMap words are rewritten at the end; they
// number at least N / 64 >= L / 64 > L / 256).  A leaf left without any active
// voxel by an edit marks its group sum with kEmptyLeaf (bit 63; a group sum is
// at most 256 * 512).
constexpr uint64_t kEmptyLeaf = uint64_t(1) << 63;

__global__ void __launch_bounds__(256) k_meta_counts(MutableGrid m) {
  __shared__ uint32_t group_sum, empty;
  const uint32_t l = blockIdx.x * blockDim.x + threadIdx.x;
  if (threadIdx.x == 0) group_sum = empty = 0;
  __syncthreads();
  if (l < m.n_leaves) {
    Leaf& L = m.leaves[l];
    uint32_t count = 0, lo = 0, hi = 0;
#pragma unroll
    for (uint32_t w = 0; w < 8; ++w) {
      count += __popcll(L.mask[w]);
      if (w < 7) {  // field w at bits 9w .. 9w+8, assembled in two 32-bit halves
        const uint32_t p = 9 * w;
        if (p < 32) lo |= count << p;
        if (p + 9 > 32) hi |= p < 32 ? count >> (32 - p) : count << (p - 32);
      }
    }
    L.prefix = uint64_t(lo) | (uint64_t(hi) << 32);
    L.first = count;
    atomicAdd(&group_sum, count);
    if (count == 0) atomicOr(&empty, 1u);
  }
  __syncthreads();
  if (threadIdx.x == 0) m.block_jump[blockIdx.x] = group_sum | (empty ? kEmptyLeaf : 0);
}

// One workgroup: the G group sums in block_jump[0 .. G) become exclusive
// prefix sums; *total = their sum (N), or ~0 if a leaf is empty.  Each
// work-item owns a contiguous run.
__global__ void __launch_bounds__(1024) k_meta_scan(MutableGrid m, uint32_t G, uint64_t* __restrict__ total) {
  __shared__ uint64_t part[1024];
  __shared__ uint32_t empty;
  const uint32_t T = blockDim.x, t = threadIdx.x;
  if (t == 0) empty = 0;
  const uint32_t per = (G + T - 1) / T;
  const uint32_t a = min(G, t * per), e = min(G, a + per);
  uint64_t s = 0;
  bool any_empty = false;
  for (uint32_t k = a; k < e; ++k) {
    const uint64_t v = m.block_jump[k];
    any_empty |= (v & kEmptyLeaf) != 0;
    s += v & ~kEmptyLeaf;
  }
  part[t] = s;
  __syncthreads();
  if (any_empty) atomicOr(&empty, 1u);
  for (uint32_t d = 1; d < T; d <<= 1) {  // inclusive scan of the runs' sums
    const uint64_t v = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  uint64_t run = t ? part[t - 1] : 0;
  for (uint32_t k = a; k < e; ++k) {
    const uint64_t c = m.block_jump[k] & ~kEmptyLeaf;
    m.block_jump[k] = run;
    run += c;
  }
  if (t == T - 1 && total) *total = empty ? ~uint64_t(0) : part[T - 1];
}

// Per workgroup of 256 leaves: leafFirst = 1 + the group's offset + the
// exclusive scan of the counts inside the group.
__global__ void __launch_bounds__(256) k_meta_first(MutableGrid m) {
  __shared__ uint32_t sums[256];
  const uint32_t t = threadIdx.x, l = blockIdx.x * blockDim.x + t;
  const uint32_t count = l < m.n_leaves ? uint32_t(m.leaves[l].first) : 0u;
  sums[t] = count;
  __syncthreads();
  for (uint32_t d = 1; d < 256; d <<= 1) {  // inclusive scan
    const uint32_t v = t >= d ? sums[t - d] : 0u;
    __syncthreads();
    sums[t] += v;
    __syncthreads();
  }
  if (l < m.n_leaves) m.leaves[l].first = 1 + m.block_jump[blockIdx.x] + (sums[t] - count);
}

// The jumpMap words are cleared once the scan's partial sums are consumed.
__global__ void __launch_bounds__(256) k_meta_clear_jump(MutableGrid m) {
  const uint64_t words = uint64_t(m.n_blocks) << (m.log2w - 6);
  for (uint64_t i = blockIdx.x * uint64_t(blockDim.x) + threadIdx.x; i < words; i += uint64_t(gridDim.x) * blockDim.x)
    m.block_jump[i] = 0;
}

// Block metadata by scatter, one work-item per leaf (first index f, next
// leaf's first index or N + 1 as its end): the leaf sets the jumpMap bit of
// slot (f - 1) % W of block (f - 1) / W unless it starts that block, and is
// firstLeafID of every block whose first index 1 + bW lies in [f, end).
// Blocks are those of the header's N (ids past them are skipped).
__global__ void __launch_bounds__(256) k_meta_scatter(MutableGrid m, uint64_t n_active) {
  const uint32_t l = blockIdx.x * blockDim.x + threadIdx.x;
  if (l >= m.n_leaves) return;
  const uint64_t W = uint64_t(1) << m.log2w;
  const uint64_t f = m.leaves[l].first;
  const uint64_t end = l + 1 < m.n_leaves ? uint64_t(m.leaves[l + 1].first) : n_active + 1;
  const uint64_t s = (f - 1) & (W - 1), b = (f - 1) >> m.log2w;
  if (s != 0 && b < m.n_blocks)  // the bit's 32-bit half of the jumpMap word (32-bit shifts only)
    atomicOr(reinterpret_cast<uint32_t*>(&m.block_jump[(b << (m.log2w - 6)) + (s >> 6)]) + ((s >> 5) & 1),
             1u << (s & 31));
  for (uint64_t bb = (f - 1 + W - 1) >> m.log2w; bb < m.n_blocks && 1 + (bb << m.log2w) < end; ++bb)
    m.block_first_leaf[bb] = l;
}

__global__ void k_zero_index_row(float* __restrict__ out, uint32_t C) {
  for (uint32_t c = threadIdx.x; c < C; c += blockDim.x) out[c] = 0.0f;
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------

int check_grid(const vbm_grid* grid, const void* d_blob) {
  if (!grid || grid->magic != VBM_GRID_MAGIC) return VBM_ERR_ARG;
  if (grid->log2_width < 6 || grid->log2_width > 9) return VBM_ERR_ARG;
  if (grid->n_active > 0xFFFFFFFEull) return VBM_ERR_ARG;
  const uint64_t W = uint64_t(1) << grid->log2_width;
  if (grid->n_blocks != (grid->n_active + W - 1) / W) return VBM_ERR_ARG;
  if ((grid->n_active == 0) != (grid->n_leaves == 0)) return VBM_ERR_ARG;
  if (grid->n_upper != grid->n_root) return VBM_ERR_ARG;
  const uint64_t ends[6] = {grid->off_leaves + uint64_t(grid->n_leaves) * 128,
                            grid->off_root + uint64_t(grid->n_root) * 16,
                            grid->off_upper + uint64_t(grid->n_upper) * 32768 * 4,
                            grid->off_lower + uint64_t(grid->n_lower) * 4096 * 4,
                            grid->off_block_first_leaf + uint64_t(grid->n_blocks) * 4,
                            grid->off_block_jump + uint64_t(grid->n_blocks) * (W / 8)};
  for (uint64_t e : ends)
    if (e > grid->blob_bytes) return VBM_ERR_ARG;
  if (grid->n_active > 0 && !d_blob) return VBM_ERR_ARG;
  return VBM_OK;
}

DeviceGrid device_grid(const vbm_grid* grid, const void* d_blob) { return device_grid_of(*grid, d_blob); }

using vbm_host::check_kernel_memory;
using vbm_host::launch_status;

int check_float_buffers(const vbm_grid* grid, const float* sc, const float* out, int C) {
  if (!sc || !out || C < 1) return VBM_ERR_ARG;
  if (uint64_t(C) * 4 > 0xFFFFFFFFull) return VBM_ERR_SIZE;  // a row's byte size is 32-bit
  if ((reinterpret_cast<uintptr_t>(sc) | reinterpret_cast<uintptr_t>(out)) & 3) return VBM_ERR_ALIGN;
  const uint64_t bytes = (grid->n_active + 1) * uint64_t(C) * 4;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(sc), b0 = reinterpret_cast<uintptr_t>(out);
  if (a0 < b0 + bytes && b0 < a0 + bytes) return VBM_ERR_ALIAS;
  return VBM_OK;
}

// Whether a filter reaches its sidecar rows by 64-bit addresses: asked for, or
// a sidecar whose (N+1) * C * 4 bytes do not end below the buffer-resource
// offset kInactive that marks an inactive tap.
bool wide_rows(const vbm_grid* grid, int C, int flags) {
  return (flags & VBM_WIDE_ROWS) || (grid->n_active + 1) * uint64_t(C) * 4 > kInactive;
}

// Brick capacity (spanned leaves resolved per pass) for BlockWidth 2^log2w:
// one pass covers about 98% of the blocks of a sphere shell.  A W64 workgroup
// is a single wave, so its LDS sets how many are resident: capacity 2 (8.3 KB)
// keeps 19 per CU where 3 kept 12, measured 12-15 % faster on the shell at one
// to four channels (capacity 1: more passes, a little slower than 2).
#ifndef VBM_CAP_W128
#define VBM_CAP_W128 3
#endif
#ifndef VBM_CAP_W512
#define VBM_CAP_W512 8
#endif
uint32_t brick_capacity(int log2w) {
  return log2w <= 6 ? 2u : log2w == 7 ? uint32_t(VBM_CAP_W128) : log2w == 8 ? 6u : uint32_t(VBM_CAP_W512);
}

// Brick capacity of the split-row kernel, whose staged leaf records take
// 27 * 80 bytes of LDS per spanned leaf on top of the brick: sized so that a
// W128 workgroup still fits eight to a CU.  At W64 (workgroups of two waves at
// 8 channels, four at 16) capacity 2 is 11 % faster than 3 at 8 channels and
// 3 % slower at 16, measured on the shell.
#ifndef VBM_SPLIT_CAP_W128
#define VBM_SPLIT_CAP_W128 3
#endif
#ifndef VBM_SPLIT_CAP_W512
#define VBM_SPLIT_CAP_W512 8
#endif
uint32_t split_capacity(int log2w, int ch) {
  if (!VBM_STAGE_LEAVES) return brick_capacity(log2w);
  return log2w <= 6 ? (ch == 8 ? 2u : 3u) : log2w == 7 ? uint32_t(VBM_SPLIT_CAP_W128) : log2w == 8 ? 4u : uint32_t(VBM_SPLIT_CAP_W512);
}

template <bool CACHED, bool STREAM, bool WIDE = false>
struct BoxLauncher {
  static constexpr uint32_t kWideChunk = 16;  // widest channel chunk of the wide path
  template <int CH, bool VEC>
  static void go(const DeviceGrid& g, const float* sc, uint32_t bytes, float* out, uint32_t C, uint32_t ch0,
                 hipStream_t st) {
    if constexpr (WIDE && CACHED && VEC && (CH == 8 || CH == 16)) {  // rows by 64-bit addresses
      const uint32_t cap = split_capacity(g.log2w, CH);
      const uint32_t W = 1u << g.log2w;
      const uint32_t tasks = W * (CH / 4);
      const uint32_t threads = tasks < VBM_SPLIT_MAX ? tasks : (W > VBM_SPLIT_MAX ? W : VBM_SPLIT_MAX);
      hipLaunchKernelGGL((k_box_cached_split<CH, STREAM, WideSidecar>), dim3(box_grid_size(g.n_blocks)),
                         dim3(threads), split_lds_bytes(cap, W), st, g, sc, bytes, out, C, ch0, cap);
    } else if constexpr (WIDE) {
      if constexpr (CACHED) {
        const uint32_t cap = brick_capacity(g.log2w);
        hipLaunchKernelGGL((k_box_cached<CH, VEC, STREAM, WideSidecar>), dim3(box_grid_size(g.n_blocks)),
                           dim3(1u << g.log2w), brick_lds_bytes(cap), st, g, sc, bytes, out, C, ch0, cap);
      } else {
        hipLaunchKernelGGL((k_box_plain<CH, VEC, STREAM, WideSidecar>), dim3(g.n_blocks), dim3(1u << g.log2w), 0,
                           st, g, sc, bytes, out, C, ch0);
      }
    } else if constexpr (CACHED && VEC && (CH == 8 || CH == 16)) {
      const uint32_t cap = split_capacity(g.log2w, CH);
      const uint32_t W = 1u << g.log2w;
      const uint32_t tasks = W * (CH / 4);
      const uint32_t threads = tasks < VBM_SPLIT_MAX ? tasks : (W > VBM_SPLIT_MAX ? W : VBM_SPLIT_MAX);
      hipLaunchKernelGGL((k_box_cached_split<CH, STREAM>), dim3(box_grid_size(g.n_blocks)), dim3(threads),
                         split_lds_bytes(cap, W), st, g, sc, bytes, out, C, ch0, cap);
    } else if constexpr (CACHED) {
      const uint32_t cap = brick_capacity(g.log2w);
      if constexpr (CH == 1) {
        // rows 4 bytes apart: value bricks.  Measured on the 1.29M-voxel shell:
        // 3-7 % faster than the handle bricks at W256 and W512, 5-14 % slower
        // at W64 and W128, where a block rebuilds more brick columns per voxel
        // and the value loads lengthen its setup chain
        if (C == 1 && g.log2w >= 8) {
          hipLaunchKernelGGL((k_box_cached<1, false, STREAM, Sidecar, true>), dim3(box_grid_size(g.n_blocks)),
                             dim3(1u << g.log2w), brick_lds_bytes(cap), st, g, sc, bytes, out, C, ch0, cap);
          return;
        }
      }
      hipLaunchKernelGGL((k_box_cached<CH, VEC, STREAM>), dim3(box_grid_size(g.n_blocks)), dim3(1u << g.log2w),
                         brick_lds_bytes(cap), st, g, sc, bytes, out, C, ch0, cap);
    } else if constexpr (VBM_PLAIN_SPLIT && VEC && CH == 16) {
      // tree walk with the rows split over quads: the split 7-direction kernel on
      // the box shape, no table (each tap walked once per slot, shared in the quad)
      const uint32_t W = 1u << g.log2w, tasks = W * (CH / 4);
      const uint32_t threads = tasks < 256 ? tasks : (W > 256 ? W : 256u);
      hipLaunchKernelGGL((k_stencil_split<BoxShape, CH, false, false, STREAM>), dim3(box_grid_size(g.n_blocks)),
                         dim3(threads), 0, st, g, sc, bytes, out, C, ch0);
    } else {
      hipLaunchKernelGGL((k_box_plain<CH, VEC, STREAM>), dim3(g.n_blocks), dim3(1u << g.log2w), 0, st, g, sc,
                         bytes, out, C, ch0);
    }
  }
};

template <class S, bool CACHED, bool LAP, bool STREAM, bool WIDE = false>
struct StencilLauncher {
  static constexpr uint32_t kWideChunk = VBM_STENCIL_SPLIT ? 16 : 8;  // one row per work-item at 16 would spill
  template <int CH, bool VEC>
  static void go(const DeviceGrid& g, const float* sc, uint32_t bytes, float* out, uint32_t C, uint32_t ch0,
                 hipStream_t st) {
    using SC = std::conditional_t<WIDE, WideSidecar, Sidecar>;
    if constexpr (VBM_STENCIL_SPLIT && VEC && CH == 16) {  // at CH = 8 one work-item per row is as fast or faster
      const uint32_t W = 1u << g.log2w, tasks = W * (CH / 4);
      const uint32_t threads = tasks < 256 ? tasks : (W > 256 ? W : 256u);
      hipLaunchKernelGGL((k_stencil_split<S, CH, CACHED, LAP, STREAM, SC>), dim3(box_grid_size(g.n_blocks)),
                         dim3(threads), 0, st, g, sc, bytes, out, C, ch0);
    } else if constexpr (WIDE) {
      hipLaunchKernelGGL((k_stencil<S, CH, VEC, CACHED, LAP, STREAM, WideSidecar>), dim3(g.n_blocks),
                         dim3(1u << g.log2w), 0, st, g, sc, bytes, out, C, ch0);
    } else {
      if constexpr (CACHED && S::kTaps == 7) {
        if (g.log2w == 6) {
          // single-wave workgroups: records staged four leaves at a time, so that
          // LDS (2.2 KB instead of 8.75 KB) does not cap how many are resident.
          // Measured on the shell: cross sum and Laplacian 13-17 % faster at one
          // channel, 0-10 % at eight; the 19-tap axis stencil's pass loop needs
          // 105 VGPRs instead of 56 at eight channels and is 5 % slower, so it
          // keeps one pass
          hipLaunchKernelGGL((k_stencil<S, CH, VEC, CACHED, LAP, STREAM, Sidecar, 4>), dim3(g.n_blocks), dim3(64), 0,
                             st, g, sc, bytes, out, C, ch0);
          return;
        }
      }
      hipLaunchKernelGGL((k_stencil<S, CH, VEC, CACHED, LAP, STREAM>), dim3(g.n_blocks), dim3(1u << g.log2w), 0, st,
                         g, sc, bytes, out, C, ch0);
    }
  }
};

// Channel chunks of one launch: exact kernels for C in {1,2,3,4,8,16}, other
// C as a sequence of 16/8/4/2/1-channel chunks.  float4 access when C is a
// multiple of 4 and both buffers are 16-byte aligned.
template <class L>
void launch_channels(const DeviceGrid& g, const float* sc, float* out, int C, hipStream_t st) {
  const uint32_t bytes = uint32_t((uint64_t(g.n_active) + 1) * uint64_t(C) * 4);
  const bool vec = ((reinterpret_cast<uintptr_t>(sc) | reinterpret_cast<uintptr_t>(out)) & 15) == 0 && C % 4 == 0;
  const uint32_t uc = uint32_t(C);
  switch (C) {
    case 1: L::template go<1, false>(g, sc, bytes, out, uc, 0, st); return;
    case 2: L::template go<2, false>(g, sc, bytes, out, uc, 0, st); return;
    case 3: L::template go<3, false>(g, sc, bytes, out, uc, 0, st); return;
    default: break;
  }
  uint32_t ch0 = 0;
  while (ch0 < uc) {
    const uint32_t left = uc - ch0;
    if (left >= 16) {
      if (vec) L::template go<16, true>(g, sc, bytes, out, uc, ch0, st);
      else L::template go<16, false>(g, sc, bytes, out, uc, ch0, st);
      ch0 += 16;
    } else if (left >= 8) {
      if (vec) L::template go<8, true>(g, sc, bytes, out, uc, ch0, st);
      else L::template go<8, false>(g, sc, bytes, out, uc, ch0, st);
      ch0 += 8;
    } else if (left >= 4) {
      if (vec) L::template go<4, true>(g, sc, bytes, out, uc, ch0, st);
      else L::template go<4, false>(g, sc, bytes, out, uc, ch0, st);
      ch0 += 4;
    } else if (left >= 2) {
      L::template go<2, false>(g, sc, bytes, out, uc, ch0, st);
      ch0 += 2;
    } else {
      L::template go<1, false>(g, sc, bytes, out, uc, ch0, st);
      ch0 += 1;
    }
  }
}

// Channel chunks with rows reached by 64-bit addresses (a sidecar of 4 GiB or
// more, or VBM_WIDE_ROWS): 16 (up to L::kWideChunk) / 8 / 4 channels as float4
// when both buffers are 16-byte aligned and C is a multiple of 4, else one
// channel at a time.
template <class L>
void launch_channels_wide(const DeviceGrid& g, const float* sc, float* out, int C, hipStream_t st) {
  const bool vec = ((reinterpret_cast<uintptr_t>(sc) | reinterpret_cast<uintptr_t>(out)) & 15) == 0 && C % 4 == 0;
  const uint32_t uc = uint32_t(C);
  for (uint32_t ch0 = 0; ch0 < uc;) {
    const uint32_t left = uc - ch0;
    if constexpr (L::kWideChunk >= 16) {
      if (vec && left >= 16) {
        L::template go<16, true>(g, sc, 0u, out, uc, ch0, st);
        ch0 += 16;
        continue;
      }
    }
    if (vec && left >= 8) {
      L::template go<8, true>(g, sc, 0u, out, uc, ch0, st);
      ch0 += 8;
    } else if (vec) {
      L::template go<4, true>(g, sc, 0u, out, uc, ch0, st);
      ch0 += 4;
    } else {
      L::template go<1, false>(g, sc, 0u, out, uc, ch0, st);
      ch0 += 1;
    }
  }
}

}  // namespace

extern "C" int vbm_decode(const vbm_grid* grid, const void* d_blob, uint32_t* d_leaf_index, uint16_t* d_voxel_offset,
                          void* stream) {
  int rc = check_grid(grid, d_blob);
  if (rc) return rc;
  if (grid->n_blocks == 0) return VBM_OK;
  if (!d_leaf_index || !d_voxel_offset) return VBM_ERR_ARG;
  if ((rc = check_kernel_memory({d_blob, d_leaf_index, d_voxel_offset}))) return rc;
  const DeviceGrid g = device_grid(grid, d_blob);
  const uint32_t W = 1u << g.log2w;
  const uint32_t threads = W > VBM_DECODE_THREADS ? W : uint32_t(VBM_DECODE_THREADS);
  const uint32_t per_wg = threads / W;
  hipLaunchKernelGGL(k_decode, dim3((g.n_blocks + per_wg - 1) / per_wg), dim3(threads), 0,
                     static_cast<hipStream_t>(stream), g, d_leaf_index, d_voxel_offset);
  return launch_status();
}

extern "C" int vbm_decode_sweep(const vbm_grid* grid, const void* d_blob, uint32_t* d_leaf_index,
                                uint16_t* d_voxel_offset, void* stream) {
  int rc = check_grid(grid, d_blob);
  if (rc) return rc;
  if (grid->n_blocks == 0) return VBM_OK;
  if (!d_leaf_index || !d_voxel_offset) return VBM_ERR_ARG;
  if ((rc = check_kernel_memory({d_blob, d_leaf_index, d_voxel_offset}))) return rc;
  const DeviceGrid g = device_grid(grid, d_blob);
  hipLaunchKernelGGL(k_decode_sweep, dim3(g.n_blocks), dim3(1u << g.log2w), 0, static_cast<hipStream_t>(stream), g,
                     d_leaf_index, d_voxel_offset);
  return launch_status();
}

extern "C" int vbm_stencil_indices(const vbm_grid* grid, const void* d_blob, int shape, int flags, uint64_t* d_taps,
                                   void* stream) {
  int rc = check_grid(grid, d_blob);
  if (rc) return rc;
  if (shape != 27 && shape != 7 && shape != 19) return VBM_ERR_ARG;
  if (flags & ~(VBM_CACHED | VBM_STREAMING)) return VBM_ERR_ARG;
  if (grid->n_blocks == 0) return VBM_OK;
  if (!d_taps) return VBM_ERR_ARG;
  if ((rc = check_kernel_memory({d_blob, d_taps}))) return rc;
  const DeviceGrid g = device_grid(grid, d_blob);
  const dim3 gd(g.n_blocks), bd(1u << g.log2w);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool cached = flags & VBM_CACHED, stream_taps = flags & VBM_STREAMING;
  if (shape == 27) {
    const uint32_t cap = brick_capacity(g.log2w);
    if (cached && stream_taps)
      hipLaunchKernelGGL((k_taps_box_cached<true>), gd, bd, brick_lds_bytes(cap), st, g, d_taps, cap);
    else if (cached)
      hipLaunchKernelGGL((k_taps_box_cached<false>), gd, bd, brick_lds_bytes(cap), st, g, d_taps, cap);
    else if (stream_taps) hipLaunchKernelGGL((k_taps<BoxShape, false, true>), gd, bd, 0, st, g, d_taps);
    else hipLaunchKernelGGL((k_taps<BoxShape, false, false>), gd, bd, 0, st, g, d_taps);
  } else if (shape == 7) {
    if (cached && stream_taps) hipLaunchKernelGGL((k_taps<CrossShape, true, true>), gd, bd, 0, st, g, d_taps);
    else if (cached) hipLaunchKernelGGL((k_taps<CrossShape, true, false>), gd, bd, 0, st, g, d_taps);
    else if (stream_taps) hipLaunchKernelGGL((k_taps<CrossShape, false, true>), gd, bd, 0, st, g, d_taps);
    else hipLaunchKernelGGL((k_taps<CrossShape, false, false>), gd, bd, 0, st, g, d_taps);
  } else {
    if (cached && stream_taps) hipLaunchKernelGGL((k_taps<AxisShape, true, true>), gd, bd, 0, st, g, d_taps);
    else if (cached) hipLaunchKernelGGL((k_taps<AxisShape, true, false>), gd, bd, 0, st, g, d_taps);
    else if (stream_taps) hipLaunchKernelGGL((k_taps<AxisShape, false, true>), gd, bd, 0, st, g, d_taps);
    else hipLaunchKernelGGL((k_taps<AxisShape, false, false>), gd, bd, 0, st, g, d_taps);
  }
  return launch_status();
}

extern "C" int vbm_box_filter(const vbm_grid* grid, const void* d_blob, const float* d_sidecar, float* d_out, int C,
                              int flags, void* stream) {
  int rc = check_grid(grid, d_blob);
  if (rc) return rc;
  rc = check_float_buffers(grid, d_sidecar, d_out, C);
  if (rc) return rc;
  if (flags & ~(VBM_CACHED | VBM_STREAMING | VBM_WIDE_ROWS)) return VBM_ERR_ARG;
  if ((rc = check_kernel_memory({d_blob, d_sidecar, d_out}))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (grid->n_blocks == 0) {
    hipLaunchKernelGGL(k_zero_index_row, dim3(1), dim3(64), 0, st, d_out, uint32_t(C));
    return launch_status();
  }
  const DeviceGrid g = device_grid(grid, d_blob);
  const bool cached = flags & VBM_CACHED, streaming = flags & VBM_STREAMING;
  if (wide_rows(grid, C, flags)) {
    if (cached && streaming) launch_channels_wide<BoxLauncher<true, true, true>>(g, d_sidecar, d_out, C, st);
    else if (cached) launch_channels_wide<BoxLauncher<true, false, true>>(g, d_sidecar, d_out, C, st);
    else if (streaming) launch_channels_wide<BoxLauncher<false, true, true>>(g, d_sidecar, d_out, C, st);
    else launch_channels_wide<BoxLauncher<false, false, true>>(g, d_sidecar, d_out, C, st);
  } else {
    if (cached && streaming) launch_channels<BoxLauncher<true, true>>(g, d_sidecar, d_out, C, st);
    else if (cached) launch_channels<BoxLauncher<true, false>>(g, d_sidecar, d_out, C, st);
    else if (streaming) launch_channels<BoxLauncher<false, true>>(g, d_sidecar, d_out, C, st);
    else launch_channels<BoxLauncher<false, false>>(g, d_sidecar, d_out, C, st);
  }
  return launch_status();
}

// The 7-direction filters (cross, 19-tap axis): flags pick the resolver and
// the delivery; LAP only for the cross.
template <class S, bool LAP>
void launch_stencil(const DeviceGrid& g, const float* sc, float* out, int C, bool cached, bool streaming, bool wide,
                    hipStream_t st) {
  if (wide) {
    if (cached && streaming) launch_channels_wide<StencilLauncher<S, true, LAP, true, true>>(g, sc, out, C, st);
    else if (cached) launch_channels_wide<StencilLauncher<S, true, LAP, false, true>>(g, sc, out, C, st);
    else if (streaming) launch_channels_wide<StencilLauncher<S, false, LAP, true, true>>(g, sc, out, C, st);
    else launch_channels_wide<StencilLauncher<S, false, LAP, false, true>>(g, sc, out, C, st);
  } else {
    if (cached && streaming) launch_channels<StencilLauncher<S, true, LAP, true>>(g, sc, out, C, st);
    else if (cached) launch_channels<StencilLauncher<S, true, LAP, false>>(g, sc, out, C, st);
    else if (streaming) launch_channels<StencilLauncher<S, false, LAP, true>>(g, sc, out, C, st);
    else launch_channels<StencilLauncher<S, false, LAP, false>>(g, sc, out, C, st);
  }
}

extern "C" int vbm_cross_filter(const vbm_grid* grid, const void* d_blob, const float* d_sidecar, float* d_out, int C,
                                int flags, void* stream) {
  int rc = check_grid(grid, d_blob);
  if (rc) return rc;
  rc = check_float_buffers(grid, d_sidecar, d_out, C);
  if (rc) return rc;
  if (flags & ~(VBM_CACHED | VBM_STREAMING | VBM_OP_LAPLACIAN | VBM_WIDE_ROWS)) return VBM_ERR_ARG;
  if ((rc = check_kernel_memory({d_blob, d_sidecar, d_out}))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (grid->n_blocks == 0) {
    hipLaunchKernelGGL(k_zero_index_row, dim3(1), dim3(64), 0, st, d_out, uint32_t(C));
    return launch_status();
  }
  const DeviceGrid g = device_grid(grid, d_blob);
  const bool cached = flags & VBM_CACHED, streaming = flags & VBM_STREAMING;
  const bool wide = wide_rows(grid, C, flags);
  if (flags & VBM_OP_LAPLACIAN) launch_stencil<CrossShape, true>(g, d_sidecar, d_out, C, cached, streaming, wide, st);
  else launch_stencil<CrossShape, false>(g, d_sidecar, d_out, C, cached, streaming, wide, st);
  return launch_status();
}

extern "C" int vbm_axis_filter(const vbm_grid* grid, const void* d_blob, const float* d_sidecar, float* d_out, int C,
                               int flags, void* stream) {
  int rc = check_grid(grid, d_blob);
  if (rc) return rc;
  rc = check_float_buffers(grid, d_sidecar, d_out, C);
  if (rc) return rc;
  if (flags & ~(VBM_CACHED | VBM_STREAMING | VBM_WIDE_ROWS)) return VBM_ERR_ARG;
  if ((rc = check_kernel_memory({d_blob, d_sidecar, d_out}))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (grid->n_blocks == 0) {
    hipLaunchKernelGGL(k_zero_index_row, dim3(1), dim3(64), 0, st, d_out, uint32_t(C));
    return launch_status();
  }
  const DeviceGrid g = device_grid(grid, d_blob);
  launch_stencil<AxisShape, false>(g, d_sidecar, d_out, C, flags & VBM_CACHED, flags & VBM_STREAMING,
                                   wide_rows(grid, C, flags), st);
  return launch_status();
}

extern "C" int vbm_weno_filter(const vbm_grid* grid, const void* d_blob, const float* d_sidecar, float* d_out, int C,
                               int flags, void* stream) {
  int rc = check_grid(grid, d_blob);
  if (rc) return rc;
  rc = check_float_buffers(grid, d_sidecar, d_out, C);
  if (rc) return rc;
  if (flags & ~(VBM_CACHED | VBM_STREAMING | VBM_WIDE_ROWS)) return VBM_ERR_ARG;
  if ((rc = check_kernel_memory({d_blob, d_sidecar, d_out}))) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (grid->n_blocks == 0) {
    hipLaunchKernelGGL(k_zero_index_row, dim3(1), dim3(64), 0, st, d_out, uint32_t(C));
    return launch_status();
  }
  const DeviceGrid g = device_grid(grid, d_blob);
  const bool wide = wide_rows(grid, C, flags);
  const uint32_t bytes = wide ? 0u : uint32_t((uint64_t(g.n_active) + 1) * uint64_t(C) * 4);
  const bool vec = ((reinterpret_cast<uintptr_t>(d_sidecar) | reinterpret_cast<uintptr_t>(d_out)) & 15) == 0 &&
                   C % 4 == 0;
  const bool cached = flags & VBM_CACHED, streaming = flags & VBM_STREAMING;
  const dim3 gd(g.n_blocks), bd(1u << g.log2w);
  const uint32_t uc = uint32_t(C);
#define VBM_WENO_LAUNCH(V, CA, ST)                                                                      \
  do {                                                                                                  \
    if (wide) hipLaunchKernelGGL((k_weno<V, CA, ST, WideSidecar>), gd, bd, 0, st, g, d_sidecar, bytes, d_out, uc); \
    else hipLaunchKernelGGL((k_weno<V, CA, ST>), gd, bd, 0, st, g, d_sidecar, bytes, d_out, uc);      \
  } while (0)
  if (vec) {
    if (cached && streaming) VBM_WENO_LAUNCH(true, true, true);
    else if (cached) VBM_WENO_LAUNCH(true, true, false);
    else if (streaming) VBM_WENO_LAUNCH(true, false, true);
    else VBM_WENO_LAUNCH(true, false, false);
  } else {
    if (cached && streaming) VBM_WENO_LAUNCH(false, true, true);
    else if (cached) VBM_WENO_LAUNCH(false, true, false);
    else if (streaming) VBM_WENO_LAUNCH(false, false, true);
    else VBM_WENO_LAUNCH(false, false, false);
  }
#undef VBM_WENO_LAUNCH
  return launch_status();
}

extern "C" int vbm_build_metadata(const vbm_grid* grid, void* d_blob, uint64_t* d_total, void* stream) {
  int rc = check_grid(grid, d_blob);
  if (rc) return rc;
  if (grid->n_leaves == 0) return VBM_OK;
  if ((rc = check_kernel_memory({d_blob}))) return rc;
  if (d_total && (rc = check_kernel_memory({d_total}))) return rc;
  uint8_t* base = static_cast<uint8_t*>(d_blob);
  MutableGrid m;
  m.leaves = reinterpret_cast<Leaf*>(base + grid->off_leaves);
  m.block_first_leaf = reinterpret_cast<uint32_t*>(base + grid->off_block_first_leaf);
  m.block_jump = reinterpret_cast<uint64_t*>(base + grid->off_block_jump);
  m.n_leaves = grid->n_leaves;
  m.n_blocks = grid->n_blocks;
  m.log2w = grid->log2_width;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint32_t groups = (m.n_leaves + 255) / 256;
  // the group sums live in the jumpMap words until they are cleared for the scatter
  // (a grid with every leaf non-empty always has room: N / 64 >= L / 64 words)
  if (uint64_t(groups) > uint64_t(m.n_blocks) << (m.log2w - 6)) return VBM_ERR_ARG;
  hipLaunchKernelGGL(k_meta_counts, dim3(groups), dim3(256), 0, st, m);
  hipLaunchKernelGGL(k_meta_scan, dim3(1), dim3(1024), 0, st, m, groups, d_total);
  hipLaunchKernelGGL(k_meta_first, dim3(groups), dim3(256), 0, st, m);
  if (m.n_blocks) {
    const uint64_t words = uint64_t(m.n_blocks) << (m.log2w - 6);
    const uint64_t wg = (words + 255) / 256;
    hipLaunchKernelGGL(k_meta_clear_jump, dim3(uint32_t(wg < 4096 ? wg : 4096)), dim3(256), 0, st, m);
    hipLaunchKernelGGL(k_meta_scatter, dim3(groups), dim3(256), 0, st, m, grid->n_active);
  }
  return launch_status();
}

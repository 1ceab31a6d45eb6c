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

#include "vbm.h"
#include "vbm_device.hpp"

using namespace vbm;

namespace {

// Row of zeros read by inactive taps (up to 16 channels per launch chunk).
__device__ __align__(64) float g_zero_row[16];

// ---------------------------------------------------------------------------
// row I/O: CH channels starting at p; VEC = 16-byte aligned float4 access
// ---------------------------------------------------------------------------
template <int CH, bool VEC>
__device__ __forceinline__ void add_row(float (&acc)[CH], const float* __restrict__ p) {
  if constexpr (VEC && CH % 4 == 0) {
#pragma unroll
    for (int q = 0; q < CH / 4; ++q) {
      const float4 v = reinterpret_cast<const float4*>(p)[q];
      acc[4 * q + 0] = acc[4 * q + 0] + v.x;
      acc[4 * q + 1] = acc[4 * q + 1] + v.y;
      acc[4 * q + 2] = acc[4 * q + 2] + v.z;
      acc[4 * q + 3] = acc[4 * q + 3] + v.w;
    }
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) acc[c] = acc[c] + p[c];
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

template <int CH>
__device__ __forceinline__ void zero_index_row(float* __restrict__ out, uint32_t ch0) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) out[ch0 + c] = 0.0f;
  }
}

__device__ __forceinline__ const float* tap_row(const float* __restrict__ sc, uint32_t idx, uint32_t C, uint32_t ch0) {
  return idx ? sc + uint64_t(idx) * C + ch0 : g_zero_row;
}

// ---------------------------------------------------------------------------
// kernels
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(512) k_decode(DeviceGrid g, uint32_t* __restrict__ leaf_index,
                                                uint16_t* __restrict__ voxel_offset) {
  const Slot s = decode_own_slot(g, blockIdx.x);
  const uint64_t row = (uint64_t(blockIdx.x) << g.log2w) + threadIdx.x;
  leaf_index[row] = s.leaf;
  voxel_offset[row] = uint16_t(s.offset);
}

// Raw taps of every slot.  SHAPE 27 (box) or 7 (cross).
template <int SHAPE, bool CACHED, bool STREAM>
__global__ void __launch_bounds__(512) k_taps(DeviceGrid g, uint64_t* __restrict__ taps) {
  __shared__ uint32_t table[CACHED ? kMaxCachedLeaves * SHAPE : 1];
  const uint32_t b = blockIdx.x;
  const Slot s = decode_own_slot(g, b);
  const bool valid = s.leaf != kSentinelLeaf;
  uint64_t* out = taps + ((uint64_t(b) << g.log2w) + threadIdx.x) * SHAPE;
  bool cached = false;
  uint32_t first = 0;
  if constexpr (CACHED) {
    first = g.block_first_leaf[b];
    const uint32_t span = block_span(g, b);  // block-uniform: the barrier below is uniform
    if (span <= kMaxCachedLeaves) {
      stage_neighbour_table<SHAPE>(g, first, span, table);
      cached = true;
    }
  }
  if (!valid) {
#pragma unroll
    for (int j = 0; j < SHAPE; ++j) out[j] = 0;
    return;
  }
  if constexpr (SHAPE == 27) {
    if constexpr (STREAM) {
      auto put = [&](int t, uint32_t idx) { out[t] = idx; };
      if (cached) for_each_box_cached(g, table, first, s, put);
      else for_each_box(g, s, put);
    } else {
      uint64_t st[kBoxTaps];
      if (cached) compute_box_cached(g, table, first, s, st);
      else compute_box(g, s, st);
#pragma unroll
      for (int t = 0; t < kBoxTaps; ++t) out[t] = st[t];
    }
  } else {
    uint64_t st[kCrossTaps];
    if (cached) compute_cross_cached(g, table, first, s, st);
    else compute_cross(g, s, st);
#pragma unroll
    for (int j = 0; j < kCrossTaps; ++j) out[j] = st[j];
  }
}

// 27-tap box filter over channels [ch0, ch0 + CH) of a C-channel sidecar.
template <int CH, bool VEC, bool CACHED, bool STREAM>
__global__ void __launch_bounds__(512) k_box(DeviceGrid g, const float* __restrict__ sc, float* __restrict__ out,
                                             uint32_t C, uint32_t ch0) {
  __shared__ uint32_t table[CACHED ? kMaxCachedLeaves * kBoxTaps : 1];
  const uint32_t b = blockIdx.x;
  zero_index_row<CH>(out, ch0);
  const Slot s = decode_own_slot(g, b);
  const bool valid = s.leaf != kSentinelLeaf;
  bool cached = false;
  uint32_t first = 0;
  if constexpr (CACHED) {
    first = g.block_first_leaf[b];
    const uint32_t span = block_span(g, b);
    if (span <= kMaxCachedLeaves) {
      stage_neighbour_table<kBoxTaps>(g, first, span, table);
      cached = true;
    }
  }
  if (!valid) return;
  float acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = 0.0f;
  auto gather = [&](int, uint32_t idx) { add_row<CH, VEC>(acc, tap_row(sc, idx, C, ch0)); };
  if constexpr (STREAM) {
    if (cached) for_each_box_cached(g, table, first, s, gather);
    else for_each_box(g, s, gather);
  } else {
    uint64_t st[kBoxTaps];
    if (cached) compute_box_cached(g, table, first, s, st);
    else compute_box(g, s, st);
#pragma unroll
    for (int t = 0; t < kBoxTaps; ++t) gather(t, uint32_t(st[t]));
  }
  const uint64_t idx = 1 + (uint64_t(b) << g.log2w) + threadIdx.x;
  store_row<CH, VEC>(out + idx * C + ch0, acc);
}

// 7-tap cross filter: sum, or 7-point Laplacian (faces in cross order) - fl(6 c).
template <int CH, bool VEC, bool CACHED, bool LAP>
__global__ void __launch_bounds__(512) k_cross(DeviceGrid g, const float* __restrict__ sc, float* __restrict__ out,
                                               uint32_t C, uint32_t ch0) {
  __shared__ uint32_t table[CACHED ? kMaxCachedLeaves * kCrossTaps : 1];
  const uint32_t b = blockIdx.x;
  zero_index_row<CH>(out, ch0);
  const Slot s = decode_own_slot(g, b);
  const bool valid = s.leaf != kSentinelLeaf;
  bool cached = false;
  uint32_t first = 0;
  if constexpr (CACHED) {
    first = g.block_first_leaf[b];
    const uint32_t span = block_span(g, b);
    if (span <= kMaxCachedLeaves) {
      stage_neighbour_table<kCrossTaps>(g, first, span, table);
      cached = true;
    }
  }
  if (!valid) return;
  uint64_t st[kCrossTaps];
  if (cached) compute_cross_cached(g, table, first, s, st);
  else compute_cross(g, s, st);
  float acc[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) acc[c] = 0.0f;
#pragma unroll
  for (int j = 0; j < kCrossTaps; ++j) {
    if (LAP && j == 3) continue;  // the centre enters the Laplacian only as -6*centre
    add_row<CH, VEC>(acc, tap_row(sc, uint32_t(st[j]), C, ch0));
  }
  const uint64_t idx = 1 + (uint64_t(b) << g.log2w) + threadIdx.x;
  if constexpr (LAP) {
    float centre[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) centre[c] = 0.0f;
    add_row<CH, VEC>(centre, sc + idx * C + ch0);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const float six_c = 6.0f * centre[c];
      acc[c] = acc[c] - six_c;
    }
  }
  store_row<CH, VEC>(out + idx * C + ch0, acc);
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

DeviceGrid device_grid(const vbm_grid* grid, const void* d_blob) {
  const uint8_t* base = static_cast<const uint8_t*>(d_blob);
  DeviceGrid g;
  g.leaves = reinterpret_cast<const Leaf*>(base + grid->off_leaves);
  g.root = reinterpret_cast<const RootTile*>(base + grid->off_root);
  g.upper = reinterpret_cast<const uint32_t*>(base + grid->off_upper);
  g.lower = reinterpret_cast<const uint32_t*>(base + grid->off_lower);
  g.block_first_leaf = reinterpret_cast<const uint32_t*>(base + grid->off_block_first_leaf);
  g.block_jump = reinterpret_cast<const uint64_t*>(base + grid->off_block_jump);
  g.n_active = uint32_t(grid->n_active);
  g.n_root = grid->n_root;
  g.n_blocks = grid->n_blocks;
  g.log2w = grid->log2_width;
  return g;
}

int launch_status() { return hipGetLastError() == hipSuccess ? VBM_OK : VBM_ERR_HIP; }

int check_float_buffers(const vbm_grid* grid, const float* sc, const float* out, int C) {
  if (!sc || !out || C < 1) return VBM_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(sc) | reinterpret_cast<uintptr_t>(out)) & 3) return VBM_ERR_ALIGN;
  const uint64_t bytes = (grid->n_active + 1) * uint64_t(C) * 4;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(sc), b0 = reinterpret_cast<uintptr_t>(out);
  if (a0 < b0 + bytes && b0 < a0 + bytes) return VBM_ERR_ALIAS;
  return VBM_OK;
}

template <bool CACHED, bool STREAM>
struct BoxLauncher {
  template <int CH, bool VEC>
  static void go(const DeviceGrid& g, const float* sc, float* out, uint32_t C, uint32_t ch0, hipStream_t st) {
    hipLaunchKernelGGL((k_box<CH, VEC, CACHED, STREAM>), dim3(g.n_blocks), dim3(1u << g.log2w), 0, st, g, sc, out,
                       C, ch0);
  }
};

template <bool CACHED, bool LAP>
struct CrossLauncher {
  template <int CH, bool VEC>
  static void go(const DeviceGrid& g, const float* sc, float* out, uint32_t C, uint32_t ch0, hipStream_t st) {
    hipLaunchKernelGGL((k_cross<CH, VEC, CACHED, LAP>), dim3(g.n_blocks), dim3(1u << g.log2w), 0, st, g, sc, out,
                       C, ch0);
  }
};

// Channel chunks of one launch: exact kernels for C in {1,2,3,4,8,16}, other
// C as a sequence of 16/8/4/2/1-channel chunks.  float4 access when C is a
// multiple of 4 and both buffers are 16-byte aligned.
template <class L>
void launch_channels(const DeviceGrid& g, const float* sc, float* out, int C, hipStream_t st) {
  const bool vec = ((reinterpret_cast<uintptr_t>(sc) | reinterpret_cast<uintptr_t>(out)) & 15) == 0 && C % 4 == 0;
  const uint32_t uc = uint32_t(C);
  switch (C) {
    case 1: L::template go<1, false>(g, sc, out, uc, 0, st); return;
    case 2: L::template go<2, false>(g, sc, out, uc, 0, st); return;
    case 3: L::template go<3, false>(g, sc, out, uc, 0, st); return;
    default: break;
  }
  uint32_t ch0 = 0;
  while (ch0 < uc) {
    const uint32_t left = uc - ch0;
    if (left >= 16) {
      if (vec) L::template go<16, true>(g, sc, out, uc, ch0, st);
      else L::template go<16, false>(g, sc, out, uc, ch0, st);
      ch0 += 16;
    } else if (left >= 8) {
      if (vec) L::template go<8, true>(g, sc, out, uc, ch0, st);
      else L::template go<8, false>(g, sc, out, uc, ch0, st);
      ch0 += 8;
    } else if (left >= 4) {
      if (vec) L::template go<4, true>(g, sc, out, uc, ch0, st);
      else L::template go<4, false>(g, sc, out, uc, ch0, st);
      ch0 += 4;
    } else if (left >= 2) {
      L::template go<2, false>(g, sc, out, uc, ch0, st);
      ch0 += 2;
    } else {
      L::template go<1, false>(g, sc, out, uc, ch0, st);
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
  const DeviceGrid g = device_grid(grid, d_blob);
  hipLaunchKernelGGL(k_decode, dim3(g.n_blocks), dim3(1u << g.log2w), 0, static_cast<hipStream_t>(stream), g,
                     d_leaf_index, d_voxel_offset);
  return launch_status();
}

extern "C" int vbm_stencil_indices(const vbm_grid* grid, const void* d_blob, int shape, int flags, uint64_t* d_taps,
                                   void* stream) {
  int rc = check_grid(grid, d_blob);
  if (rc) return rc;
  if (shape != 27 && shape != 7) return VBM_ERR_ARG;
  if (flags & ~(VBM_CACHED | VBM_STREAMING)) return VBM_ERR_ARG;
  if (shape == 7 && (flags & VBM_STREAMING)) return VBM_ERR_UNSUPPORTED;
  if (grid->n_blocks == 0) return VBM_OK;
  if (!d_taps) return VBM_ERR_ARG;
  const DeviceGrid g = device_grid(grid, d_blob);
  const dim3 gd(g.n_blocks), bd(1u << g.log2w);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const bool cached = flags & VBM_CACHED, stream_taps = flags & VBM_STREAMING;
  if (shape == 27) {
    if (cached && stream_taps) hipLaunchKernelGGL((k_taps<27, true, true>), gd, bd, 0, st, g, d_taps);
    else if (cached) hipLaunchKernelGGL((k_taps<27, true, false>), gd, bd, 0, st, g, d_taps);
    else if (stream_taps) hipLaunchKernelGGL((k_taps<27, false, true>), gd, bd, 0, st, g, d_taps);
    else hipLaunchKernelGGL((k_taps<27, false, false>), gd, bd, 0, st, g, d_taps);
  } else {
    if (cached) hipLaunchKernelGGL((k_taps<7, true, false>), gd, bd, 0, st, g, d_taps);
    else hipLaunchKernelGGL((k_taps<7, false, false>), gd, bd, 0, st, g, d_taps);
  }
  return launch_status();
}

extern "C" int vbm_box_filter(const vbm_grid* grid, const void* d_blob, const float* d_sidecar, float* d_out, int C,
                              int flags, void* stream) {
  int rc = check_grid(grid, d_blob);
  if (rc) return rc;
  rc = check_float_buffers(grid, d_sidecar, d_out, C);
  if (rc) return rc;
  if (flags & ~(VBM_CACHED | VBM_STREAMING)) return VBM_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (grid->n_blocks == 0) {
    hipLaunchKernelGGL(k_zero_index_row, dim3(1), dim3(64), 0, st, d_out, uint32_t(C));
    return launch_status();
  }
  const DeviceGrid g = device_grid(grid, d_blob);
  const bool cached = flags & VBM_CACHED, streaming = flags & VBM_STREAMING;
  if (cached && streaming) launch_channels<BoxLauncher<true, true>>(g, d_sidecar, d_out, C, st);
  else if (cached) launch_channels<BoxLauncher<true, false>>(g, d_sidecar, d_out, C, st);
  else if (streaming) launch_channels<BoxLauncher<false, true>>(g, d_sidecar, d_out, C, st);
  else launch_channels<BoxLauncher<false, false>>(g, d_sidecar, d_out, C, st);
  return launch_status();
}

extern "C" int vbm_cross_filter(const vbm_grid* grid, const void* d_blob, const float* d_sidecar, float* d_out, int C,
                                int flags, void* stream) {
  int rc = check_grid(grid, d_blob);
  if (rc) return rc;
  rc = check_float_buffers(grid, d_sidecar, d_out, C);
  if (rc) return rc;
  if (flags & VBM_STREAMING) return VBM_ERR_UNSUPPORTED;
  if (flags & ~(VBM_CACHED | VBM_OP_LAPLACIAN)) return VBM_ERR_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (grid->n_blocks == 0) {
    hipLaunchKernelGGL(k_zero_index_row, dim3(1), dim3(64), 0, st, d_out, uint32_t(C));
    return launch_status();
  }
  const DeviceGrid g = device_grid(grid, d_blob);
  const bool cached = flags & VBM_CACHED, lap = flags & VBM_OP_LAPLACIAN;
  if (cached && lap) launch_channels<CrossLauncher<true, true>>(g, d_sidecar, d_out, C, st);
  else if (cached) launch_channels<CrossLauncher<true, false>>(g, d_sidecar, d_out, C, st);
  else if (lap) launch_channels<CrossLauncher<false, true>>(g, d_sidecar, d_out, C, st);
  else launch_channels<CrossLauncher<false, false>>(g, d_sidecar, d_out, C, st);
  return launch_status();
}

// A consumer written on the library's device header alone (vbm.h +
// vbm_device.hpp), the way the pages' streaming callback is meant to be used:
// each work-item decodes its slot, the block stages its neighbour-leaf table
// once (Cached) or not at all (tree walks), and the 27 box taps are streamed
// to a lambda that keeps, per voxel, the number of active neighbours and the
// largest channel-0 value among them.  Test code: built into its own library
// (libvbm_example.so) and checked by tests/test_gpu_custom_consumer.py.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "vbm.h"
#include "vbm_device.hpp"

namespace {

template <bool CACHED>
__global__ void __launch_bounds__(512) k_neighbour_stats(vbm::DeviceGrid g, const float* __restrict__ sc, uint32_t C,
                                                         float* __restrict__ largest, uint32_t* __restrict__ count) {
  __shared__ uint32_t table[vbm::kMaxCachedLeaves * 27];
  const uint32_t b = blockIdx.x;
  const vbm::Slot s = vbm::decode_own_slot(g, b);
  const uint32_t first = g.block_first_leaf[b];
  const uint32_t span = vbm::block_span(g, b);
  const bool cached = CACHED && span <= uint32_t(vbm::kMaxCachedLeaves);  // the same in the whole block
  if (cached) vbm::stage_neighbour_table<27>(g, first, span, table);    // every work-item, one barrier
  if (s.leaf == vbm::kSentinelLeaf) return;
  uint32_t n = 0;
  float m = -INFINITY;
  auto visit = [&](int /*tap*/, uint32_t index) {
    if (index) {
      ++n;
      m = fmaxf(m, sc[uint64_t(index) * C]);
    }
  };
  if (cached) vbm::for_each_box_cached(g, table, first, s, visit);
  else vbm::for_each_box(g, s, visit);
  const uint64_t slot = (uint64_t(b) << g.log2w) + threadIdx.x;
  largest[slot] = m;
  count[slot] = n;
}

}  // namespace

// largest, count: device [n_blocks * W], slot b*W + s; sentinel slots untouched.
extern "C" int vbm_example_neighbour_stats(const vbm_grid* grid, const void* d_blob, const float* d_sidecar, int C,
                                           float* d_largest, uint32_t* d_count, int cached) {
  if (!grid || !d_blob || !d_sidecar || !d_largest || !d_count || C < 1) return VBM_ERR_ARG;
  if (grid->n_blocks == 0) return VBM_OK;
  const vbm::DeviceGrid g = vbm::device_grid_of(*grid, d_blob);
  const dim3 gd(grid->n_blocks), bd(1u << grid->log2_width);
  if (cached) hipLaunchKernelGGL(k_neighbour_stats<true>, gd, bd, 0, 0, g, d_sidecar, uint32_t(C), d_largest, d_count);
  else hipLaunchKernelGGL(k_neighbour_stats<false>, gd, bd, 0, 0, g, d_sidecar, uint32_t(C), d_largest, d_count);
  return hipGetLastError() == hipSuccess ? VBM_OK : VBM_ERR_HIP;
}

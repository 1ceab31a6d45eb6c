// GPU check of the WENO kernels' shortcut divisions (vbm_division.hpp, the
// same device functions the kernels call) against the IEEE quotient, which
// this file computes with plain correctly rounded division.  Test code: built
// into its own library (libvbm_divcheck.so) and called by
// tests/test_gpu_division_check.py.  Each work-item writes its own mismatch
// counts (plain vector stores, no atomics).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vbm_division.hpp"

namespace {

__device__ __forceinline__ uint32_t bits_of(float x) { return __builtin_bit_cast(uint32_t, x); }

// y over the bit patterns [lo, lo + count): recip(y) against 1 / y, and
// div_by_recip(n, y, recip(y)) against n / y for n = 6 and 3.
__global__ void k_check_recip(uint32_t lo, uint64_t count, uint32_t* __restrict__ counts) {
  const uint64_t tid = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
  uint32_t bad1 = 0, bad6 = 0, bad3 = 0;
  for (uint64_t i = tid; i < count; i += stride) {
    const float y = __builtin_bit_cast(float, uint32_t(lo + i));
    const float r = vbm_div::recip(y);
    bad1 += bits_of(r) != bits_of(1.0f / y);
    bad6 += bits_of(vbm_div::div_by_recip(6.0f, y, r)) != bits_of(6.0f / y);
    bad3 += bits_of(vbm_div::div_by_recip(3.0f, y, r)) != bits_of(3.0f / y);
  }
  counts[3 * tid + 0] = bad1;
  counts[3 * tid + 1] = bad6;
  counts[3 * tid + 2] = bad3;
}

// x over the bit patterns [lo, lo + count) and their negatives:
// div_const(x, 6, 1/6) and div_const(x, 12, 1/12) against x / 6 and x / 12.
__global__ void k_check_const(uint32_t lo, uint64_t count, uint32_t* __restrict__ counts) {
  const uint64_t tid = uint64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const uint64_t stride = uint64_t(gridDim.x) * blockDim.x;
  uint32_t bad6 = 0, bad12 = 0;
  for (uint64_t i = tid; i < count; i += stride) {
    const float p = __builtin_bit_cast(float, uint32_t(lo + i));
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float x = s ? -p : p;
      bad6 += bits_of(vbm_div::div_const(x, 6.0f, 1.0f / 6.0f)) != bits_of(x / 6.0f);
      bad12 += bits_of(vbm_div::div_const(x, 12.0f, 1.0f / 12.0f)) != bits_of(x / 12.0f);
    }
  }
  counts[2 * tid + 0] = bad6;
  counts[2 * tid + 1] = bad12;
}

}  // namespace

// counts: device u32 [blocks * threads * 3] (recip) or [blocks * threads * 2] (const).
extern "C" int vbm_divcheck_recip(uint32_t lo, uint64_t count, uint32_t* counts, uint32_t blocks, uint32_t threads) {
  hipLaunchKernelGGL(k_check_recip, dim3(blocks), dim3(threads), 0, 0, lo, count, counts);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

extern "C" int vbm_divcheck_const(uint32_t lo, uint64_t count, uint32_t* counts, uint32_t blocks, uint32_t threads) {
  hipLaunchKernelGGL(k_check_const, dim3(blocks), dim3(threads), 0, 0, lo, count, counts);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

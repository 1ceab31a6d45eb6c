// Shortcut fp32 divisions of the WENO kernels, each equal to the IEEE quotient
// (round to nearest even) on a stated range, outside of which the kernels use
// plain division.  Shared by the kernels and by the GPU check of the ranges
// (tests/division_check.hip).
#pragma once

#include <hip/hip_runtime.h>

namespace vbm_div {

// x / d for a constant d with rd = 1/d rounded: the product x * rd corrected by
// its remainder, which one fma computes exactly (Markstein's division step).
// For d = 6 and d = 12: the IEEE quotient for +0 and for every finite x of
// magnitude at least 2^-124 (checked over all fp32 x on the CPU and the GPU);
// -0 gives +0 (the remainder step adds +0 to the -0 product).
__device__ __forceinline__ float div_const(float x, float d, float rd) {
  const float q = x * rd;
  return __builtin_fmaf(__builtin_fmaf(-q, d, x), rd, q);
}

// 1 / y: the hardware reciprocal refined by one Newton step.  The IEEE
// quotient for every y in [2^-40, 2^126) (checked on the MI355X for all of
// them; near 2^126 and above the quotient is subnormal and it is not).
__device__ __forceinline__ float recip(float y) {
  const float r = __builtin_amdgcn_rcpf(y);
  return __builtin_fmaf(__builtin_fmaf(-y, r, 1.0f), r, r);
}

// n / y for n = 3 or 6 given r = recip(y): the product n * r corrected by its
// remainder.  The IEEE quotient for every y in [2^-40, 2^126) (same check).
__device__ __forceinline__ float div_by_recip(float n, float y, float r) {
  const float q = n * r;
  return __builtin_fmaf(__builtin_fmaf(-y, q, n), r, q);
}

}  // namespace vbm_div

// Host-side checks shared by the C-ABI entry points of the library.
#pragma once

#include <hip/hip_runtime.h>

#include <initializer_list>

#include "vbm.h"

namespace vbm_host {

inline int launch_status() { return hipGetLastError() == hipSuccess ? VBM_OK : VBM_ERR_HIP; }

// Every pointer a kernel dereferences must be memory the GPU can reach: device
// memory, pinned host memory or managed memory.  A pageable host pointer, or
// an address HIP does not know, would fault the GPU, so it is refused before
// any launch.
inline int check_kernel_memory(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs) {
    hipPointerAttribute_t a;
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
      (void)hipGetLastError();  // the failed query must not surface as a later launch error
      return VBM_ERR_ARG;
    }
    if (a.type != hipMemoryTypeDevice && a.type != hipMemoryTypeHost && a.type != hipMemoryTypeManaged)
      return VBM_ERR_ARG;
  }
  return VBM_OK;
}

}  // namespace vbm_host

// Host-side argument checks shared by the launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

inline int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    default: return 0;
  }
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int log2_exact(int32_t x) {
  if (x <= 0 || (x & (x - 1)) != 0) return -1;
  int l = 0;
  while ((1 << l) < x) ++l;
  return l;
}

// Shapes with a kernel instance: head_dim 64/128, block_size 8..128.
inline int check_shape(int32_t head_dim, int32_t block_size, int32_t dtype) {
  if (elem_bytes(dtype) == 0) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  const int lb = log2_exact(block_size);
  if (lb < 3 || lb > 7) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa

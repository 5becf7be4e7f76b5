// Status strings, version and debug status of the C ABI.
#include <hip/hip_runtime_api.h>

#include "internal.hpp"
#include "pa.h"

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID: return "PA_ERR_INVALID: invalid argument (null pointer, size or alignment)";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: no kernel for this dtype/head_dim/block_size";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP launch or runtime error";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS: the block pool has no free block";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: decode workspace missing or too small";
    case PA_ERR_NOT_FOUND: return "PA_ERR_NOT_FOUND: unknown sequence id";
    case PA_ERR_EXISTS: return "PA_ERR_EXISTS: sequence id already in use";
    case PA_ERR_CAPACITY: return "PA_ERR_CAPACITY: output buffer too small";
    default: return "unknown pa status";
  }
}

int pa_version(void) { return 100; }

int pa_debug_status(void* stream) {
  if (hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream)) != hipSuccess) return PA_ERR_HIP;
  const uint32_t w = pa::debug_take_decode() | pa::debug_take_prefill() | pa::debug_take_cache_ops();
  if (w == ~0u) return PA_ERR_HIP;  // a symbol copy failed
  return int(w & (PA_DEBUG_TABLE | PA_DEBUG_SLOT | PA_DEBUG_PAIR | PA_DEBUG_ITEM));
}

int pa_debug_enabled(void) {
#ifdef PA_DEBUG
  return 1;
#else
  return 0;
#endif
}

}  // extern "C"

// Library-internal entry points shared between translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace pa {

// One launch at the start of an engine step: copy `copy_bytes` (a multiple of
// 16) of staging from pinned host memory (device-visible address `host_src`)
// to `dev_dst`, and write the n new tokens' K/V into the pools with the slots
// read from the host staging `host_slots`.  Returns a pa_status.
int launch_step_prologue(const void* host_src, void* dev_dst, size_t copy_bytes,
                         const int64_t* host_slots, const void* k, const void* v, int64_t n,
                         void* k_cache, void* v_cache, int32_t num_heads, int32_t head_dim,
                         int32_t block_size, int32_t dtype, hipStream_t stream);

}  // namespace pa

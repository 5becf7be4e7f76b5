// Measurement kernel: a plain streaming read of a device buffer, the
// achievable-bandwidth reference for the decode's roofline.  Decode one token
// at a time is bound by HBM reads (brentwoodlivery "5.3.18 LLM serving", the
// intuition and the prefill/decode cards; ki.herwig.de, the vLLM paper's
// statement that the sequential generation phase is memory-bound), so the
// decode is compared with the fastest plain read this library can do.
//
// Each wave reads 8 KiB chunks (eight 1 KiB wave-wide 16-byte loads, all in
// flight, non-temporal), grid-stride over the buffer, and folds the words
// with XOR so the loads cannot be dropped; one atomic XOR per wave to a sink.
#include "launch_common.hpp"
#include "pa_device.hpp"

namespace pa {

constexpr int kReadLoads = 8;                                  // 1 KiB loads per chunk
constexpr int64_t kReadChunk = int64_t(kReadLoads) * kWave * 16;  // 8 KiB

__global__ __launch_bounds__(kWave) void stream_read_kernel(const u32x4* __restrict__ src,
                                                            int64_t nchunks,
                                                            uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x;
  uint32_t acc = 0;
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const u32x4* p = src + c * (kReadChunk / 16) + lane;
    u32x4 v[kReadLoads];
#pragma unroll
    for (int i = 0; i < kReadLoads; ++i) v[i] = __builtin_nontemporal_load(p + i * kWave);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kReadLoads; ++i) acc ^= v[i][0] ^ v[i][1] ^ v[i][2] ^ v[i][3];
  }
  if (acc != 0) atomicXor(sink, acc);
}

}  // namespace pa

extern "C" {

int pa_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t waves, void* stream) {
  if (bytes < 0 || waves < 0) return PA_ERR_INVALID;
  if (bytes == 0) return PA_OK;
  if (!src || !sink || !pa::aligned16(src)) return PA_ERR_INVALID;
  if (bytes % pa::kReadChunk != 0) return PA_ERR_INVALID;
  const int64_t nchunks = bytes / pa::kReadChunk;
  int64_t grid = waves > 0 ? waves : 256 * 16;
  if (grid > nchunks) grid = nchunks;
  (void)hipGetLastError();
  hipLaunchKernelGGL(pa::stream_read_kernel, dim3(unsigned(grid)), dim3(pa::kWave), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const pa::u32x4*>(src),
                     nchunks, sink);
  return pa::launch_status();
}

}  // extern "C"

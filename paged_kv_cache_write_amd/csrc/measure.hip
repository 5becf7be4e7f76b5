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
//
// A second kernel reads tiles gathered through a list from two arrays: the
// paged decode's own access pattern (each (block, head) tile of K and of V
// that a work unit covers) without its arithmetic, so the decode can also be
// compared with the fastest read of the same scattered tiles.
#include "launch_common.hpp"
#include "pa_device.hpp"
#include "xcd_order.hpp"

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

// One wave per unit of the list: unit u reads tiles ids[offsets[u] ..
// offsets[u + 1]) of a and of b, 1 KiB per wave-wide 16-byte load,
// non-temporal, in batches of kReadLoads loads of each array with the next
// batch issued before the current one is folded (16 KiB of each array in
// flight, as the decode keeps its next chunk in flight).  Units go to
// workgroups in the decode's XCD-aware order (xcd_order.hpp).  Tile ids
// outside [0, num_tiles) are skipped.  Every load is issued (past the end of
// the list, or for a skipped id, from an in-bounds tile already read, whose
// value is then dropped), so that the compiler's wait counts stay exact.
__global__ __launch_bounds__(kWave) void tile_read_kernel(
    const char* __restrict__ a, const char* __restrict__ b, int log2_tile, int64_t num_tiles,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ ids, int units,
    uint32_t* __restrict__ sink) {
  const int u = xcd_order_unit(int(blockIdx.x), 0);
  if (u >= units) return;
  const int lane = threadIdx.x;
  const int begin = offsets[u], end = offsets[u + 1];
  const int log2_loads = log2_tile - 10;  // 1 KiB loads per tile
  const int64_t total = int64_t(end - begin) << log2_loads;
  if (total <= 0 || num_tiles <= 0) return;
  // a batch: its tile ids first (scalar loads, one wait), then its loads
  auto issue = [&](int64_t i0, u32x4* va, u32x4* vb, bool* live) {
    int64_t kv[kReadLoads], raw[kReadLoads];
#pragma unroll
    for (int i = 0; i < kReadLoads; ++i) {
      kv[i] = min(i0 + i, total - 1);
      raw[i] = ids[begin + int(kv[i] >> log2_loads)];
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kReadLoads; ++i) {
      const bool ok = raw[i] >= 0 && raw[i] < num_tiles;
      live[i] = i0 + i < total && ok;
      const int64_t off = ((ok ? raw[i] : 0) << log2_tile) +
                          ((kv[i] & ((1 << log2_loads) - 1)) << 10) + lane * 16;
      va[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a + off));
      vb[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b + off));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  uint32_t acc = 0;
  auto fold = [&](const u32x4* va, const u32x4* vb, const bool* live) {
#pragma unroll
    for (int i = 0; i < kReadLoads; ++i) {
      const uint32_t w = va[i][0] ^ va[i][1] ^ va[i][2] ^ va[i][3] ^ vb[i][0] ^ vb[i][1] ^
                         vb[i][2] ^ vb[i][3];
      acc ^= live[i] ? w : 0u;
    }
  };
  u32x4 a0[kReadLoads], b0[kReadLoads], a1[kReadLoads], b1[kReadLoads];
  bool l0[kReadLoads], l1[kReadLoads];
  issue(0, a0, b0, l0);
  for (int64_t i0 = 0; i0 < total; i0 += 2 * kReadLoads) {
    issue(i0 + kReadLoads, a1, b1, l1);
    fold(a0, b0, l0);
    __builtin_amdgcn_sched_barrier(0);
    issue(i0 + 2 * kReadLoads, a0, b0, l0);
    fold(a1, b1, l1);
    __builtin_amdgcn_sched_barrier(0);
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

int pa_tile_read(const void* a, const void* b, int64_t tile_bytes, int64_t num_tiles,
                 const int32_t* offsets, const int32_t* ids, int32_t units, uint32_t* sink,
                 void* stream) {
  if (units < 0 || num_tiles < 0) return PA_ERR_INVALID;
  if (tile_bytes < 1024 || (tile_bytes & (tile_bytes - 1)) != 0 || tile_bytes > (int64_t(1) << 20))
    return PA_ERR_INVALID;
  if (units == 0) return PA_OK;
  if (!a || !b || !offsets || !ids || !sink || !pa::aligned16(a) || !pa::aligned16(b))
    return PA_ERR_INVALID;
  const int64_t wgs = pa::xcd_order_positions(units, 0);
  if (wgs > 0x7FFFFFFF) return PA_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  hipLaunchKernelGGL(pa::tile_read_kernel, dim3(unsigned(wgs)), dim3(pa::kWave), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const char*>(a),
                     static_cast<const char*>(b), pa::log2_exact(int32_t(tile_bytes)), num_tiles,
                     offsets, ids, units, sink);
  return pa::launch_status();
}

}  // extern "C"

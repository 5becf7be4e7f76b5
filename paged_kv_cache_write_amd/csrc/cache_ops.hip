// Slot-mapped KV-cache write and whole-block copy (copy-on-write) for gfx950.
//
// Cache write (polomodov.tech "vLLM and PagedAttention" slide 11: a new
// token's K/V go into the free slot of the sequence's last block): token n
// with slot s >= 0 is stored at [s / bs, h, s % bs, :] of both caches.
// Block copy (comfyai.app "6.4 PagedAttention" 6.4.3; slide 13: only the last
// block is copied when shared samples diverge): dst block = src block.
//
// Both are pure 16-byte moves: each lane carries one 16-byte slice of a
// token row (D elements), so a wave moves 1 KiB of contiguous source per
// instruction and writes whole 16-byte slices of contiguous destination rows.
#include <algorithm>

#include "internal.hpp"
#include "launch_common.hpp"
#include "pa_device.hpp"

namespace pa {

constexpr int kCwThreads = 256;

// One lane per 16-byte slice of a token's H rows: x covers the token's
// H * vecs_per_row slices (lane r: head r >> log2_vpr, slice r mod vpr), y
// strides over the tokens.  No division: vecs_per_row is a power of two.
__global__ __launch_bounds__(kCwThreads) void cache_write_kernel(
    const char* __restrict__ k, const char* __restrict__ v, const int64_t* __restrict__ slots,
    char* __restrict__ k_cache, char* __restrict__ v_cache, int64_t num_tokens, int H,
    int log2_vpr, int row_bytes, int log2_bs, int64_t num_slots) {
  const int per_token = H << log2_vpr;
  const int r = int(blockIdx.x) * kCwThreads + int(threadIdx.x);
  if (r >= per_token) return;
  const int h = r >> log2_vpr;
  const int col = r & ((1 << log2_vpr) - 1);
  for (int64_t n = blockIdx.y; n < num_tokens; n += gridDim.y) {
    // the slices are loaded while the slot is (both are in bounds whatever
    // the slot holds): one memory round trip, not two
    const int64_t src = (n * per_token + r) * 16;
    const u32x4 kx = *reinterpret_cast<const u32x4*>(k + src);
    const u32x4 vx = *reinterpret_cast<const u32x4*>(v + src);
    const int64_t slot = slots[n];
    if (slot < 0) continue;
    if (debug_bad(slot, num_slots, PA_DEBUG_SLOT)) continue;
    const int64_t blk = slot >> log2_bs;
    const int64_t off = slot & ((int64_t(1) << log2_bs) - 1);
    const int64_t dst = ((((blk * H + h) << log2_bs) + off) * row_bytes) + int64_t(col) * 16;
    *reinterpret_cast<u32x4*>(k_cache + dst) = kx;
    *reinterpret_cast<u32x4*>(v_cache + dst) = vx;
  }
}

// blockIdx.y = pair; blocks of blockIdx.x stride over the block's 16-byte
// vectors.  Source and destination pools may be the same (copy on write) or
// different (swapping between the device pool and a host pool).
__global__ __launch_bounds__(kCwThreads) void copy_blocks_kernel(
    const char* src_k, const char* src_v, char* dst_k, char* dst_v,
    const int32_t* __restrict__ pairs, int64_t tile_vecs, int64_t src_blocks, int64_t dst_blocks) {
  const int pair = blockIdx.y;
  const int64_t src = pairs[2 * pair], dst = pairs[2 * pair + 1];
  // both ends are checked (and flagged) before either is used
  if (int(debug_bad(src, src_blocks, PA_DEBUG_PAIR)) | int(debug_bad(dst, dst_blocks, PA_DEBUG_PAIR)))
    return;
  const u32x4* ks = reinterpret_cast<const u32x4*>(src_k) + src * tile_vecs;
  const u32x4* vs = reinterpret_cast<const u32x4*>(src_v) + src * tile_vecs;
  u32x4* kd = reinterpret_cast<u32x4*>(dst_k) + dst * tile_vecs;
  u32x4* vd = reinterpret_cast<u32x4*>(dst_v) + dst * tile_vecs;
  for (int64_t i = int64_t(blockIdx.x) * kCwThreads + threadIdx.x; i < tile_vecs;
       i += int64_t(gridDim.x) * kCwThreads) {
    const u32x4 a = ks[i];
    const u32x4 b = vs[i];
    kd[i] = a;
    vd[i] = b;
  }
}

// Engine step prologue.  Workgroups [0, copy_wgs) copy the staging bytes
// from pinned host memory (read over the host link) to device memory, each
// lane kPrologueVecs 16-byte vectors whose loads are all issued before the
// first store (one host round trip, not one per vector); each workgroup
// after them writes one new token: one lane reads the token's slot from host
// memory, the workgroup then moves the token's H rows of K and V.
constexpr int kPrologueVecs = 4;

__global__ __launch_bounds__(kCwThreads) void step_prologue_kernel(
    const u32x4* __restrict__ host_src, u32x4* __restrict__ dev_dst, int64_t copy_vecs,
    int copy_wgs, const int64_t* __restrict__ host_slots, const char* __restrict__ k,
    const char* __restrict__ v, char* __restrict__ k_cache, char* __restrict__ v_cache, int H,
    int vecs_per_row, int row_bytes, int log2_bs, int64_t num_slots) {
  if (int(blockIdx.x) < copy_wgs) {
    const int64_t i0 = int64_t(blockIdx.x) * kCwThreads * kPrologueVecs + threadIdx.x;
    u32x4 x[kPrologueVecs];
#pragma unroll
    for (int j = 0; j < kPrologueVecs; ++j)  // clamped: every lane loads, in bounds
      x[j] = host_src[min(i0 + int64_t(j) * kCwThreads, copy_vecs - 1)];
#pragma unroll
    for (int j = 0; j < kPrologueVecs; ++j)
      if (i0 + int64_t(j) * kCwThreads < copy_vecs) dev_dst[i0 + int64_t(j) * kCwThreads] = x[j];
    return;
  }
  // Every lane reads the slot (one host request per wave) while its K/V
  // loads from device memory are already in flight: the two round trips
  // overlap, and no barrier is needed.
  const int64_t n = int64_t(blockIdx.x) - copy_wgs;
  const int64_t slot = host_slots[n];
  const int total = H * vecs_per_row;
  for (int base = 0; base < total; base += kCwThreads * kPrologueVecs) {
    u32x4 kx[kPrologueVecs], vx[kPrologueVecs];
#pragma unroll
    for (int j = 0; j < kPrologueVecs; ++j) {  // clamped: every lane loads, in bounds
      const int i = min(base + j * kCwThreads + int(threadIdx.x), total - 1);
      const int64_t src = (n * total + i) * 16;
      kx[j] = *reinterpret_cast<const u32x4*>(k + src);
      vx[j] = *reinterpret_cast<const u32x4*>(v + src);
    }
    if (slot < 0) return;  // a padding token
    if (debug_bad(slot, num_slots, PA_DEBUG_SLOT)) return;
    const int64_t blk = slot >> log2_bs;
    const int64_t off = slot & ((int64_t(1) << log2_bs) - 1);
#pragma unroll
    for (int j = 0; j < kPrologueVecs; ++j) {
      const int i = base + j * kCwThreads + int(threadIdx.x);
      if (i >= total) break;
      const int h = i / vecs_per_row;
      const int col = i - h * vecs_per_row;
      const int64_t dst = ((((blk * H + h) << log2_bs) + off) * row_bytes) + int64_t(col) * 16;
      *reinterpret_cast<u32x4*>(k_cache + dst) = kx[j];
      *reinterpret_cast<u32x4*>(v_cache + dst) = vx[j];
    }
  }
}

int launch_step_prologue(const void* host_src, void* dev_dst, size_t copy_bytes,
                         const int64_t* host_slots, const void* k, const void* v, int64_t n,
                         void* k_cache, void* v_cache, int64_t num_blocks, int32_t num_heads,
                         int32_t head_dim, int32_t block_size, int32_t dtype,
                         hipStream_t stream) {
  int rc = check_shape(head_dim, block_size, dtype);
  if (rc != PA_OK) return rc;
  if (copy_bytes % 16 || !aligned16(host_src) || !aligned16(dev_dst) || n < 0 || n > 65535)
    return PA_ERR_INVALID;
  if (n > 0 && (!k || !v || !aligned16(k) || !aligned16(v) || !host_slots)) return PA_ERR_INVALID;
  const int64_t copy_vecs = int64_t(copy_bytes / 16);
  const int64_t per_wg = int64_t(kCwThreads) * kPrologueVecs;
  const int64_t copy_wgs64 = (copy_vecs + per_wg - 1) / per_wg;
  if (copy_wgs64 + n > INT32_MAX) return PA_ERR_UNSUPPORTED;
  const int copy_wgs = int(copy_wgs64);  // 0 when nothing is staged
  if (copy_wgs + n == 0) return PA_OK;
  const int row_bytes = head_dim * elem_bytes(dtype);
  (void)hipGetLastError();
  hipLaunchKernelGGL(step_prologue_kernel, dim3(unsigned(copy_wgs + n)), dim3(kCwThreads), 0,
                     stream, static_cast<const u32x4*>(host_src), static_cast<u32x4*>(dev_dst),
                     copy_vecs, copy_wgs, host_slots, static_cast<const char*>(k),
                     static_cast<const char*>(v), static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), num_heads, row_bytes / 16, row_bytes,
                     log2_exact(block_size), num_blocks * block_size);
  return launch_status();
}

}  // namespace pa

namespace pa {
uint32_t debug_take_cache_ops() { return debug_take_word(); }
}  // namespace pa

extern "C" {

int pa_cache_write(const void* k, const void* v, const int64_t* slot_mapping, int64_t num_tokens,
                   void* k_cache, void* v_cache, int64_t num_blocks, int32_t num_heads,
                   int32_t head_dim, int32_t block_size, int32_t dtype, void* stream) {
  int rc = pa::check_shape(head_dim, block_size, dtype);
  if (rc != PA_OK) return rc;
  if (num_tokens < 0 || num_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID;
  if (num_tokens == 0) return PA_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID;
  if (!pa::aligned16(k) || !pa::aligned16(v) || !pa::aligned16(k_cache) || !pa::aligned16(v_cache))
    return PA_ERR_INVALID;
  const int row_bytes = head_dim * pa::elem_bytes(dtype);
  const int log2_vpr = pa::log2_exact(row_bytes / 16);  // 8, 16 or 32 slices per row
  const int64_t per_token = int64_t(num_heads) << log2_vpr;
  if (per_token > INT32_MAX) return PA_ERR_UNSUPPORTED;
  const unsigned gx = unsigned((per_token + pa::kCwThreads - 1) / pa::kCwThreads);
  const unsigned gy = unsigned(std::min<int64_t>(num_tokens, 65535));
  (void)hipGetLastError();
  hipLaunchKernelGGL(pa::cache_write_kernel, dim3(gx, gy), dim3(pa::kCwThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const char*>(k),
                     static_cast<const char*>(v), slot_mapping, static_cast<char*>(k_cache),
                     static_cast<char*>(v_cache), num_tokens, num_heads, log2_vpr, row_bytes,
                     pa::log2_exact(block_size), num_blocks * block_size);
  return pa::launch_status();
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int32_t num_pairs,
                   int64_t num_blocks, int32_t num_heads, int32_t head_dim, int32_t block_size,
                   int32_t dtype, void* stream) {
  int rc = pa::check_shape(head_dim, block_size, dtype);
  if (rc != PA_OK) return rc;
  if (num_pairs < 0 || num_heads <= 0 || num_blocks <= 0) return PA_ERR_INVALID;
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > 65535) return PA_ERR_UNSUPPORTED;
  if (!k_cache || !v_cache || !block_pairs) return PA_ERR_INVALID;
  if (!pa::aligned16(k_cache) || !pa::aligned16(v_cache)) return PA_ERR_INVALID;
  const int64_t tile_vecs =
      int64_t(num_heads) * block_size * head_dim * pa::elem_bytes(dtype) / 16;
  int64_t gx = (tile_vecs + pa::kCwThreads - 1) / pa::kCwThreads;
  if (gx > 64) gx = 64;
  (void)hipGetLastError();
  hipLaunchKernelGGL(pa::copy_blocks_kernel, dim3(unsigned(gx), unsigned(num_pairs)),
                     dim3(pa::kCwThreads), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const char*>(k_cache), static_cast<const char*>(v_cache),
                     static_cast<char*>(k_cache), static_cast<char*>(v_cache), block_pairs,
                     tile_vecs, num_blocks, num_blocks);
  return pa::launch_status();
}

int pa_copy_blocks_between(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                           const int32_t* block_pairs, int32_t num_pairs, int64_t src_blocks,
                           int64_t dst_blocks, int32_t num_heads, int32_t head_dim,
                           int32_t block_size, int32_t dtype, void* stream) {
  int rc = pa::check_shape(head_dim, block_size, dtype);
  if (rc != PA_OK) return rc;
  if (num_pairs < 0 || num_heads <= 0 || src_blocks <= 0 || dst_blocks <= 0)
    return PA_ERR_INVALID;
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > 65535) return PA_ERR_UNSUPPORTED;
  if (!src_k || !src_v || !dst_k || !dst_v || !block_pairs) return PA_ERR_INVALID;
  if (!pa::aligned16(src_k) || !pa::aligned16(src_v) || !pa::aligned16(dst_k) ||
      !pa::aligned16(dst_v))
    return PA_ERR_INVALID;
  const int64_t tile_vecs =
      int64_t(num_heads) * block_size * head_dim * pa::elem_bytes(dtype) / 16;
  int64_t gx = (tile_vecs + pa::kCwThreads - 1) / pa::kCwThreads;
  if (gx > 64) gx = 64;
  (void)hipGetLastError();
  hipLaunchKernelGGL(pa::copy_blocks_kernel, dim3(unsigned(gx), unsigned(num_pairs)),
                     dim3(pa::kCwThreads), 0, reinterpret_cast<hipStream_t>(stream),
                     static_cast<const char*>(src_k), static_cast<const char*>(src_v),
                     static_cast<char*>(dst_k), static_cast<char*>(dst_v), block_pairs,
                     tile_vecs, src_blocks, dst_blocks);
  return pa::launch_status();
}

}  // extern "C"

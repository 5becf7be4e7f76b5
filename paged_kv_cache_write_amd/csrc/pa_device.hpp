// Device-side building blocks for gfx950 (CDNA4, wave64): storage types,
// 16-byte vector access, float32 dot products and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Reinterpret one 32-bit word.  The word is taken by value: applying
// __builtin_bit_cast directly to an ext_vector element (v[i], v.y) makes this
// clang read element 0 whatever the index, so element bits always pass
// through this function.
template <class To>
__device__ __forceinline__ To bits_as(uint32_t w) {
  return __builtin_bit_cast(To, w);
}
// The 32 bits of a float (a bit copy; bits_as<uint32_t>(x) would convert the value).
__device__ __forceinline__ uint32_t float_bits(float x) { return __builtin_bit_cast(uint32_t, x); }

// Storage types.  Every kernel moves data as 16-byte vectors (u32x4) and
// computes in float32.
struct F32 {
  using T = float;
  static constexpr int kVec = 4;  // elements per 16 bytes
};
struct F16 {
  using T = _Float16;
  static constexpr int kVec = 8;
};
struct BF16 {
  using T = uint16_t;  // raw bfloat16 bits
  static constexpr int kVec = 8;
};

// <a, b> over one 16-byte vector, accumulated onto c in float32.
__device__ __forceinline__ float dot16(F32, u32x4 a, u32x4 b, float c) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_fmaf(bits_as<float>(a[i]), bits_as<float>(b[i]), c);
  return c;
}
__device__ __forceinline__ float dot16(F16, u32x4 a, u32x4 b, float c) {
#pragma unroll
  for (int i = 0; i < 4; ++i)  // v_dot2_f32_f16: products exact, float32 sum
    c = __builtin_amdgcn_fdot2(bits_as<half2_t>(a[i]), bits_as<half2_t>(b[i]), c, false);
  return c;
}
__device__ __forceinline__ float dot16(BF16, u32x4 a, u32x4 b, float c) {
#pragma unroll
  for (int i = 0; i < 4; ++i)  // v_dot2_f32_bf16
    c = __builtin_amdgcn_fdot2_f32_bf16(bits_as<bf162_t>(a[i]), bits_as<bf162_t>(b[i]), c, false);
  return c;
}

// acc[e] = acc[e] * 1 + p * v[e] for the elements of one 16-byte vector.
__device__ __forceinline__ void axpy16(F32, float* acc, u32x4 v, float p) {
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(p, bits_as<float>(v[i]), acc[i]);
}
__device__ __forceinline__ void axpy16(F16, float* acc, u32x4 v, float p) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2_t h = bits_as<half2_t>(v[i]);
    acc[2 * i] = __builtin_fmaf(p, float(h.x), acc[2 * i]);  // v_fma_mix_f32
    acc[2 * i + 1] = __builtin_fmaf(p, float(h.y), acc[2 * i + 1]);
  }
}
__device__ __forceinline__ void axpy16(BF16, float* acc, u32x4 v, float p) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // a bfloat16 is the high half of a float32
    const uint32_t w = v[i];
    acc[2 * i] = __builtin_fmaf(p, bits_as<float>(w << 16), acc[2 * i]);
    acc[2 * i + 1] = __builtin_fmaf(p, bits_as<float>(w & 0xffff0000u), acc[2 * i + 1]);
  }
}

// float32 -> storage, round to nearest even.
__device__ __forceinline__ float to_store(F32, float x) { return x; }
__device__ __forceinline__ _Float16 to_store(F16, float x) { return (_Float16)x; }
__device__ __forceinline__ uint16_t to_store(BF16, float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// DPP row (16-lane) butterflies: every lane of a group of G lanes ends with
// the group's sum.  quad_perm [1,0,3,2] and [2,3,0,1] pair lanes within a
// quad; row_half_mirror pairs the two quads of 8 lanes; row_mirror pairs the
// two halves of a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

template <int G>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group size");
  x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (G >= 8) x += dpp_mov<0x141>(x);   // row_half_mirror
  if constexpr (G >= 16) x += dpp_mov<0x140>(x);  // row_mirror
  if constexpr (G >= 32)  // lanes 16 apart, within 32: ds_swizzle xor 0x10
    x += __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
  if constexpr (G >= 64) x += __shfl_xor(x, 32, 64);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Matrix cores, 16x16x32 with float32 accumulation (gfx950).  Lane l supplies
// row (l % 16) of A and column (l % 16) of B, each over k = 8 (l / 16) ..
// 8 (l / 16) + 7 (eight storage elements in one 16-byte vector), and receives
// D[4 (l / 16) + r][l % 16] in element r.
__device__ __forceinline__ f32x4 mma16x16x32(F16, u32x4 a, u32x4 b, f32x4 c) {
  typedef _Float16 v8 __attribute__((ext_vector_type(8)));
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8, a),
                                                __builtin_bit_cast(v8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16x16x32(BF16, u32x4 a, u32x4 b, f32x4 c) {
  typedef __bf16 v8 __attribute__((ext_vector_type(8)));
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8, a),
                                                 __builtin_bit_cast(v8, b), c, 0, 0, 0);
}

// Two float32 values as storage-type pairs hi + lo, packed two per word
// (first value in the low half): hi is x truncated to the storage type and lo
// the storage value of the exact remainder x - hi, so hi + lo equals x to
// about 2^-15 (bfloat16) or 2^-20 (float16) relative.
__device__ __forceinline__ void split_pair(F16, float x0, float x1, uint32_t& hi, uint32_t& lo) {
  typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));
  const fp16x2 h = __builtin_amdgcn_cvt_pkrtz(x0, x1);  // toward zero
  const float r0 = x0 - float(h.x), r1 = x1 - float(h.y);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(r0, r1));
}
__device__ __forceinline__ void split_pair(BF16, float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t b0 = __builtin_bit_cast(uint32_t, x0), b1 = __builtin_bit_cast(uint32_t, x1);
  const float r0 = x0 - bits_as<float>(b0 & 0xffff0000u);
  const float r1 = x1 - bits_as<float>(b1 & 0xffff0000u);
  hi = __builtin_amdgcn_perm(b1, b0, 0x07060302u);  // high halves of b0, b1
  lo = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, r1), __builtin_bit_cast(uint32_t, r0),
                             0x07060302u);
}

// Two float32 values rounded (nearest even) to the storage type, packed
// (one v_cvt_pk_f16_f32 / v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t round_pair(F16, float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), h2));
}
__device__ __forceinline__ uint32_t round_pair(BF16, float a, float b) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  typedef float f2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2{a, b}), b2));
}
__device__ __forceinline__ uint32_t pack_store(F16, float a, float b) {
  return round_pair(F16{}, a, b);
}
__device__ __forceinline__ uint32_t pack_store(BF16, float a, float b) {
  return round_pair(BF16{}, a, b);
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Debug builds (PA_DEBUG): a kernel checks every table entry, slot and copy
// pair before it becomes an address.  A value outside [0, n) sets `bit` in
// this translation unit's device error word (read and cleared by
// pa_debug_status) and is reported as invalid, so the caller substitutes an
// in-bounds block or skips the write.  Release builds check nothing.
#ifdef PA_DEBUG
static __device__ uint32_t pa_debug_word;
__device__ __forceinline__ bool debug_bad(int64_t v, int64_t n, uint32_t bit) {
  if (v >= 0 && v < n) return false;
  atomicOr(&pa_debug_word, bit);
  return true;
}
// Report `bit` (a check that does not guard an address).
__device__ __forceinline__ void debug_flag(uint32_t bit) { atomicOr(&pa_debug_word, bit); }
// The error word of this translation unit, then cleared (host; synchronous).
static inline uint32_t debug_take_word() {
  uint32_t w = 0, zero = 0;
  if (hipMemcpyFromSymbol(&w, HIP_SYMBOL(pa_debug_word), sizeof(w)) != hipSuccess) return ~0u;
  if (hipMemcpyToSymbol(HIP_SYMBOL(pa_debug_word), &zero, sizeof(zero)) != hipSuccess) return ~0u;
  return w;
}
#else
__device__ __forceinline__ bool debug_bad(int64_t, int64_t, uint32_t) { return false; }
__device__ __forceinline__ void debug_flag(uint32_t) {}
static inline uint32_t debug_take_word() { return 0; }
#endif

}  // namespace pa

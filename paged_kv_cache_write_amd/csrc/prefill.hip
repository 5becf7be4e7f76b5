// Paged prefill attention for gfx950: several new tokens per sequence attend
// causally over the paged cache (their own K/V already written into it).
//
// What is computed (brentwoodlivery "5.3.18 LLM serving", the prefill/decode
// cards: prefill processes a prompt's tokens together; polomodov.tech "vLLM
// and PagedAttention" slide 3; comfyai.app "6.4 PagedAttention" 6.4.3, the
// prefill writes the prompt's K/V into blocks): query i of sequence s sits at
// position p = context_lens[s] - q_len[s] + i and attends to the sequence's
// tokens 0..p, with token t at block_tables[s, t / bs], offset t % bs.
// Earlier tokens (a cached prefix or earlier chunks) and the new ones are
// read the same way.
//
// How (MI355X design): with 16 queries of one sequence against each key
// tile, q.K and P.V are dense products for the matrix cores.  One wave owns
// (sequence, head, 16 consecutive queries) and streams keys 0 .. last query's
// position in steps of 32 (two 16-token tiles):
//   S^T[t][q] = sum_d K[t][d] Q[q][d]        (v_mfma_f32_16x16x32, A = K rows)
//   O^T[d][q] += sum_t V^T[d][t] P^T[t][q]   (P^T is S^T's layout; the d axis
//                                             of this product is permuted so V
//                                             comes from plain row loads)
// with the online softmax per query column, the causal mask (key t > query
// position -> weight 0) on the steps that reach the tile's own positions, and
// P split into storage-type hi + lo parts so the weights keep float32-like
// precision.  Block ids come from wave-uniform (scalar) table loads, so
// contexts of any length stream without a table window; addresses past the
// last key are clamped to it (never an unwritten slot or a table entry past
// the sequence) and masked.
#include <type_traits>

#include "launch_common.hpp"
#include "pa_device.hpp"

namespace pa {

namespace {

constexpr float kPfLog2e = 1.4426950408889634f;
constexpr float kPfNegBig = -1.0e30f;  // running-max start: finite

struct PrefillParams {
  const void* q;       // [T, H, D] queries of all sequences, packed
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;  // [S, maxB]
  const int32_t* cu_q;          // [S + 1] query offsets
  const int32_t* context_lens;  // [S] tokens in the cache, the new ones included
  void* out;                    // [T, H, D]
  int H;
  int maxB;
  int log2_bs;
  float qk_scale;  // scale * log2(e)
};

template <class DT, int D>
__global__ __launch_bounds__(kWave, 2) void prefill_mfma_kernel(PrefillParams P) {
  using T = typename DT::T;
  constexpr int NK = D / 32;
  constexpr int NJ = D / 16;
  constexpr uint32_t kRowBytes = uint32_t(D) * sizeof(T);
  constexpr int kLog2Row = __builtin_ctz(kRowBytes);
  using VRow = typename std::conditional<NJ == 8, u32x4, u32x2>::type;
  static_assert(sizeof(T) == 2 && (NJ == 8 || NJ == 4), "16-bit storage, D 64 or 128");

  const int lane = threadIdx.x;
  const int qt = blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int H = P.H;
  const int q_begin = P.cu_q[s];
  const int q_len = P.cu_q[s + 1] - q_begin;
  const int q0 = qt * 16;
  if (q0 >= q_len) return;
  const int nq = min(16, q_len - q0);
  const int ctx = P.context_lens[s];
  const int pos0 = ctx - q_len + q0;  // position of the tile's first query
  const int kv_end = pos0 + nq;       // keys [0, kv_end)
  if (pos0 < 0) return;               // inconsistent lengths: nothing is read
  const int qi = lane & 15;
  const int g = lane >> 4;
  const bool has_q = qi < nq;
  const int my_pos = pos0 + qi;
  const size_t qrow = (size_t(q_begin + q0 + (has_q ? qi : 0)) * H + h);

  u32x4 qv[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j)
    qv[j] = has_q ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(P.q) +
                                                    qrow * kRowBytes + (32 * j + 8 * g) * sizeof(T))
                  : u32x4{0, 0, 0, 0};

  const int log2_bs = P.log2_bs;
  const int bs_mask = (1 << log2_bs) - 1;
  const int log2_tile = kLog2Row + log2_bs;
  const int32_t* trow = P.block_tables + size_t(s) * P.maxB;
  const char* kc = reinterpret_cast<const char*>(P.k_cache);
  const char* vc = reinterpret_cast<const char*>(P.v_cache);
  const int last = kv_end - 1;
  // Byte offset of token row tt + r (r < 16) of the sequence, clamped to the
  // last key; a 16-token tile spans at most two blocks.
  auto row_off = [&](int tt, int r) -> size_t {
    const int lo = __builtin_amdgcn_readfirstlane(min(tt, last) >> log2_bs);
    const int hi = __builtin_amdgcn_readfirstlane(min(tt + 15, last) >> log2_bs);
    const int b_lo = trow[lo];
    const int b_hi = trow[hi];
    const int t = min(tt + r, last);
    const int b = (t >> log2_bs) == lo ? b_lo : b_hi;
    return (size_t(uint32_t(b) * uint32_t(H) + uint32_t(h)) << log2_tile) +
           size_t(t & bs_mask) * kRowBytes;
  };

  float m = kPfNegBig, l = 0.f;
  f32x4 o[NJ];
#pragma unroll
  for (int jd = 0; jd < NJ; ++jd) o[jd] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float qk_scale = P.qk_scale;

  for (int base = 0; base < kv_end; base += 32) {
    u32x4 kr[2][NK];
    VRow vr[8];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int tt = base + 16 * a;
      const char* kp = kc + row_off(tt, qi) + 8 * g * sizeof(T);
#pragma unroll
      for (int j = 0; j < NK; ++j)
        kr[a][j] = *reinterpret_cast<const u32x4*>(kp + 32 * j * sizeof(T));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vr[4 * a + i] = *reinterpret_cast<const VRow*>(vc + row_off(tt, 4 * g + i) +
                                                       qi * NJ * sizeof(T));
    }
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sc[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      sc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NK; ++j) sc[a] = mma16x16x32(DT{}, kr[a][j], qv[j], sc[a]);
    }
    // x[e]: key base + 16 (e / 4) + 4 g + e % 4, query qi; keys after the
    // query's position (and past the last key) get weight 0
    float x[8];
    const bool masked = base + 32 > pos0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = base + 16 * (e >> 2) + 4 * g + (e & 3);
      x[e] = sc[e >> 2][e & 3] * qk_scale;
      if (masked && t > my_pos) x[e] = -__builtin_inff();
    }
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mn);
    m = mn;
    l *= alpha;
    u32x4 phi, plo;
#pragma unroll
    for (int p2 = 0; p2 < 4; ++p2) {
      const float p0 = fast_exp2(x[2 * p2] - mn), p1 = fast_exp2(x[2 * p2 + 1] - mn);
      l += p0 + p1;
      uint32_t hw, lw;
      split_pair(DT{}, p0, p1, hw, lw);
      phi[p2] = hw;
      plo[p2] = lw;
    }
#pragma unroll
    for (int jd = 0; jd < NJ; ++jd) o[jd] *= alpha;
#pragma unroll
    for (int jd = 0; jd < NJ; ++jd) {
      const uint32_t sel = (jd & 1) ? 0x07060302u : 0x05040100u;
      u32x4 va;
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2)
        va[p2] = __builtin_amdgcn_perm(uint32_t(vr[2 * p2 + 1][jd >> 1]),
                                       uint32_t(vr[2 * p2][jd >> 1]), sel);
      o[jd] = mma16x16x32(DT{}, va, phi, o[jd]);
      o[jd] = mma16x16x32(DT{}, va, plo, o[jd]);
    }
  }

  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);
  if (!has_q) return;
  const float inv = 1.0f / l;  // l >= 1: the running max key contributes 2^0
  T* out = reinterpret_cast<T*>(P.out) + qrow * D;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    VRow w;
#pragma unroll
    for (int p2 = 0; p2 < NJ / 2; ++p2)
      w[p2] = pack_store(DT{}, o[2 * p2][r] * inv, o[2 * p2 + 1][r] * inv);
    *reinterpret_cast<VRow*>(out + NJ * (4 * g + r)) = w;
  }
}

template <class DT, int D>
void launch_prefill(const PrefillParams& p, int S, int max_q_len, hipStream_t st) {
  const dim3 grid(unsigned((max_q_len + 15) / 16), unsigned(p.H), unsigned(S));
  hipLaunchKernelGGL((prefill_mfma_kernel<DT, D>), grid, dim3(kWave), 0, st, p);
}

}  // namespace

}  // namespace pa

extern "C" {

int pa_prefill(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* cu_q,
               const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
               int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
               int32_t max_q_len, int32_t dtype, void* out, void* stream) {
  int rc = pa::check_shape(head_dim, block_size, dtype);
  if (rc != PA_OK) return rc;
  if (dtype == PA_F32) return PA_ERR_UNSUPPORTED;  // the matrix-core path is 16-bit
  if (num_seqs < 0 || num_heads <= 0 || max_q_len < 0) return PA_ERR_INVALID;
  if (num_seqs > 65535 || num_heads > 65535) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || max_q_len == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !cu_q || !context_lens || !out)
    return PA_ERR_INVALID;
  if (max_blocks_per_seq <= 0 || num_blocks <= 0) return PA_ERR_INVALID;
  if (uint64_t(num_blocks) * uint64_t(num_heads) > 0xFFFFFFFFull) return PA_ERR_UNSUPPORTED;
  if (!pa::aligned16(q) || !pa::aligned16(k_cache) || !pa::aligned16(v_cache) ||
      !pa::aligned16(out))
    return PA_ERR_INVALID;
  pa::PrefillParams p;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.cu_q = cu_q;
  p.context_lens = context_lens;
  p.out = out;
  p.H = num_heads;
  p.maxB = max_blocks_per_seq;
  p.log2_bs = pa::log2_exact(block_size);
  p.qk_scale = scale * pa::kPfLog2e;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dtype == PA_F16) {
    if (head_dim == 64) pa::launch_prefill<pa::F16, 64>(p, num_seqs, max_q_len, st);
    else pa::launch_prefill<pa::F16, 128>(p, num_seqs, max_q_len, st);
  } else {
    if (head_dim == 64) pa::launch_prefill<pa::BF16, 64>(p, num_seqs, max_q_len, st);
    else pa::launch_prefill<pa::BF16, 128>(p, num_seqs, max_q_len, st);
  }
  return pa::launch_status();
}

}  // extern "C"

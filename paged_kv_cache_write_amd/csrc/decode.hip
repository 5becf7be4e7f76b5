// PagedAttention decode for gfx950: one query token per sequence attends over
// K/V stored in fixed-size blocks scattered across a shared pool.
//
// What is computed (polomodov.tech "vLLM and PagedAttention" slides 9-10;
// comfyai.app "6.4 PagedAttention" 6.4.1; brentwoodlivery "5.3.18", the
// card saying paging leaves the attention arithmetic unchanged): for each
// sequence s and head h, softmax(scale * q K^T) V over the sequence's first
// context_lens[s] tokens, where token t lives in physical block
// block_tables[s, t / bs] at offset t % bs.
//
// How (MI355X design, not taken from the pages):
//  * The context of each (sequence, head) is cut into partitions of
//    part_tokens tokens.  One wave (64 lanes) owns one (sequence, head,
//    partition) from start to end; a workgroup packs kWaves waves for
//    consecutive heads of the same (sequence, partition), which read the
//    same table entries.  Partitions give the 256 CUs enough independent
//    waves when there are few sequences or long contexts, and even out the
//    work when context lengths differ.
//  * A (block, head) tile is bs * D contiguous elements.  A lane owns a
//    16-byte slice of one token row, so one wave-wide load instruction reads
//    64 x 16 B = 1 KiB of consecutive bytes of one tile: fully coalesced.
//    Each lane consumes exactly the bytes it loaded, so K/V go from HBM
//    straight to registers; there is no LDS staging and no barrier.
//  * A wave works on chunks of U load instructions for K and U for V issued
//    back to back, so each lane has 2U 16-byte loads in flight.
//  * q.k partial dots use v_dot2_f32_{f16,bf16} (exact products, float32
//    sums); the lanes of one token row are summed with DPP butterflies; the
//    softmax is the online (running max / running sum) form in base 2 with
//    scale*log2(e) folded into the logit; P.V accumulates in float32
//    (v_fma_mix_f32 for fp16).
//  * The partition's table entries are loaded once per wave into one VGPR
//    (lane j = j-th block of the partition), in parallel with the context
//    length, and read with v_readlane, so a block's address is wave-uniform
//    scalar arithmetic.
//  * A wave merges (max, sum, accumulator) across its token rows with
//    shuffles.  A sequence with one partition stores its output row
//    directly.  Otherwise the partial (max, sum, normalised output) goes to
//    the workspace and the partitions are merged with the log-sum-exp rule:
//    by the last wave to finish that (sequence, head) (pa_decode, one launch,
//    an agent-scope counter per row), or by a second kernel
//    (pa_decode_partitions + pa_decode_reduce).
#include <algorithm>
#include <vector>

#include "launch_common.hpp"
#include "pa_device.hpp"

namespace pa {

#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 1
#endif
#ifndef PA_DECODE_UNROLL
#define PA_DECODE_UNROLL 8
#endif
constexpr int kWaves = PA_DECODE_WAVES;  // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so max - max never is NaN

struct DecodeParams {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* ws_ml;  // [S, H, max_parts, 2]: running max (log2 units), sum
  float* ws_o;   // [S, H, max_parts, D]: partition output normalised by its sum
  int* counters; // [S, H] partitions finished; NULL = leave the merge to the reduce kernel
  const int32_t* items;  // [n, 2] (sequence, partition) in launch order; NULL = grid order
  int H;
  int maxB;
  int log2_bs;
  int part_tokens;
  int max_parts;
  float qk_scale;  // scale * log2(e)
};

template <class DT, int D, int U>
struct Shape {
  static constexpr int kVec = DT::kVec;
  static constexpr int kLPT = D / kVec;          // lanes per token row
  static constexpr int kTPI = kWave / kLPT;      // token rows per wave load
  static constexpr int kChunk = kTPI * U;        // tokens per wave chunk
  static_assert(kLPT >= 4 && kLPT <= 64, "row width");
};

__device__ __forceinline__ u32x4 load16(const char* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// K/V are read exactly once per decode: non-temporal loads keep them from
// displacing reusable lines (measured ~15% faster on the 13B-layer shape).
__device__ __forceinline__ u32x4 load_stream(const char* p) {
#ifdef PA_TEMPORAL_LOADS
  return *reinterpret_cast<const u32x4*>(p);
#else
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#endif
}

// Per-wave state for streaming one partition's chunks.
struct ChunkCtx {
  const char* kc;
  const char* vc;
  int log2_tile;       // log2 of the bytes of one (block, head) tile: bs * D * elem
  int H;
  int h;
  uint32_t lane_off;   // this lane's byte offset inside a group of token rows
  int tbl;             // this lane's table entry (lane j = j-th block of the partition)
  int log2_bs;
  int bs_mask;
  int row;             // this lane's token row inside a load group
  int ntok;            // tokens in the partition
  int last_group;      // first token of the last group holding a valid token
  float qk_scale;
};

// One chunk of U token-row groups: issue 2U 16-byte loads (K and V), then
// q.k, online softmax update and P.V.  kMasked is the partition's last,
// partial chunk: its loads are clamped to rows of groups that hold valid
// tokens (so no extra memory is touched and no table entry past the
// sequence is read) and the loaded values of invalid tokens are zeroed.
template <class DT, int D, int U, bool kMasked>
__device__ __forceinline__ void chunk_step(const ChunkCtx& cx, int t0, u32x4 qv, float& m,
                                           float& l, float* acc) {
  using Sh = Shape<DT, D, U>;
  constexpr int kVec = DT::kVec;
  constexpr uint32_t kRowBytes = uint32_t(D) * sizeof(typename DT::T);
  u32x4 kr[U], vr[U];
  bool ok[U];
#pragma unroll
  for (int i = 0; i < U; ++i) {
    int tt = t0 + i * Sh::kTPI;  // wave-uniform token offset in the partition
    uint32_t off = cx.lane_off;
    ok[i] = true;
    if constexpr (kMasked) {
      ok[i] = tt + cx.row < cx.ntok;
      tt = min(tt, cx.last_group);
      if (tt + cx.row >= cx.ntok) off = cx.lane_off - uint32_t(cx.row) * kRowBytes;  // row 0
    }
    const int pb = __builtin_amdgcn_readlane(cx.tbl, tt >> cx.log2_bs);
    // (block, head) tile index fits 32 bits; tiles are a power of two in size
    const uint32_t tile_idx = uint32_t(pb) * uint32_t(cx.H) + uint32_t(cx.h);
    const size_t tile = (size_t(tile_idx) << cx.log2_tile) + uint32_t(tt & cx.bs_mask) * kRowBytes;
    kr[i] = load_stream(cx.kc + tile + off);
    vr[i] = load_stream(cx.vc + tile + off);
  }
  // Keep all 2U loads in flight before any of them is consumed: without this
  // fence the scheduler interleaves the dot products with the loads to save
  // registers, which serialises the memory latency.
  __builtin_amdgcn_sched_barrier(0);
  float sc[U];
  float mx = kNegBig;
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const float d = group_sum<Sh::kLPT>(dot16(DT{}, kr[i], qv, 0.f));
    sc[i] = d * cx.qk_scale;
    if constexpr (kMasked) {
      sc[i] = ok[i] ? sc[i] : -__builtin_inff();
      vr[i] = ok[i] ? vr[i] : u32x4{0, 0, 0, 0};
    }
    mx = fmaxf(mx, sc[i]);
  }
  const float mn = fmaxf(m, mx);
  const float alpha = fast_exp2(m - mn);
  l *= alpha;
#pragma unroll
  for (int e = 0; e < kVec; ++e) acc[e] *= alpha;
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const float p = fast_exp2(sc[i] - mn);
    l += p;
    axpy16(DT{}, acc, vr[i], p);
  }
  m = mn;
}

// Log-sum-exp merge of the partitions of one (sequence, head) row by one
// wave: with M = max_p m_p and w_p = l_p * 2^(m_p - M),
// out = sum_p w_p o_p / sum_p w_p.  Partials are read with agent-scope atomic
// loads (coherent across the XCDs' L2s).  Used by the fused path and by the
// reduce kernel, so both give the same bits.
template <class DT, int D, int U>
__device__ __forceinline__ void merge_partials(const DecodeParams& P, size_t row_id, int nparts,
                                               int lane) {
  using T = typename DT::T;
  using Sh = Shape<DT, D, U>;
  constexpr int kVec = DT::kVec;
  const int row = lane / Sh::kLPT;
  const int col = lane % Sh::kLPT;
  const size_t pi0 = row_id * P.max_parts;
  const float* ml = P.ws_ml + 2 * pi0;
  float L = 0.f, O[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) O[e] = 0.f;
  if (nparts <= kWave) {
    // Lane p holds partition p's (max, sum); the token rows of the wave share
    // the partitions' output loads (row r takes p = r, r + kTPI, ...), so the
    // merge costs two dependent round trips whatever nparts is.
    const bool has = lane < nparts;
    const float mp = has ? __hip_atomic_load(ml + 2 * lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                         : kNegBig;
    const float lp = has ? __hip_atomic_load(ml + 2 * lane + 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)
                         : 0.f;
    float M = mp;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
    const float wl = has ? lp * fast_exp2(mp - M) : 0.f;
    // Uniform trip count: the shuffle runs with every lane active (a lane
    // shuffling from an inactive lane would read 0).
    const int rounds = (nparts + Sh::kTPI - 1) / Sh::kTPI;
    for (int k = 0; k < rounds; ++k) {
      const int p = row + k * Sh::kTPI;
      const float w = __shfl(wl, min(p, kWave - 1), kWave);
      if (p < nparts) {
        const float* po = P.ws_o + (pi0 + p) * D + col * kVec;
#pragma unroll
        for (int e = 0; e < kVec; ++e)
          O[e] += w * __hip_atomic_load(po + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    L = wl;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) L += __shfl_xor(L, off, kWave);
#pragma unroll
    for (int off = Sh::kLPT; off < kWave; off <<= 1) {
#pragma unroll
      for (int e = 0; e < kVec; ++e) O[e] += __shfl_xor(O[e], off, kWave);
    }
  } else {
    float M = kNegBig;
    for (int p = 0; p < nparts; ++p)
      M = fmaxf(M, __hip_atomic_load(ml + 2 * p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    for (int p = 0; p < nparts; ++p) {
      const float mp = __hip_atomic_load(ml + 2 * p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float lp = __hip_atomic_load(ml + 2 * p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float w = lp * fast_exp2(mp - M);
      L += w;
      const float* po = P.ws_o + (pi0 + p) * D + col * kVec;
#pragma unroll
      for (int e = 0; e < kVec; ++e)
        O[e] += w * __hip_atomic_load(po + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (row != 0) return;
  T* o = reinterpret_cast<T*>(P.out) + row_id * D + col * kVec;
#pragma unroll
  for (int e = 0; e < kVec; ++e) o[e] = to_store(DT{}, O[e] / L);
}

// One wave owns one (sequence, head, partition) from start to end; a
// workgroup is kWaves independent waves for kWaves consecutive heads of the
// same (sequence, partition), which read the same table entries.  No LDS and
// no barrier: a wave merges its token rows with shuffles and stores its row.
template <class DT, int D, int U>
__global__ __launch_bounds__(kThreads) void decode_wave_kernel(DecodeParams P) {
  using T = typename DT::T;
  using Sh = Shape<DT, D, U>;
  constexpr int kVec = DT::kVec;
  constexpr size_t kRowBytes = size_t(D) * sizeof(T);

  const int wave = wave_uniform(threadIdx.x / kWave);
  const int H = P.H;
  int hg = blockIdx.x, part = blockIdx.y, s = blockIdx.z;
  if (P.items != nullptr) {  // scheduled launch: x = item * head_groups + head group
    const int ngroups = (H + kWaves - 1) / kWaves;
    const int item = blockIdx.x / ngroups;
    hg = blockIdx.x - item * ngroups;
    s = P.items[2 * item];
    part = P.items[2 * item + 1];
  }
  const int h = hg * kWaves + wave;
  if (h >= H) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int log2_bs = P.log2_bs;
  const size_t row_id = size_t(s) * H + h;

  const int row = lane / Sh::kLPT;
  const int col = lane % Sh::kLPT;
  const int p0 = part * P.part_tokens;
  const int blk0 = p0 >> log2_bs;
  // The table entries of the whole partition window are read together with
  // the context length (entries past the context are loaded as integers but
  // never used as addresses), so the K/V loads wait for one round trip only.
  int tbl = 0;
  if (lane < (P.part_tokens >> log2_bs) && blk0 + lane < P.maxB)
    tbl = P.block_tables[size_t(s) * P.maxB + blk0 + lane];
  int ctx = P.context_lens[s];
  ctx = min(ctx, min(P.maxB << log2_bs, P.max_parts * P.part_tokens));
  const int nparts = (ctx + P.part_tokens - 1) / P.part_tokens;
  if (part >= nparts) {
    if (part == 0 && row == 0) {  // empty context: zero output row
      T* o = reinterpret_cast<T*>(P.out) + row_id * D + col * kVec;
#pragma unroll
      for (int e = 0; e < kVec; ++e) o[e] = to_store(DT{}, 0.f);
    }
    return;
  }
  const int ntok = min(P.part_tokens, ctx - p0);
  const u32x4 qv = load16(reinterpret_cast<const char*>(P.q) + row_id * kRowBytes + col * 16);

  constexpr int kLog2Row = __builtin_ctz(unsigned(kRowBytes));
  const uint32_t lane_off = uint32_t(row) * uint32_t(kRowBytes) + uint32_t(col) * 16u;
  ChunkCtx cx{reinterpret_cast<const char*>(P.k_cache), reinterpret_cast<const char*>(P.v_cache),
              kLog2Row + log2_bs, H, h, lane_off, tbl,
              log2_bs, (1 << log2_bs) - 1, row, ntok, (ntok - 1) & ~(Sh::kTPI - 1), P.qk_scale};

  float m = kNegBig, l = 0.f;
  float acc[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) acc[e] = 0.f;
  const int nfull = ntok / Sh::kChunk;
  int c = 0;
  for (; c < nfull; ++c) chunk_step<DT, D, U, false>(cx, c * Sh::kChunk, qv, m, l, acc);
  if (c * Sh::kChunk < ntok) chunk_step<DT, D, U, true>(cx, c * Sh::kChunk, qv, m, l, acc);

#pragma unroll
  for (int off = Sh::kLPT; off < kWave; off <<= 1) {
    const float mo = __shfl_xor(m, off, kWave);
    const float lo = __shfl_xor(l, off, kWave);
    const float mn = fmaxf(m, mo);
    const float a = fast_exp2(m - mn), b = fast_exp2(mo - mn);
    l = l * a + lo * b;
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[e] = acc[e] * a + __shfl_xor(acc[e], off, kWave) * b;
    m = mn;
  }
  const float inv = 1.0f / l;  // l >= 1: the running max token contributes 2^0
  if (nparts == 1) {
    if (row != 0) return;
    T* o = reinterpret_cast<T*>(P.out) + row_id * D + col * kVec;
#pragma unroll
    for (int e = 0; e < kVec; ++e) o[e] = to_store(DT{}, acc[e] * inv);
    return;
  }
  const size_t pi0 = row_id * P.max_parts;
  if (P.counters == nullptr) {  // two-launch form: the reduce kernel merges
    if (row == 0) {
      float* o = P.ws_o + (pi0 + part) * D + col * kVec;
#pragma unroll
      for (int e = 0; e < kVec; ++e) o[e] = acc[e] * inv;
      if (col == 0) {
        P.ws_ml[2 * (pi0 + part)] = m;
        P.ws_ml[2 * (pi0 + part) + 1] = l;
      }
    }
    return;
  }
  // Fused merge: the wave that finishes a (sequence, head) last merges all of
  // its partitions.  Partials and the counter are exchanged only through
  // agent-scope atomic accesses, which are coherent across the XCDs' L2s
  // without cache-wide write-back/invalidate fences: the partial stores are
  // complete (s_waitcnt) before this wave's counter increment is issued, and
  // the merging wave issues its partial loads only after its increment
  // returned the count of all the others.
  if (row == 0) {
    float* o = P.ws_o + (pi0 + part) * D + col * kVec;
#pragma unroll
    for (int e = 0; e < kVec; ++e)
      __hip_atomic_store(o + e, acc[e] * inv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (col == 0) {
      __hip_atomic_store(P.ws_ml + 2 * (pi0 + part), m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(P.ws_ml + 2 * (pi0 + part) + 1, l, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // all counters zero: this wave's stores are complete
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int prev = 0;
  if (lane == 0)
    prev = __hip_atomic_fetch_add(P.counters + row_id, 1, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0, kWave);
  if (prev != nparts - 1) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (lane == 0)  // every partition has counted: reset for the next call
    __hip_atomic_store(P.counters + row_id, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  merge_partials<DT, D, U>(P, row_id, nparts, lane);
}


// Second launch of the two-launch form: one wave per (sequence, head) row.
template <class DT, int D, int U>
__global__ __launch_bounds__(kWave) void decode_reduce_kernel(DecodeParams P) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  int ctx = P.context_lens[s];
  ctx = min(ctx, min(P.maxB << P.log2_bs, P.max_parts * P.part_tokens));
  const int nparts = (ctx + P.part_tokens - 1) / P.part_tokens;
  if (nparts <= 1) return;  // written by the partition kernel
  merge_partials<DT, D, U>(P, size_t(s) * P.H + h, nparts, threadIdx.x);
}

// ------------------------------------------------------------------ host side
constexpr int kUnroll = PA_DECODE_UNROLL;  // 16-byte K loads (and V loads) per lane per chunk

constexpr int64_t kSchedTargetWaves = 1536;  // 256 CUs x 6

struct Plan {
  int part_tokens;
  int max_parts;
  size_t ws_bytes;
};

// Workspace: [S*H int32 counters, padded to 256 B][S*H*P*2 float (max, sum)][S*H*P*D float]
static size_t counter_bytes(int32_t S, int32_t H) {
  return (size_t(S) * H * sizeof(int) + 255) & ~size_t(255);
}

static int chunk_tokens(int32_t head_dim, int32_t dtype) {
  const int vec = 16 / elem_bytes(dtype);
  return (kWave / (head_dim / vec)) * kUnroll;
}

// Context-partition size.  Requested sizes must be multiples of 32 and of the
// block size and span at most 64 blocks.  The automatic choice keeps
// partitions short (better balance across CUs) unless the launch already has
// many workgroups.
static int make_plan(int32_t S, int32_t H, int32_t D, int32_t bs, int32_t max_ctx,
                     int32_t dtype, int32_t requested, Plan* plan) {
  int rc = check_shape(D, bs, dtype);
  if (rc != PA_OK) return rc;
  if (S < 0 || H <= 0 || max_ctx < 0 || requested < 0) return PA_ERR_INVALID;
  if (S > 65535 || H > 65535) return PA_ERR_UNSUPPORTED;
  const int max_tokens = 64 * bs;
  int pt = requested;
  if (pt == 0) {
    const int64_t rows = int64_t(S) * H;
    pt = 256;
    // Larger partitions once there are plenty of workgroups anyway.
    while (pt * 2 <= max_tokens && pt < 1024 &&
           rows * ((int64_t(max_ctx) + 2 * pt - 1) / (2 * pt)) >= 16384)
      pt *= 2;
    if (pt < bs) pt = bs;
    if (pt > max_tokens) pt = max_tokens;
  } else {
    if (pt % 32 != 0 || pt % bs != 0 || pt > max_tokens) return PA_ERR_INVALID;
  }
  (void)chunk_tokens;
  const int parts = max_ctx == 0 ? 1 : (max_ctx + pt - 1) / pt;
  plan->part_tokens = pt;
  plan->max_parts = parts;
  plan->ws_bytes = parts > 1 ? counter_bytes(S, H) + size_t(S) * H * parts * (size_t(D) + 2) * sizeof(float)
                             : 0;
  return PA_OK;
}

template <class DT, int D>
static void launch_partitions(const DecodeParams& p, int S, int num_items, hipStream_t st) {
  const int ngroups = (p.H + kWaves - 1) / kWaves;
  const dim3 grid = p.items ? dim3(unsigned(num_items) * unsigned(ngroups), 1, 1)
                            : dim3(ngroups, p.max_parts, S);
  hipLaunchKernelGGL((decode_wave_kernel<DT, D, kUnroll>), grid, dim3(kThreads), 0, st, p);
}

template <class DT, int D>
static void launch_reduce(const DecodeParams& p, int S, int, hipStream_t st) {
  dim3 grid(p.H, S);
  hipLaunchKernelGGL((decode_reduce_kernel<DT, D, kUnroll>), grid, dim3(kWave), 0, st, p);
}

template <bool kPartitions>
static void dispatch(int32_t dtype, int32_t D, const DecodeParams& p, int S, int n_items,
                     hipStream_t st) {
#define PA_LAUNCH(DT_, D_)                               \
  do {                                                   \
    if (kPartitions)                                     \
      launch_partitions<DT_, D_>(p, S, n_items, st);     \
    else                                                 \
      launch_reduce<DT_, D_>(p, S, n_items, st);         \
  } while (0)
  if (dtype == PA_F32) {
    if (D == 64) PA_LAUNCH(F32, 64); else PA_LAUNCH(F32, 128);
  } else if (dtype == PA_F16) {
    if (D == 64) PA_LAUNCH(F16, 64); else PA_LAUNCH(F16, 128);
  } else {
    if (D == 64) PA_LAUNCH(BF16, 64); else PA_LAUNCH(BF16, 128);
  }
#undef PA_LAUNCH
}

enum { kDoPartitions = 1, kDoReduce = 2, kFused = 4 };

static int decode_impl(int what, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t maxB, const int32_t* context_lens,
                       int32_t S, int32_t H, int32_t D, int32_t bs, int64_t NB, float scale,
                       int32_t max_ctx, int32_t dtype, void* out, void* workspace,
                       size_t workspace_bytes, int32_t partition_tokens, void* stream,
                       const int32_t* items = nullptr, int32_t num_items = 0) {
  Plan plan;
  int rc = make_plan(S, H, D, bs, max_ctx, dtype, partition_tokens, &plan);
  if (rc != PA_OK) return rc;
  if (S == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PA_ERR_INVALID;
  if (maxB <= 0 || NB <= 0) return PA_ERR_INVALID;
  if (uint64_t(NB) * uint64_t(H) > 0xFFFFFFFFull) return PA_ERR_UNSUPPORTED;  // 32-bit tile index
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return PA_ERR_INVALID;
  if (plan.ws_bytes > 0) {
    if (!workspace || workspace_bytes < plan.ws_bytes) return PA_ERR_WORKSPACE;
    if (!aligned16(workspace)) return PA_ERR_INVALID;
  }
  DecodeParams p;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = out;
  char* ws = reinterpret_cast<char*>(workspace);
  const bool split = plan.ws_bytes > 0;
  p.counters = (split && (what & kFused)) ? reinterpret_cast<int*>(ws) : nullptr;
  p.ws_ml = split ? reinterpret_cast<float*>(ws + counter_bytes(S, H)) : nullptr;
  p.ws_o = split ? p.ws_ml + size_t(S) * H * plan.max_parts * 2 : nullptr;
  p.H = H;
  p.maxB = maxB;
  p.log2_bs = log2_exact(bs);
  p.part_tokens = plan.part_tokens;
  p.max_parts = plan.max_parts;
  p.qk_scale = scale * kLog2e;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  p.items = items;
  if (items && num_items <= 0) {
    // empty schedule: nothing to attend to, but ctx = 0 rows still need zeros;
    // fall back to grid order, whose empty partitions exit at once
    p.items = nullptr;
  }
  if (what & kDoPartitions) dispatch<true>(dtype, D, p, S, num_items, st);
  if ((what & kDoReduce) && !(what & kFused) && plan.max_parts > 1)
    dispatch<false>(dtype, D, p, S, num_items, st);
  return launch_status();
}

}  // namespace pa

extern "C" {

int pa_decode_plan(int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t block_size,
                   int32_t max_context_len, int32_t dtype, int32_t partition_tokens,
                   int32_t* partition_tokens_out, int32_t* num_partitions_out,
                   size_t* workspace_bytes_out) {
  pa::Plan plan;
  int rc = pa::make_plan(num_seqs, num_heads, head_dim, block_size, max_context_len, dtype,
                         partition_tokens, &plan);
  if (rc != PA_OK) return rc;
  if (partition_tokens_out) *partition_tokens_out = plan.part_tokens;
  if (num_partitions_out) *num_partitions_out = plan.max_parts;
  if (workspace_bytes_out) *workspace_bytes_out = plan.ws_bytes;
  return PA_OK;
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_context_len, int32_t dtype,
                                int32_t partition_tokens) {
  pa::Plan plan;
  int rc = pa::make_plan(num_seqs, num_heads, head_dim, block_size, max_context_len, dtype,
                         partition_tokens, &plan);
  return rc == PA_OK ? plan.ws_bytes : size_t(-1);
}

int pa_decode_schedule(const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                       int32_t head_dim, int32_t block_size, int32_t dtype,
                       int32_t partition_tokens, int32_t* items, int32_t capacity,
                       int32_t* num_items, int32_t* partition_tokens_out,
                       int32_t* max_context_len_out) {
  if (!context_lens || num_seqs < 0 || !num_items || (capacity > 0 && !items))
    return PA_ERR_INVALID;
  int32_t max_ctx = 0;
  for (int32_t s = 0; s < num_seqs; ++s) {
    if (context_lens[s] < 0) return PA_ERR_INVALID;
    max_ctx = context_lens[s] > max_ctx ? context_lens[s] : max_ctx;
  }
  int32_t req = partition_tokens;
  if (req == 0) {
    // Largest partition (up to 1024 tokens and 64 blocks) that still gives
    // about six waves per CU: long waves stream without pause, the
    // longest-first order evens out the end, and fewer partials are merged.
    int rc0 = pa::check_shape(head_dim, block_size, dtype);
    if (rc0 != PA_OK) return rc0;
    if (num_heads <= 0) return PA_ERR_INVALID;
    const int max_pt = 64 * block_size < 1024 ? 64 * block_size : 1024;
    req = max_pt;
    while (req > 256 && req > block_size) {
      int64_t waves = 0;
      for (int32_t s = 0; s < num_seqs; ++s) waves += (context_lens[s] + req - 1) / req;
      if (waves * num_heads >= pa::kSchedTargetWaves) break;
      req /= 2;
    }
  }
  pa::Plan plan;
  int rc = pa::make_plan(num_seqs, num_heads, head_dim, block_size, max_ctx, dtype, req, &plan);
  if (rc != PA_OK) return rc;
  const int pt = plan.part_tokens;
  // Longest first: every full partition (in sequence order), then the partial
  // last partitions from longest to shortest, then empty sequences (their
  // item only writes the zero row).  Short items end the launch, so the last
  // waves to start are the quickest to finish.
  int64_t n = 0;
  for (int32_t s = 0; s < num_seqs; ++s) n += context_lens[s] / pt;
  for (int32_t s = 0; s < num_seqs; ++s) n += (context_lens[s] % pt != 0 || context_lens[s] == 0);
  *num_items = int32_t(n);
  if (partition_tokens_out) *partition_tokens_out = pt;
  if (max_context_len_out) *max_context_len_out = max_ctx;
  if (n > capacity) return PA_ERR_CAPACITY;
  int64_t k = 0;
  for (int32_t s = 0; s < num_seqs; ++s)
    for (int32_t p = 0; p < context_lens[s] / pt; ++p) {
      items[2 * k] = s;
      items[2 * k + 1] = p;
      ++k;
    }
  // partial partitions by decreasing size (ties in sequence order)
  std::vector<int32_t> partial;
  for (int32_t s = 0; s < num_seqs; ++s)
    if (context_lens[s] % pt != 0) partial.push_back(s);
  std::stable_sort(partial.begin(), partial.end(), [&](int32_t a, int32_t b) {
    return context_lens[a] % pt > context_lens[b] % pt;
  });
  for (int32_t s : partial) {
    items[2 * k] = s;
    items[2 * k + 1] = context_lens[s] / pt;
    ++k;
  }
  for (int32_t s = 0; s < num_seqs; ++s)
    if (context_lens[s] == 0) {
      items[2 * k] = s;
      items[2 * k + 1] = 0;
      ++k;
    }
  return PA_OK;
}

#define PA_DECODE_ARGS                                                                      \
  const void *q, const void *k_cache, const void *v_cache, const int32_t *block_tables,    \
      int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs,            \
      int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,          \
      float scale, int32_t max_context_len, int32_t dtype, void *out, void *workspace,      \
      size_t workspace_bytes, int32_t partition_tokens, void *stream
#define PA_DECODE_PASS                                                                      \
  q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads, \
      head_dim, block_size, num_blocks, scale, max_context_len, dtype, out, workspace,      \
      workspace_bytes, partition_tokens, stream

int pa_decode(PA_DECODE_ARGS) {
  return pa::decode_impl(pa::kDoPartitions | pa::kDoReduce | pa::kFused, PA_DECODE_PASS);
}
int pa_decode_partitions(PA_DECODE_ARGS) {
  return pa::decode_impl(pa::kDoPartitions, PA_DECODE_PASS);
}
int pa_decode_reduce(PA_DECODE_ARGS) { return pa::decode_impl(pa::kDoReduce, PA_DECODE_PASS); }

int pa_decode_scheduled(PA_DECODE_ARGS, const int32_t* items, int32_t num_items) {
  if (num_seqs > 0 && (!items || num_items <= 0)) return PA_ERR_INVALID;
  return pa::decode_impl(pa::kDoPartitions | pa::kDoReduce | pa::kFused, PA_DECODE_PASS, items,
                         num_items);
}

}  // extern "C"

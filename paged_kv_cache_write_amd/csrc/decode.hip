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
//  * A row (sequence, head) is cut into partitions (token ranges).  One wave
//    (64 lanes) owns one (row, partition) from start to end; a workgroup is
//    one wave, or, in launches with many rounds of waves, 4 waves of
//    consecutive heads of one item (they read 16 KiB runs of each block
//    together).  Partitions give the 256 CUs enough independent waves and
//    even out unequal context lengths.
//  * A (block, head) tile is bs * D contiguous elements.  A lane owns a
//    16-byte slice of one token row, so one wave-wide load reads 64 x 16 B =
//    1 KiB of consecutive bytes of one tile: fully coalesced.  Each lane
//    consumes exactly the bytes it loaded, so K/V go from HBM to registers;
//    there is no LDS staging and no barrier.
//  * A wave works on chunks of U load instructions for K and U for V issued
//    back to back (non-temporal: K/V are read once).
//  * q.k partial dots use v_dot2_f32_{f16,bf16} (exact products, float32
//    sums); the lanes of one token row are summed with DPP butterflies; the
//    softmax is the online (running max / running sum) form in base 2 with
//    scale*log2(e) folded into the logit; P.V accumulates in float32
//    (v_fma_mix_f32 for fp16).
//  * The partition's table entries are loaded once per wave into one VGPR
//    (lane j = j-th block of the partition) and read with v_readlane, so a
//    block's address is wave-uniform scalar arithmetic.
//  * Shared prefixes (comfyai.app 6.4.2-6.4.3: sequences map logical blocks
//    to the same physical blocks): a group wave streams each shared tile
//    once and runs up to kGroup queries of the sharing sequences against it.
//  * A wave merges (max, sum, accumulator) across its token rows with
//    shuffles.  A row with one partition is stored directly.  Otherwise the
//    partial (max, sum, normalised output) goes to the workspace and the
//    partitions are merged with the log-sum-exp rule: by the last wave to
//    finish the row (one launch, an agent-scope counter per row), or by a
//    second kernel (pa_decode_partitions + pa_decode_reduce).

#include <hip/hip_ext.h>

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <unordered_map>
#include <vector>

#include "internal.hpp"
#include "launch_common.hpp"
#include "pa_device.hpp"
#include "xcd_order.hpp"

namespace pa {

constexpr int kWaves = 1;  // waves per workgroup
constexpr int kThreads = kWaves * kWave;
// Scheduled launches of at least this many waves (several rounds of the
// wave slots) use workgroups of kWideWaves consecutive heads: their waves
// read kWideWaves adjacent tiles of each block at once (measured: 2.7% less
// time at 256 sequences x 40 heads; 5% more at 2360 waves, where 4-wave
// workgroups spread unevenly over the CUs).
constexpr int64_t kWideLaunchWaves = 8192;
constexpr int kWideWaves = 4;
constexpr int kUnroll = 8;   // 16-byte K loads (and V loads) per lane per chunk
constexpr int kGroup = 8;                  // queries per group wave (float32, vector ALU)
constexpr int kGroupMfma = 16;             // queries per group wave on the matrix cores
constexpr int kGroupUnroll = 4;            // chunk of a group wave (register budget)
constexpr int kSharedPartTokens = 256;  // partition of a shared range
constexpr float kGroupSlack = 8.0f;  // lazy rescale threshold of the group waves, log2 units
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // running-max start: finite, so max - max never is NaN

// Scheduled work items (int32 fields):
//   single item [5]: sequence, partition index, first token, tokens, partitions of the row
//   group item  [5]: first member, member count, partition index, first token, tokens
//   member      [2]: sequence, partitions of its rows
constexpr int kItemInts = 5;
constexpr int kMemberInts = 2;

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
  const int32_t* items;          // single items in launch order; NULL = grid order
  const int32_t* group_items;    // group items
  const int32_t* group_members;  // members of the group items
  int H;
  int maxB;
  int log2_bs;
  int part_tokens;    // partition of the grid order
  int window_tokens;  // partition window of the launch (table entries loaded per wave)
  int max_parts;      // partition stride of the workspace
  float qk_scale;     // scale * log2(e)
  // contiguous (non-paged) K/V: token t of sequence s, head h at element
  // s * stride_s + t * stride_t + h * stride_h; max_tokens bounds t
  bool contig;
  int64_t stride_s, stride_t, stride_h, max_tokens;
  int64_t num_blocks;  // pool size (checked against table entries in debug builds)
  int num_seqs;        // sequences of the launch (checked against work items in debug builds)
  int64_t ws_o_bytes;  // bytes of the ws_o region
  int num_group_wgs;   // decode_shared_kernel: workgroups of the group items
  // Engine step: each row's new token, K and V as [S, H, D] like q, which is
  // the last token of the row's context and lies in the row's last single
  // item, and its slot (int64 [S]; negative: none).  The wave of the row's
  // last partition reads the token from here; workgroups after the launch's
  // single-item workgroups write it into the slot.  NULL: no new tokens.
  const void* new_k;
  const void* new_v;
  const int64_t* new_slots;
  int num_item_wgs;  // workgroups of the items (the token writers follow them)
  int num_units;     // scheduled launches: item workgroup units (items x head groups)
  int order_offset;  // global index of the first position of the items' region
  int num_group_pos; // shared-prefix launch: positions of the group workgroups' region
};

template <class DT, int D, int U>
struct Shape {
  static constexpr int kVec = DT::kVec;
  static constexpr int kLPT = D / kVec;          // lanes per token row
  static constexpr int kTPI = kWave / kLPT;      // token rows per wave load
  static constexpr int kChunk = kTPI * U;        // tokens per wave chunk
  static_assert(kLPT >= 4 && kLPT <= 64, "row width");
};

// Element d of a partial output is stored at (d % kVec) * kLPT + d / kVec:
// lane col's element e (d = col * kVec + e) goes to e * kLPT + col, so one
// store (or load) instruction over the lanes of a token row touches
// consecutive words.  Agent-scope stores are written through to memory one
// instruction at a time; contiguous words avoid partial-line writes.
template <class DT, int D>
__device__ __forceinline__ int part_pos(int d) {
  constexpr int kVec = DT::kVec, kLPT = D / DT::kVec;
  return (d % kVec) * kLPT + d / kVec;
}

__device__ __forceinline__ u32x4 load16(const char* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// K/V are read exactly once per decode: non-temporal loads keep them from
// displacing reusable lines (measured ~15% faster on the 13B-layer shape).
__device__ __forceinline__ u32x4 load_stream(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Loads of the matrix-core group kernel: each K line is read by two load
// instructions (half a row each), so these are ordinary (temporal) loads.
template <class V>
__device__ __forceinline__ V group_load(const char* p) {
  return *reinterpret_cast<const V*>(p);
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
  // contiguous layout: the partition's first token row of this (s, h), the
  // distance between token rows, and this lane's byte offset in a row group
  const char* kbase;
  const char* vbase;
  uint64_t row_stride;
  uint64_t lane_off_c;
  // the row's new token (the partition's last token), K and V rows, read
  // from here instead of the pool (NULL: none)
  const char* nk;
  const char* nv;
};

// Issue the 2U 16-byte loads (K and V) of one chunk.  kMasked is the
// partition's last, partial chunk: its loads are clamped to rows of groups
// that hold valid tokens (no extra memory is touched and no table entry past
// the partition is used) and ok[] marks the valid rows (chunk_apply zeroes
// the others, so the loads stay in flight until the chunk is used).
template <class DT, int D, int U, bool kMasked, bool kContig = false>
__device__ __forceinline__ void chunk_load(const ChunkCtx& cx, int t0, u32x4 (&kr)[U],
                                           u32x4 (&vr)[U], bool (&ok)[U]) {
  using Sh = Shape<DT, D, U>;
  constexpr uint32_t kRowBytes = uint32_t(D) * sizeof(typename DT::T);
#pragma unroll
  for (int i = 0; i < U; ++i) {
    int tt = t0 + i * Sh::kTPI;  // wave-uniform token offset in the partition
    uint32_t off = cx.lane_off;
    uint64_t off_c = cx.lane_off_c;
    ok[i] = true;
    if constexpr (kMasked) {
      ok[i] = tt + cx.row < cx.ntok;
      tt = min(tt, cx.last_group);
      if (tt + cx.row >= cx.ntok) {  // row 0 of the group
        off = cx.lane_off - uint32_t(cx.row) * kRowBytes;
        off_c = cx.lane_off_c - uint64_t(cx.row) * cx.row_stride;
      }
    }
    if constexpr (kContig) {
      const uint64_t rows = uint64_t(tt) * cx.row_stride + off_c;
      kr[i] = load_stream(cx.kbase + rows);
      vr[i] = load_stream(cx.vbase + rows);
      continue;
    }
    const int pb = __builtin_amdgcn_readlane(cx.tbl, tt >> cx.log2_bs);
    // (block, head) tile index fits 32 bits; tiles are a power of two in size
    const uint32_t tile_idx = uint32_t(pb) * uint32_t(cx.H) + uint32_t(cx.h);
    const size_t tile = (size_t(tile_idx) << cx.log2_tile) + uint32_t(tt & cx.bs_mask) * kRowBytes;
    const char* kp = cx.kc + tile + off;
    const char* vp = cx.vc + tile + off;
    if constexpr (kMasked) {
      // the lanes of the new token's row read it from the new K/V (token
      // writer workgroups of the launch put it into its slot)
      if (cx.nk != nullptr && t0 + i * Sh::kTPI + cx.row == cx.ntok - 1) {
        const uint32_t in_row = cx.lane_off - uint32_t(cx.row) * kRowBytes;
        kp = cx.nk + in_row;
        vp = cx.nv + in_row;
      }
    }
    kr[i] = load_stream(kp);
    vr[i] = load_stream(vp);
  }
  // Keep all 2U loads in flight before any of them is consumed: without this
  // fence the scheduler interleaves the dot products with the loads to save
  // registers, which serialises the memory latency.
  __builtin_amdgcn_sched_barrier(0);
}

// q.k, online softmax update and P.V of one query over one loaded chunk.
template <class DT, int D, int U, bool kMasked>
__device__ __forceinline__ void chunk_apply(const ChunkCtx& cx, const u32x4 (&kr)[U],
                                            const u32x4 (&vr_in)[U], const bool (&ok)[U], u32x4 qv,
                                            float& m, float& l, float* acc) {
  // rows past the partition may hold anything (NaN included): their values
  // are zeroed and their weights are 0
  u32x4 vr[U];
#pragma unroll
  for (int i = 0; i < U; ++i) vr[i] = (!kMasked || ok[i]) ? vr_in[i] : u32x4{0, 0, 0, 0};
  using Sh = Shape<DT, D, U>;
  constexpr int kVec = DT::kVec;
  // A valid row's score and weight are computed by the same operations
  // whether the chunk is masked or not (the mask selects only around them),
  // so a full chunk gives the same bits on either path.
  float sc[U];
  float mx = kNegBig;
#pragma unroll
  for (int i = 0; i < U; ++i) {
    const float d = group_sum<Sh::kLPT>(dot16(DT{}, kr[i], qv, 0.f));
    sc[i] = d * cx.qk_scale;
    mx = fmaxf(mx, (!kMasked || ok[i]) ? sc[i] : -__builtin_inff());
  }
  const float mn = fmaxf(m, mx);
  const float alpha = fast_exp2(m - mn);
  l *= alpha;
#pragma unroll
  for (int e = 0; e < kVec; ++e) acc[e] *= alpha;
#pragma unroll
  for (int i = 0; i < U; ++i) {
    float p = fast_exp2(sc[i] - mn);
    if constexpr (kMasked) p = ok[i] ? p : 0.f;
    l += p;
    axpy16(DT{}, acc, vr[i], p);
  }
  m = mn;
}

// A token writer workgroup of a launch with new tokens: row s's new token,
// its H rows of K and V, into its slot, 16 bytes per lane (the slices of a
// row are a power of two).  No wave of the launch reads the slot (the wave
// of the row's last partition takes the token from the new K/V, chunk_load),
// so the writers need no ordering with the decode waves; later launches see
// the token through the kernel boundary, as after a separate cache-write
// kernel.
template <class DT, int D>
__device__ __forceinline__ void write_new_token(const DecodeParams& P, int s) {
  constexpr int kRowBytes = D * int(sizeof(typename DT::T));
  constexpr int kLog2Vecs = __builtin_ctz(kRowBytes / 16);
  const int64_t slot = P.new_slots[s];
  if (slot < 0) return;
  if (debug_bad(slot, P.num_blocks << P.log2_bs, PA_DEBUG_SLOT)) return;
  const int64_t blk = slot >> P.log2_bs;
  const int64_t off = slot & ((int64_t(1) << P.log2_bs) - 1);
  const int per_token = P.H << kLog2Vecs;
  const char* ks = static_cast<const char*>(P.new_k) + int64_t(s) * per_token * 16;
  const char* vs = static_cast<const char*>(P.new_v) + int64_t(s) * per_token * 16;
  char* kd = static_cast<char*>(const_cast<void*>(P.k_cache));
  char* vd = static_cast<char*>(const_cast<void*>(P.v_cache));
  for (int r = int(threadIdx.x); r < per_token; r += int(blockDim.x)) {
    const int h = r >> kLog2Vecs;
    const int col = r & ((1 << kLog2Vecs) - 1);
    const u32x4 kx = load16(ks + int64_t(r) * 16);
    const u32x4 vx = load16(vs + int64_t(r) * 16);
    const int64_t dst = ((((blk * P.H + h) << P.log2_bs) + off) * kRowBytes) + int64_t(col) * 16;
    *reinterpret_cast<u32x4*>(kd + dst) = kx;
    *reinterpret_cast<u32x4*>(vd + dst) = vx;
  }
}

// Merge the token rows of a wave (lanes with equal col): afterwards every
// lane holds the wave's (max, sum, accumulator) for its columns.
template <class DT, int D, int U>
__device__ __forceinline__ void merge_rows(float& m, float& l, float* acc) {
  using Sh = Shape<DT, D, U>;
#pragma unroll
  for (int off = Sh::kLPT; off < kWave; off <<= 1) {
    const float mo = __shfl_xor(m, off, kWave);
    const float lo = __shfl_xor(l, off, kWave);
    const float mn = fmaxf(m, mo);
    const float a = fast_exp2(m - mn), b = fast_exp2(mo - mn);
    l = l * a + lo * b;
#pragma unroll
    for (int e = 0; e < DT::kVec; ++e) acc[e] = acc[e] * a + __shfl_xor(acc[e], off, kWave) * b;
    m = mn;
  }
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
        const float* po = P.ws_o + (pi0 + p) * D + col;
#pragma unroll
        for (int e = 0; e < kVec; ++e)
          O[e] += w * __hip_atomic_load(po + e * Sh::kLPT, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
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
      const float* po = P.ws_o + (pi0 + p) * D + col;
#pragma unroll
      for (int e = 0; e < kVec; ++e)
        O[e] += w * __hip_atomic_load(po + e * Sh::kLPT, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (row != 0) return;
  T* o = reinterpret_cast<T*>(P.out) + row_id * D + col * kVec;
#pragma unroll
  for (int e = 0; e < kVec; ++e) o[e] = to_store(DT{}, O[e] / L);
}

// The same merge for up to kTPI rows at once: the lanes of token row r of
// the wave (kLPT of them) merge the row `row_id` they were given (active),
// which has at most kMergeParts partitions.  Lane c of a group holds
// partition c's (max, sum); every lane loads its columns of all the
// partitions in one batch, so the rows cost two dependent round trips
// together instead of two each.
constexpr int kMergeParts = 8;
template <class DT, int D, int U>
__device__ __forceinline__ void merge_partials_grouped(const DecodeParams& P, size_t row_id,
                                                       int nparts, bool active, int lane) {
  using T = typename DT::T;
  using Sh = Shape<DT, D, U>;
  constexpr int kVec = DT::kVec;
  static_assert(kMergeParts <= Sh::kLPT, "one lane per partition");
  const int col = lane % Sh::kLPT;
  const int base = lane - col;  // first lane of this token row
  const size_t pi0 = row_id * P.max_parts;
  const float* ml = P.ws_ml + 2 * pi0;
  const bool has = active && col < nparts;
  const float mp = has ? __hip_atomic_load(ml + 2 * col, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : kNegBig;
  const float lp = has ? __hip_atomic_load(ml + 2 * col + 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)
                       : 0.f;
  float M = mp;
#pragma unroll
  for (int off = 1; off < Sh::kLPT; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, kWave));
  const float wl = has ? lp * fast_exp2(mp - M) : 0.f;
  float L = wl;
#pragma unroll
  for (int off = 1; off < Sh::kLPT; off <<= 1) L += __shfl_xor(L, off, kWave);
  // all loads first (clamped to the row's last partition: in bounds), then
  // the weighted sum with weight 0 past the row's partitions
  const int last = active ? max(nparts - 1, 0) : 0;
  float v[kMergeParts][kVec];
#pragma unroll
  for (int p = 0; p < kMergeParts; ++p) {
    const float* po = P.ws_o + (pi0 + min(p, last)) * D + col;
#pragma unroll
    for (int e = 0; e < kVec; ++e)
      v[p][e] = __hip_atomic_load(po + e * Sh::kLPT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // The sums are formed in merge_partials' order (partition p into the
  // partial sum of token row p % kTPI, then those pairwise as its shuffles
  // add them), so either merge gives the same bits for a row.
  float O[Sh::kTPI][kVec];
#pragma unroll
  for (int r = 0; r < Sh::kTPI; ++r)
#pragma unroll
    for (int e = 0; e < kVec; ++e) O[r][e] = 0.f;
#pragma unroll
  for (int p = 0; p < kMergeParts; ++p) {
    const float w = __shfl(wl, base + p, kWave);
    const bool in = p < nparts;
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      const float acc = O[p % Sh::kTPI][e] + w * v[p][e];
      O[p % Sh::kTPI][e] = in ? acc : O[p % Sh::kTPI][e];
    }
  }
#pragma unroll
  for (int stride = 1; stride < Sh::kTPI; stride *= 2)
#pragma unroll
    for (int r = 0; r < Sh::kTPI; r += 2 * stride)
#pragma unroll
      for (int e = 0; e < kVec; ++e) O[r][e] = O[r][e] + O[r + stride][e];
  if (!active) return;
  T* o = reinterpret_cast<T*>(P.out) + row_id * D + col * kVec;
#pragma unroll
  for (int e = 0; e < kVec; ++e) o[e] = to_store(DT{}, O[0][e] / L);
}

// End of a (row, partition) for the NQ queries of one wave (rows row_id[g],
// nparts[g]; the wave's token rows are already merged).  A row with one
// partition is stored directly.  Otherwise the partial goes to the
// workspace; in the one-launch form the partials are then counted, and the
// wave whose increment returns the count of all the others merges the row
// and resets its counter.
//
// Why the merging wave sees every partial (AMDGPU memory model for
// gfx942/gfx950, where each XCD has its own L2 and device-scope coherence is
// chosen per instruction by its scope bits):
//  1. Partials are relaxed atomic stores at agent scope, which compile to
//     stores with the device scope bit (sc1): they are written through the
//     XCD's L2 to the device's point of coherence.
//  2. s_waitcnt vmcnt(0) returns only once those stores are complete, i.e.
//     performed at device scope; only then is the counter increment (a
//     device-scope atomic, sc1, performed at the point of coherence) issued.
//  3. The increments of one counter are totally ordered at that point.  The
//     wave that reads count = nparts - 1 comes after every other increment,
//     and so after every other wave's partial stores were performed.
//  4. The merging wave issues its partial loads only after its increment
//     has returned (they sit behind a branch on the returned value, which
//     waits for it; in-order issue), and they are relaxed atomic loads at
//     agent scope (sc1): they miss the CU's L1 and any stale L2 line and
//     read the point of coherence, where step 3's stores already are.
// The signal fences keep the compiler from moving memory accesses across
// the wait and the branch.  In C++ terms the accesses are relaxed; the
// release/acquire form would compile to a write-back of the whole L2 at each
// producer and an invalidate at the consumer (buffer_wbl2 / buffer_inv),
// which measured about 3x slower for this launch.
template <class DT, int D, int U, int NQ>
__device__ __forceinline__ void finish(const DecodeParams& P, const size_t (&row_id)[NQ],
                                       const int (&nparts)[NQ], int nq, int part,
                                       const float (&m)[NQ], const float (&l)[NQ],
                                       const float (&acc)[NQ][DT::kVec], int lane) {
  using T = typename DT::T;
  using Sh = Shape<DT, D, U>;
  constexpr int kVec = DT::kVec;
  const int row = lane / Sh::kLPT;
  const int col = lane % Sh::kLPT;
  const bool fused = P.counters != nullptr;
  bool any_split = false;
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    if (g >= nq) break;
    // l >= 1 after any token (the running max token contributes 2^0); l = 0
    // for a group item that streamed nothing (its partial has weight zero)
    const float inv = l[g] > 0.f ? 1.0f / l[g] : 0.f;
    if (nparts[g] <= 1) {
      if (row == 0) {
        T* o = reinterpret_cast<T*>(P.out) + row_id[g] * D + col * kVec;
#pragma unroll
        for (int e = 0; e < kVec; ++e) o[e] = to_store(DT{}, acc[g][e] * inv);
      }
      continue;
    }
    any_split = true;
    if (row != 0) continue;
    const size_t pi = row_id[g] * P.max_parts + part;
    float* o = P.ws_o + pi * D + col;  // element e at e * kLPT (part_pos)
    if (fused) {
#pragma unroll
      for (int e = 0; e < kVec; ++e)
        __hip_atomic_store(o + e * Sh::kLPT, acc[g][e] * inv, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      if (col == 0) {
        __hip_atomic_store(P.ws_ml + 2 * pi, m[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(P.ws_ml + 2 * pi + 1, l[g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
#pragma unroll
      for (int e = 0; e < kVec; ++e) o[e * Sh::kLPT] = acc[g][e] * inv;
      if (col == 0) {
        P.ws_ml[2 * pi] = m[g];
        P.ws_ml[2 * pi + 1] = l[g];
      }
    }
  }
  if (!fused || !any_split) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // all counters zero: this wave's stores are complete
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  // lane g increments query g's row counter
  int target = 0;
  size_t my_row = 0;
#pragma unroll
  for (int g = 0; g < NQ; ++g)
    if (lane == g && g < nq && nparts[g] > 1) {
      my_row = row_id[g];
      target = nparts[g] - 1;
    }
  int prev = -1;
  if (target > 0)
    prev = __hip_atomic_fetch_add(P.counters + my_row, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int last = (target > 0 && prev == target) ? 1 : 0;
#pragma unroll
  for (int g = 0; g < NQ; ++g) {
    if (g >= nq) break;
    if (!__shfl(last, g, kWave)) continue;  // wave-uniform
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0)  // every partition of this row has counted: reset for the next call
      __hip_atomic_store(P.counters + row_id[g], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merge_partials<DT, D, U>(P, row_id[g], nparts[g], lane);
  }
}

// Table entries of a partition window, one per lane, and the chunk context.
template <class DT, int D, int U, bool kContig = false>
__device__ __forceinline__ ChunkCtx make_ctx(const DecodeParams& P, int s, int h, int t0,
                                             int lane) {
  using Sh = Shape<DT, D, U>;
  constexpr uint32_t kRowBytes = uint32_t(D) * sizeof(typename DT::T);
  constexpr int kLog2Row = __builtin_ctz(kRowBytes);
  const int row = lane / Sh::kLPT;
  const int col = lane % Sh::kLPT;
  ChunkCtx cx;
  if constexpr (kContig) {
    constexpr uint64_t kElem = sizeof(typename DT::T);
    const uint64_t first = (uint64_t(s) * uint64_t(P.stride_s) + uint64_t(h) * uint64_t(P.stride_h) +
                            uint64_t(t0) * uint64_t(P.stride_t)) * kElem;
    cx.kbase = reinterpret_cast<const char*>(P.k_cache) + first;
    cx.vbase = reinterpret_cast<const char*>(P.v_cache) + first;
    cx.row_stride = uint64_t(P.stride_t) * kElem;
    cx.lane_off_c = uint64_t(row) * cx.row_stride + uint64_t(col) * 16u;
    cx.row = row;
    cx.ntok = 0;
    cx.last_group = 0;
    cx.qk_scale = P.qk_scale;
    cx.nk = cx.nv = nullptr;
    return cx;
  }
  const int blk0 = t0 >> P.log2_bs;
  // The whole window is loaded speculatively, in parallel with what decides
  // its length: entries past the partition are loaded as integers but never
  // used as addresses.
  int tbl = 0;
  if (lane < (P.window_tokens >> P.log2_bs) && blk0 + lane < P.maxB) {
    tbl = P.block_tables[size_t(s) * P.maxB + blk0 + lane];
#ifdef PA_DEBUG
    // entries of blocks inside the context are addresses; the rest are never used
    if (((blk0 + lane) << P.log2_bs) < P.context_lens[s] &&
        debug_bad(tbl, P.num_blocks, PA_DEBUG_TABLE))
      tbl = 0;
#endif
  }
  cx.kc = reinterpret_cast<const char*>(P.k_cache);
  cx.vc = reinterpret_cast<const char*>(P.v_cache);
  cx.log2_tile = kLog2Row + P.log2_bs;
  cx.H = P.H;
  cx.h = h;
  cx.lane_off = uint32_t(row) * kRowBytes + uint32_t(col) * 16u;
  cx.tbl = tbl;
  cx.log2_bs = P.log2_bs;
  cx.bs_mask = (1 << P.log2_bs) - 1;
  cx.row = row;
  cx.ntok = 0;
  cx.last_group = 0;
  cx.qk_scale = P.qk_scale;
  cx.kbase = cx.vbase = nullptr;
  cx.row_stride = cx.lane_off_c = 0;
  cx.nk = cx.nv = nullptr;
  return cx;
}

// The work of one wave on one (row, partition): stream the partition's K/V
// chunks with the online softmax, merge the wave's token rows, then store the
// row or the partial (and merge the row if this wave completes it).  cx holds
// the partition's table window (make_ctx).
template <class DT, int D, int U, bool kContig>
__device__ __forceinline__ void stream_unit(const DecodeParams& P, ChunkCtx cx, size_t row_id,
                                            int part, int ntok, int nparts, int lane) {
  using T = typename DT::T;
  using Sh = Shape<DT, D, U>;
  constexpr int kVec = DT::kVec;
  constexpr size_t kRowBytes = size_t(D) * sizeof(T);
  const int row = lane / Sh::kLPT;
  const int col = lane % Sh::kLPT;
  if (ntok <= 0) {
    if (part == 0 && nparts == 0 && row == 0) {  // empty context: zero output row
      T* o = reinterpret_cast<T*>(P.out) + row_id * D + col * kVec;
#pragma unroll
      for (int e = 0; e < kVec; ++e) o[e] = to_store(DT{}, 0.f);
    }
    return;
  }
  cx.ntok = ntok;
  cx.last_group = (ntok - 1) & ~(Sh::kTPI - 1);
  const u32x4 qv = load16(reinterpret_cast<const char*>(P.q) + row_id * kRowBytes + col * 16);

  float m[1] = {kNegBig}, l[1] = {0.f};
  float acc[1][kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) acc[0][e] = 0.f;
  // Two chunk buffers: the loads of the next chunk are in flight while one
  // is computed.  Loads inside the loop are unconditional, so the compiler's
  // wait counts stay exact (a load issued on one path only makes it wait for
  // everything where the paths join); the last chunks are peeled.
  // With a new token (the last one) the last chunk is always the masked
  // one, full or not: its loads take the new token from the new K/V.  A
  // masked full chunk computes the same bits as an unmasked one.
  const int nfull = (cx.nk != nullptr ? ntok - 1 : ntok) / Sh::kChunk;
  const bool tail = nfull * Sh::kChunk < ntok;
  const int t_tail = nfull * Sh::kChunk;
  u32x4 ka[U], va[U], kb[U], vb[U];
  bool ok[U], okm[U];
  auto apply_full = [&](const u32x4 (&kr)[U], const u32x4 (&vr)[U]) {
    chunk_apply<DT, D, U, false>(cx, kr, vr, ok, qv, m[0], l[0], acc[0]);
  };
  auto apply_tail = [&](const u32x4 (&kr)[U], const u32x4 (&vr)[U]) {
    chunk_apply<DT, D, U, true>(cx, kr, vr, okm, qv, m[0], l[0], acc[0]);
  };
  if (nfull > 0) {
    chunk_load<DT, D, U, false, kContig>(cx, 0, ka, va, ok);
    int c = 0;
    for (; c + 2 < nfull; c += 2) {  // a holds chunk c
      chunk_load<DT, D, U, false, kContig>(cx, (c + 1) * Sh::kChunk, kb, vb, ok);
      apply_full(ka, va);
      chunk_load<DT, D, U, false, kContig>(cx, (c + 2) * Sh::kChunk, ka, va, ok);
      apply_full(kb, vb);
    }
    // a holds chunk c; one or two full chunks remain, then maybe the tail
    if (c + 1 < nfull) {
      chunk_load<DT, D, U, false, kContig>(cx, (c + 1) * Sh::kChunk, kb, vb, ok);
      apply_full(ka, va);
      if (tail) {
        chunk_load<DT, D, U, true, kContig>(cx, t_tail, ka, va, okm);
        apply_full(kb, vb);
        apply_tail(ka, va);
      } else {
        apply_full(kb, vb);
      }
    } else if (tail) {
      chunk_load<DT, D, U, true, kContig>(cx, t_tail, kb, vb, okm);
      apply_full(ka, va);
      apply_tail(kb, vb);
    } else {
      apply_full(ka, va);
    }
  } else {
    chunk_load<DT, D, U, true, kContig>(cx, 0, ka, va, okm);
    apply_tail(ka, va);
  }
  merge_rows<DT, D, U>(m[0], l[0], acc[0]);
  const size_t rows[1] = {row_id};
  const int nps[1] = {nparts};
  finish<DT, D, U, 1>(P, rows, nps, 1, part, m, l, acc, lane);
}

// One wave per (sequence, head, partition): grid order from context_lens, or
// a host-scheduled work list of single items.  A workgroup holds W waves of
// consecutive heads.
template <class DT, int D, int U, bool kContig = false, int W = 1>
__device__ __forceinline__ void wave_body(DecodeParams P, uint3 block) {
  const int wave = wave_uniform(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int H = P.H;
  const int ngroups = (H + W - 1) / W;
  int hg, part, s, t0;
  const int32_t* it = nullptr;
  if (P.items != nullptr) {  // scheduled launch: unit = item * head_groups + head group
    const int unit = xcd_order_unit(int(block.x), P.order_offset);
    if (unit >= P.num_units) return;  // an empty position of the order
    const int item = unit / ngroups;
    hg = unit - item * ngroups;
    it = P.items + kItemInts * item;
    s = it[0];
    part = it[1];
    t0 = it[2];
#ifdef PA_DEBUG
    // an item outside the launch (sequence), the workspace (partition index
    // and count) or the table window (first token, tokens) does nothing
    const int nt = it[3], np = it[4];
    if (s < 0 || s >= P.num_seqs || part < 0 || t0 < 0 || nt < 0 || nt > P.window_tokens ||
        np < 0 || np > P.max_parts || (np > 0 && part >= np) || (nt > 0 && np == 0)) {
      if (threadIdx.x == 0) debug_flag(PA_DEBUG_ITEM);
      return;
    }
#endif
  } else {
    hg = block.x;
    part = block.y;
    s = block.z;
    t0 = part * P.part_tokens;
  }
  const int h = hg * W + wave;
  if (h >= H) return;
  const size_t row_id = size_t(s) * H + h;
  ChunkCtx cx = make_ctx<DT, D, U, kContig>(P, s, h, t0, lane);
  int ntok, nparts;
  if (it != nullptr) {
    ntok = it[3];
    nparts = it[4];
  } else {
    int ctx = P.context_lens[s];
    // never read past the table row (the token axis) or the launched partitions
    const int cap = kContig ? int(min(P.max_tokens, int64_t(1) << 30)) : (P.maxB << P.log2_bs);
    ctx = min(ctx, min(cap, P.max_parts * P.part_tokens));
    nparts = (ctx + P.part_tokens - 1) / P.part_tokens;
    ntok = part < nparts ? min(P.part_tokens, ctx - t0) : 0;
  }
  if constexpr (!kContig) {
    if (P.new_k != nullptr && it != nullptr && ntok > 0 && part == nparts - 1) {
      constexpr size_t kRowBytes = size_t(D) * sizeof(typename DT::T);
      cx.nk = static_cast<const char*>(P.new_k) + row_id * kRowBytes;
      cx.nv = static_cast<const char*>(P.new_v) + row_id * kRowBytes;
    }
  }
  stream_unit<DT, D, U, kContig>(P, cx, row_id, part, ntok, nparts, lane);
}

template <class DT, int D, int U, bool kContig = false, int W = 1>
__global__ __launch_bounds__(W * kWave) void decode_wave_kernel(DecodeParams P) {
  if constexpr (!kContig) {
    if (P.new_k != nullptr && int(blockIdx.x) >= P.num_item_wgs) {
      write_new_token<DT, D>(P, int(blockIdx.x) - P.num_item_wgs);
      return;
    }
  }
  wave_body<DT, D, U, kContig, W>(P, uint3{blockIdx.x, blockIdx.y, blockIdx.z});
}

// One wave per (group of sequences sharing a prefix, head, shared partition):
// the shared tiles are streamed once for up to kGroup queries.  The members
// share the physical blocks of this partition, so the first member's table
// row addresses them for all.
template <class DT, int D, int U>
__global__ __launch_bounds__(kThreads) void decode_group_kernel(DecodeParams P) {
  using T = typename DT::T;
  using Sh = Shape<DT, D, U>;
  constexpr int kVec = DT::kVec;
  constexpr size_t kRowBytes = size_t(D) * sizeof(T);

  const int wave = wave_uniform(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int H = P.H;
  const int ngroups = (H + kWaves - 1) / kWaves;
  const int item = blockIdx.x / ngroups;
  const int hg = blockIdx.x - item * ngroups;
  const int h = hg * kWaves + wave;
  if (h >= H) return;
  const int32_t* it = P.group_items + kItemInts * item;
  const int moff = it[0];
  const int nq = min(int(it[1]), kGroup);
  const int part = it[2];
  const int t0 = it[3];
  const int ntok = it[4];
  // A group item is one whole shared partition of 1..kGroup members.  Any
  // other item streams nothing; if its partition index exists, each member
  // still stores a partial of weight zero there and counts it (as the
  // matrix-core group kernel does).
  const bool part_ok = part >= 0 && part < P.max_parts;
  const bool stream = part_ok && it[1] >= 1 && it[1] <= kGroup && ntok == kSharedPartTokens &&
                      t0 >= 0;
  if (!stream) {
    if (threadIdx.x == 0) debug_flag(PA_DEBUG_ITEM);
    if (!part_ok || nq <= 0) return;
  }
  const int ntok_s = stream ? ntok : 0;
  const int32_t* mem = P.group_members + kMemberInts * moff;
  ChunkCtx cx = make_ctx<DT, D, U>(P, mem[0], h, stream ? t0 : 0, lane);
  cx.ntok = ntok_s;
  cx.last_group = (max(ntok_s, 1) - 1) & ~(Sh::kTPI - 1);
  const int col = lane % Sh::kLPT;

  size_t rows[kGroup];
  int nps[kGroup];
  u32x4 qv[kGroup];
  float m[kGroup], l[kGroup], acc[kGroup][kVec];
#pragma unroll
  for (int g = 0; g < kGroup; ++g) {
    const int gi = g < nq ? g : 0;
    rows[g] = size_t(mem[kMemberInts * gi]) * H + h;
    nps[g] = mem[kMemberInts * gi + 1];
    qv[g] = load16(reinterpret_cast<const char*>(P.q) + rows[g] * kRowBytes + col * 16);
    m[g] = kNegBig;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < kVec; ++e) acc[g][e] = 0.f;
  }
  const int nfull = ntok_s / Sh::kChunk;
  int c = 0;
  for (; c < nfull; ++c) {
    u32x4 kr[U], vr[U];
    bool ok[U];
    chunk_load<DT, D, U, false>(cx, c * Sh::kChunk, kr, vr, ok);
#pragma unroll
    for (int g = 0; g < kGroup; ++g)
      if (g < nq) chunk_apply<DT, D, U, false>(cx, kr, vr, ok, qv[g], m[g], l[g], acc[g]);
  }
  if (c * Sh::kChunk < ntok_s) {
    u32x4 kr[U], vr[U];
    bool ok[U];
    chunk_load<DT, D, U, true>(cx, c * Sh::kChunk, kr, vr, ok);
#pragma unroll
    for (int g = 0; g < kGroup; ++g)
      if (g < nq) chunk_apply<DT, D, U, true>(cx, kr, vr, ok, qv[g], m[g], l[g], acc[g]);
  }
#pragma unroll
  for (int g = 0; g < kGroup; ++g)
    if (g < nq) merge_rows<DT, D, U>(m[g], l[g], acc[g]);
  finish<DT, D, U, kGroup>(P, rows, nps, nq, part, m, l, acc, lane);
}

// Shared prefixes on the matrix cores: one wave per (group of up to
// kGroupMfma sequences sharing a prefix, head, shared partition), for
// float16 / bfloat16 storage.  With several queries against one tile, q.K and
// P.V are small dense products:
//   S^T[t][q] = sum_d K[t][d] Q[q][d]   (A = 16 token rows of K, B = Q^T)
//   O^T[d][q] += sum_t V^T[d][t] P^T[t][q]   (A = V^T, B = P^T)
// The S^T result layout (lane l: tokens 4 (l/16) + r, query l % 16) is
// exactly the B operand layout P^T needs, so P never leaves the lane.  The
// V^T operand needs, in lane l, the same d of several token rows; the d
// axis of the second product is permuted (product jd, row m <-> d = NJ m +
// jd) so that lane l loads NJ consecutive elements of each of its token rows
// with one plain load and takes element jd for product jd.  The output then
// lands in lane l as query l % 16, d = NJ (4 (l/16) + r) + jd: contiguous.
// P is split into storage-type hi + lo parts (two products), which keeps the
// weights at float32-like precision; the sums l use the float32 P.  A step is
// 32 tokens (two 16-token tiles); the next step's loads are in flight while
// one is computed.
template <class DT, int D>
__device__ __forceinline__ void group_mfma_body(DecodeParams P, unsigned block_x) {
  using T = typename DT::T;
  constexpr int NK = D / 32;  // q.K products per tile (32 d each)
  constexpr int NJ = D / 16;  // P.V products per step (16 d each) = V elements per row load
  constexpr uint32_t kRowBytes = uint32_t(D) * sizeof(T);
  constexpr int kLog2Row = __builtin_ctz(kRowBytes);
  using VRow = typename std::conditional<NJ == 8, u32x4, u32x2>::type;
  static_assert(sizeof(T) == 2 && (NJ == 8 || NJ == 4), "16-bit storage, D 64 or 128");

  const int lane = threadIdx.x;
  const int H = P.H;
  const int item = int(block_x) / H;
  const int h = int(block_x) - item * H;
  const int32_t* it = P.group_items + kItemInts * item;
  const int moff = it[0];
  const int nq = min(int(it[1]), kGroupMfma);
  const int part = it[2];
  const int t0 = it[3];
  const int ntok = it[4];
  // A group item is one whole shared partition of 1..kGroupMfma members.
  // Any other item streams nothing; if its partition index exists, each
  // member still stores a partial of weight zero there and counts it, so the
  // rows complete and the counters return to zero.
  const bool part_ok = part >= 0 && part < P.max_parts;
  const bool stream = part_ok && it[1] >= 1 && it[1] <= kGroupMfma &&
                      ntok == kSharedPartTokens && t0 >= 0;
  if (!stream) {
    if (lane == 0) debug_flag(PA_DEBUG_ITEM);
    if (!part_ok || nq <= 0) return;
  }
  const int32_t* mem = P.group_members + kMemberInts * moff;
  const int qi = lane & 15;  // this lane's query (B column, output column)
  const int g = lane >> 4;   // this lane's k / row group
  const bool has_q = qi < nq;
  const int seq_q = mem[kMemberInts * (has_q ? qi : 0)];
  const int nparts_q = mem[kMemberInts * (has_q ? qi : 0) + 1];
  const size_t row_q = size_t(seq_q) * H + h;

  // Table window of the first member (all members hold the same blocks here).
  const int log2_bs = P.log2_bs;
  const int bs_mask = (1 << log2_bs) - 1;
  const int log2_tile = kLog2Row + log2_bs;
  const int blk0 = t0 >> log2_bs;
  int tbl = 0;
  if (stream && lane < (kSharedPartTokens >> log2_bs) && blk0 + lane < P.maxB) {
    tbl = P.block_tables[size_t(mem[0]) * P.maxB + blk0 + lane];
    if (debug_bad(tbl, P.num_blocks, PA_DEBUG_TABLE)) tbl = 0;  // every entry is used
  }

  u32x4 qv[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j)
    qv[j] = has_q ? load16(reinterpret_cast<const char*>(P.q) + row_q * kRowBytes +
                           (32 * j + 8 * g) * sizeof(T))
                  : u32x4{0, 0, 0, 0};

  const char* kc = reinterpret_cast<const char*>(P.k_cache);
  const char* vc = reinterpret_cast<const char*>(P.v_cache);
  // Byte offset of token row tt + r of the partition (tt a multiple of 16,
  // r < 16): a 16-token tile spans at most two blocks.
  auto row_off = [&](int tt, int r) -> size_t {
    const int b_lo = __builtin_amdgcn_readlane(tbl, tt >> log2_bs);
    const int b_hi = __builtin_amdgcn_readlane(tbl, (tt + 15) >> log2_bs);
    const int b = ((tt + r) >> log2_bs) == (tt >> log2_bs) ? b_lo : b_hi;
    return (size_t(uint32_t(b) * uint32_t(H) + uint32_t(h)) << log2_tile) +
           size_t((tt + r) & bs_mask) * kRowBytes;
  };

  // One step = 32 tokens = two 16-token tiles a.
  //   K[a][j]: K[row l % 16 of tile a][32 j + 8 g ..]           (A of q.K)
  //   V[4 a + i]: V[row 4 g + i of tile a][NJ (l % 16) ..]       (V^T of P.V)
  struct KStep { u32x4 k[2][NK]; };
  struct VStep { VRow v[8]; };
  auto issue_k = [&](KStep& st, int c) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const char* kp = kc + row_off(32 * c + 16 * a, qi) + 8 * g * sizeof(T);
#pragma unroll
      for (int j = 0; j < NK; ++j) st.k[a][j] = group_load<u32x4>(kp + 32 * j * sizeof(T));
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto issue_v = [&](VStep& st, int c) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const char* vp = vc + row_off(32 * c + 16 * a, 4 * g) + qi * NJ * sizeof(T);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st.v[4 * a + i] = group_load<VRow>(vp + i * kRowBytes);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  float m = kNegBig, l = 0.f;
  f32x4 o[NJ];
#pragma unroll
  for (int jd = 0; jd < NJ; ++jd) o[jd] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float qk_scale = P.qk_scale;

  // S^T of the step's two tiles: element r of sc[a] is token 16 a + 4 g + r, query qi
  auto qk = [&](const KStep& st, f32x4 (&sc)[2]) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      sc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NK; ++j) sc[a] = mma16x16x32(DT{}, st.k[a][j], qv[j], sc[a]);
    }
  };
  auto softmax_pv = [&](const f32x4 (&sc)[2], const VStep& st) {
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = sc[e >> 2][e & 3] * qk_scale;
    float mx = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, x[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    // The reference m moves only when a query's maximum passes it by more
    // than kGroupSlack (log2 units): weights stay <= 2^kGroupSlack, and O and
    // l are rescaled on few steps (o / l does not depend on m).
    if (__builtin_amdgcn_ballot_w64(mx > m + kGroupSlack) != 0) {  // wave-uniform
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mn);
      m = mn;
      l *= alpha;
#pragma unroll
      for (int jd = 0; jd < NJ; ++jd) o[jd] *= alpha;
    }
    u32x4 phi, plo;
#pragma unroll
    for (int p2 = 0; p2 < 4; ++p2) {
      const float p0 = fast_exp2(x[2 * p2] - m), p1 = fast_exp2(x[2 * p2 + 1] - m);
      l += p0 + p1;
      uint32_t hw, lw;
      split_pair(DT{}, p0, p1, hw, lw);
      phi[p2] = hw;
      plo[p2] = lw;
    }
#pragma unroll
    for (int jd = 0; jd < NJ; ++jd) {
      // V^T operand of product jd: element jd of the lane's eight row loads
      const uint32_t sel = (jd & 1) ? 0x07060302u : 0x05040100u;
      u32x4 va;
#pragma unroll
      for (int p2 = 0; p2 < 4; ++p2)
        va[p2] = __builtin_amdgcn_perm(uint32_t(st.v[2 * p2 + 1][jd >> 1]),
                                       uint32_t(st.v[2 * p2][jd >> 1]), sel);
      o[jd] = mma16x16x32(DT{}, va, phi, o[jd]);
      o[jd] = mma16x16x32(DT{}, va, plo, o[jd]);
    }
  };

  // Fully unrolled with a fixed step count.  Order per step c: K loads of
  // c + 1, q.K of c, V loads of c + 1, softmax and P.V of c: one step of
  // K and V is always in flight, and with a fixed count the compiler's wait
  // counts are exact (a conditional issue would make it wait for everything
  // at the join).
  constexpr int kSteps = kSharedPartTokens / 32;
  if (stream) {  // wave-uniform
    KStep ks[2];
    VStep vs[2];
    issue_k(ks[0], 0);
    issue_v(vs[0], 0);
#pragma unroll
    for (int c = 0; c < kSteps; ++c) {
      if (c + 1 < kSteps) issue_k(ks[(c + 1) & 1], c + 1);
      f32x4 sc[2];
      qk(ks[c & 1], sc);
      if (c + 1 < kSteps) issue_v(vs[(c + 1) & 1], c + 1);
      softmax_pv(sc, vs[c & 1]);
    }
  }

  // the four lanes of a query hold partial sums over their token rows
  l += __shfl_xor(l, 16, kWave);
  l += __shfl_xor(l, 32, kWave);
  // l >= 1 after streaming (the maximum token contributes 2^(max - m) >= 1);
  // l = 0 for an item that streamed nothing (its partial has weight zero)
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  const bool split = nparts_q > 1;
  if (has_q && !split) {
    T* out = reinterpret_cast<T*>(P.out) + row_q * D;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      VRow w;
#pragma unroll
      for (int p2 = 0; p2 < NJ / 2; ++p2)
        w[p2] = pack_store(DT{}, o[2 * p2][r] * inv, o[2 * p2 + 1][r] * inv);
      *reinterpret_cast<VRow*>(out + NJ * (4 * g + r)) = w;
    }
  }
  // Partials, in the merge's layout (element d at part_pos(d)) and with
  // agent-scope stores, so that they are visible on every XCD while the
  // single items of the same rows may still run (in the same launch order
  // or concurrently on another stream).  For D = 128, lane (qi, g) holds
  // d = 8 (4 g + r) + jd, i.e. positions 16 jd + 4 g + r: one 16-byte store
  // per jd (64 contiguous bytes per member and store instruction); for D = 64
  // the same lane's values pair into 8-byte stores.  Then each member's row
  // is counted, and the wave that completes a row merges it.
  if (has_q && split) {
    const size_t pi = row_q * P.max_parts + part;
    if (P.ws_o_bytes < (int64_t(1) << 31)) {  // 32-bit buffer offsets
      const __amdgpu_buffer_rsrc_t rsrc =
          __builtin_amdgcn_make_buffer_rsrc(P.ws_o, 0, int(P.ws_o_bytes), 0x00020000);
      const uint32_t base = uint32_t(pi * D * sizeof(float));
      constexpr int kAgent = 0x10;  // sc1: agent-scope coherent store
      if constexpr (D == 128) {
#pragma unroll
        for (int jd = 0; jd < NJ; ++jd) {
          const u32x4 w = {float_bits(o[jd][0] * inv), float_bits(o[jd][1] * inv),
                           float_bits(o[jd][2] * inv), float_bits(o[jd][3] * inv)};
          __builtin_amdgcn_raw_buffer_store_b128(w, rsrc, base + (16 * jd + 4 * g) * 4, 0, kAgent);
        }
      } else {
#pragma unroll
        for (int jd = 0; jd < NJ; ++jd)
#pragma unroll
          for (int r = 0; r < 2; ++r) {  // (r, r + 2) are adjacent positions
            const u32x2 w = {float_bits(o[jd][r] * inv), float_bits(o[jd][r + 2] * inv)};
            const int pos = part_pos<DT, D>(NJ * (4 * g + r) + jd);
            __builtin_amdgcn_raw_buffer_store_b64(w, rsrc, base + pos * 4, 0, kAgent);
          }
      }
    } else {
      float* po = P.ws_o + pi * D;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int jd = 0; jd < NJ; ++jd)
          __hip_atomic_store(po + part_pos<DT, D>(NJ * (4 * g + r) + jd), o[jd][r] * inv,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (g == 0) {
      __hip_atomic_store(P.ws_ml + 2 * pi, m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(P.ws_ml + 2 * pi + 1, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // Count the rows, then merge the ones this wave completes: the same
  // ordering argument as in finish() (device-scope partial stores complete
  // before the device-scope increment; merge loads at device scope after the
  // increment returned).
  if (!P.counters) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // all counters zero: this wave's stores are complete
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int last = 0;
  if (g == 0 && has_q && split) {
    const int prev = __hip_atomic_fetch_add(P.counters + row_q, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    last = prev == nparts_q - 1 ? 1 : 0;
  }
  // Members whose row this wave completed (a wave-uniform mask): every
  // partition of such a row has counted, so its counter is reset for the
  // next call; the rows are merged kTPI at a time, one per token row of the
  // wave, when they have at most kMergeParts partitions, else one by one.
  using MSh = Shape<DT, D, kUnroll>;
  uint32_t done = 0;
  for (int k = 0; k < nq; ++k)
    if (__shfl(last, k, kWave)) done |= 1u << k;
  if (done == 0) return;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int max_parts = 0;
  for (uint32_t d = done; d; d &= d - 1) {
    const int k = __builtin_ctz(d);
    const size_t row_k = size_t(mem[kMemberInts * k]) * H + h;
    if (lane == 0)
      __hip_atomic_store(P.counters + row_k, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    max_parts = max(max_parts, mem[kMemberInts * k + 1]);
  }
  if (max_parts > kMergeParts) {
    for (uint32_t d = done; d; d &= d - 1) {
      const int k = __builtin_ctz(d);
      merge_partials<DT, D, kUnroll>(P, size_t(mem[kMemberInts * k]) * H + h,
                                     mem[kMemberInts * k + 1], lane);
    }
    return;
  }
  const int my_row = lane / MSh::kLPT;  // this lane's token row: one merged row each
  while (done) {
    int mine = -1;
#pragma unroll
    for (int r = 0; r < MSh::kTPI; ++r) {
      if (done == 0) break;
      const int k = __builtin_ctz(done);
      done &= done - 1;
      if (r == my_row) mine = k;
    }
    const int k = mine < 0 ? 0 : mine;
    merge_partials_grouped<DT, D, kUnroll>(P, size_t(mem[kMemberInts * k]) * H + h,
                                           mem[kMemberInts * k + 1], mine >= 0, lane);
  }
}

template <class DT, int D>
__global__ __launch_bounds__(kWave, 2) void decode_group_mfma_kernel(DecodeParams P) {
  group_mfma_body<DT, D>(P, blockIdx.x);
}

// Shared-prefix decode in one launch (16-bit storage): workgroups
// [0, num_group_wgs) run the group items, the rest the single items.  Every
// wave stores its partials with agent-scope stores and counts its rows, and
// the wave that completes a row merges it, so the two kinds may finish in
// any order; the group waves' streaming overlaps the short single waves.
template <class DT, int D>
__global__ __launch_bounds__(kWave, 2) void decode_shared_kernel(DecodeParams P) {
  if (blockIdx.x < unsigned(P.num_group_pos)) {
    const int u = xcd_order_unit(int(blockIdx.x), 0);
    if (u >= P.num_group_wgs) return;
    group_mfma_body<DT, D>(P, unsigned(u));
    return;
  }
  const unsigned x = blockIdx.x - unsigned(P.num_group_pos);
  if (P.new_k != nullptr && x >= unsigned(P.num_item_wgs)) {
    write_new_token<DT, D>(P, int(x) - P.num_item_wgs);
    return;
  }
  wave_body<DT, D, kUnroll>(P, uint3{x, 0u, 0u});
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
constexpr int64_t kSchedTargetWaves = 2048;  // 256 CUs x 8

struct Plan {
  int part_tokens;
  int max_parts;
  size_t ws_bytes;
};

// Workspace: [R int32 counters, padded to 256 B][S*H*P*2 float (max, sum), padded to
// 16 B][S*H*P*D float], with R = S*H rows, or more when the caller reserves a
// counter region that does not depend on the call (the engine: its largest
// batch; the no-allocation entry point: a fixed prefix of its array), so that
// no call's partials ever lie where a later, larger call's counters are.
static size_t counter_bytes_rows(int64_t rows) {
  return (size_t(rows) * sizeof(int) + 255) & ~size_t(255);
}
static size_t counter_bytes(int32_t S, int32_t H) { return counter_bytes_rows(int64_t(S) * H); }

// (max, sum) floats of all partials, padded so the outputs start 16-byte aligned
static size_t ml_floats(int32_t S, int32_t H, int max_parts) {
  return (size_t(S) * H * max_parts * 2 + 3) & ~size_t(3);
}

static size_t ws_bytes_for(int32_t S, int32_t H, int32_t D, int max_parts) {
  return max_parts > 1 ? counter_bytes(S, H) +
                             (ml_floats(S, H, max_parts) + size_t(S) * H * max_parts * D) *
                                 sizeof(float)
                       : 0;
}

// Context-partition size.  Requested sizes must be multiples of 32 and of the
// block size and span at most 64 blocks.  The automatic choice keeps
// partitions short (better balance across CUs) unless the launch already has
// many waves.  `min_part` (0 = none) is a smaller partition also used in the
// launch (shared prefixes): the workspace stride then counts partitions of
// that size.
static int make_plan(int32_t S, int32_t H, int32_t D, int32_t bs, int32_t max_ctx,
                     int32_t dtype, int32_t requested, Plan* plan, int min_part = 0) {
  int rc = check_shape(D, bs, dtype);
  if (rc != PA_OK) return rc;
  if (S < 0 || H <= 0 || max_ctx < 0 || requested < 0) return PA_ERR_INVALID;
  if (S > 65535 || H > 65535) return PA_ERR_UNSUPPORTED;
  const int max_tokens = 64 * bs;
  int pt = requested;
  if (pt == 0) {
    const int64_t rows = int64_t(S) * H;
    pt = 256;
    // Larger partitions once there are plenty of waves anyway.
    while (pt * 2 <= max_tokens && pt < 1024 &&
           rows * ((int64_t(max_ctx) + 2 * pt - 1) / (2 * pt)) >= 16384)
      pt *= 2;
    if (pt < bs) pt = bs;
    if (pt > max_tokens) pt = max_tokens;
  } else {
    if (pt % 32 != 0 || pt % bs != 0 || pt > max_tokens) return PA_ERR_INVALID;
  }
  const int stride_part = (min_part > 0 && min_part < pt) ? min_part : pt;
  const int parts = max_ctx == 0 ? 1 : (max_ctx + stride_part - 1) / stride_part;
  plan->part_tokens = pt;
  plan->max_parts = parts;
  plan->ws_bytes = ws_bytes_for(S, H, D, parts);
  return PA_OK;
}

enum class Launch { kSingles, kGroups, kShared, kReduce };

// A launch, with optional HIP events that the dispatch itself records at the
// kernel's start and end (hipExtLaunchKernelGGL): they time the kernel without
// marker packets around it.
struct Timing {
  hipEvent_t start = nullptr, stop = nullptr;
};

template <class... Args, class F>
static void launch_kernel(F kernel, dim3 grid, dim3 block, hipStream_t st, Timing t,
                          Args... args) {
  if (t.start || t.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, t.start, t.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

template <class DT, int D>
static void launch(Launch what, const DecodeParams& p, int S, int n, hipStream_t st, Timing t) {
  const int ngroups = (p.H + kWaves - 1) / kWaves;
  switch (what) {
    case Launch::kGroups:
      if constexpr (std::is_same<DT, F32>::value)
        launch_kernel(decode_group_kernel<DT, D, kGroupUnroll>,
                      dim3(unsigned(n) * unsigned(ngroups)), dim3(kThreads), st, t, p);
      else
        launch_kernel(decode_group_mfma_kernel<DT, D>, dim3(unsigned(n) * unsigned(p.H)),
                      dim3(kWave), st, t, p);
      break;
    case Launch::kSingles: {
      // with new tokens, S token writer workgroups follow the item workgroups
      DecodeParams pw = p;
      const unsigned writers = p.new_k ? unsigned(S) : 0u;
      pw.order_offset = 0;
      if (p.items && !p.contig && int64_t(n) * p.H >= kWideLaunchWaves) {
        pw.num_units = n * ((p.H + kWideWaves - 1) / kWideWaves);
        const unsigned wgs = unsigned(xcd_order_positions(pw.num_units, 0));
        pw.num_item_wgs = int(wgs);
        launch_kernel(decode_wave_kernel<DT, D, kUnroll, false, kWideWaves>,
                      dim3(wgs + writers), dim3(kWideWaves * kWave), st, t, pw);
        break;
      }
      pw.num_units = p.items ? n * ngroups : 0;
      const unsigned item_wgs = p.items ? unsigned(xcd_order_positions(pw.num_units, 0)) : 0u;
      const dim3 grid = p.items ? dim3(item_wgs + writers, 1, 1) : dim3(ngroups, p.max_parts, S);
      pw.num_item_wgs = int(item_wgs);
      if (p.contig)
        launch_kernel(decode_wave_kernel<DT, D, kUnroll, true>, grid, dim3(kThreads), st, t, pw);
      else
        launch_kernel(decode_wave_kernel<DT, D, kUnroll>, grid, dim3(kThreads), st, t, pw);
      break;
    }
    case Launch::kShared:  // group and single items in one launch (16-bit storage only)
      if constexpr (!std::is_same<DT, F32>::value) {
        // with new tokens, S token writer workgroups follow the single items
        DecodeParams pw = p;
        pw.num_units = n * ngroups;
        pw.num_group_pos = int(xcd_order_positions(p.num_group_wgs, 0));
        pw.order_offset = pw.num_group_pos;
        pw.num_item_wgs = int(xcd_order_positions(pw.num_units, pw.num_group_pos));
        const unsigned writers = p.new_k ? unsigned(S) : 0u;
        launch_kernel(decode_shared_kernel<DT, D>,
                      dim3(unsigned(pw.num_group_pos) + unsigned(pw.num_item_wgs) + writers),
                      dim3(kWave), st, t, pw);
      }
      break;
    case Launch::kReduce:
      launch_kernel(decode_reduce_kernel<DT, D, kUnroll>, dim3(p.H, S), dim3(kWave), st, t, p);
      break;
  }
}

static void dispatch(Launch what, int32_t dtype, int32_t D, const DecodeParams& p, int S, int n,
                     hipStream_t st, Timing t = Timing()) {
  if (dtype == PA_F32) {
    if (D == 64) launch<F32, 64>(what, p, S, n, st, t); else launch<F32, 128>(what, p, S, n, st, t);
  } else if (dtype == PA_F16) {
    if (D == 64) launch<F16, 64>(what, p, S, n, st, t); else launch<F16, 128>(what, p, S, n, st, t);
  } else {
    if (D == 64) launch<BF16, 64>(what, p, S, n, st, t);
    else launch<BF16, 128>(what, p, S, n, st, t);
  }
}

enum { kDoPartitions = 1, kDoReduce = 2, kFused = 4 };

struct Contig {
  bool on = false;
  int64_t stride_s = 0, stride_t = 0, stride_h = 0, max_tokens = 0;
};

struct Schedule {
  bool scheduled = false;  // work lists given (else grid order)
  Contig contig;           // contiguous K/V instead of blocks
  const int32_t* items = nullptr;
  int32_t num_items = 0;
  const int32_t* group_items = nullptr;
  int32_t num_group_items = 0;
  const int32_t* group_members = nullptr;
  Timing timing;  // optional: recorded at the start of the first and the end of the last launch
  int64_t counter_rows = 0;  // counters reserved at the workspace start (0: S*H of the call)
  NewTokens new_tokens;      // optional: new tokens written by the last partitions
};

static int decode_impl(int what, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t maxB, const int32_t* context_lens,
                       int32_t S, int32_t H, int32_t D, int32_t bs, int64_t NB, float scale,
                       int32_t max_ctx, int32_t dtype, void* out, void* workspace,
                       size_t workspace_bytes, int32_t partition_tokens, void* stream,
                       const Schedule& sched = Schedule()) {
  Plan plan;
  const bool shared = sched.num_group_items > 0;
  int rc = make_plan(S, H, D, bs, max_ctx, dtype, partition_tokens, &plan,
                     shared ? kSharedPartTokens : 0);
  if (rc != PA_OK) return rc;
  if (S == 0) {
    // nothing to launch: the events still mark this point of the stream
    hipStream_t st0 = reinterpret_cast<hipStream_t>(stream);
    if (sched.timing.start && hipEventRecord(sched.timing.start, st0) != hipSuccess)
      return PA_ERR_HIP;
    if (sched.timing.stop && hipEventRecord(sched.timing.stop, st0) != hipSuccess)
      return PA_ERR_HIP;
    return PA_OK;
  }
  const Contig& cg = sched.contig;
  if (!q || !k_cache || !v_cache || (!block_tables && !cg.on) || !context_lens || !out)
    return PA_ERR_INVALID;
  if (cg.on) {
    const int64_t eb = elem_bytes(dtype);
    if (cg.max_tokens <= 0 || cg.stride_s < 0 || cg.stride_t <= 0 || cg.stride_h < 0 ||
        (cg.stride_s * eb) % 16 || (cg.stride_t * eb) % 16 || (cg.stride_h * eb) % 16)
      return PA_ERR_INVALID;
  } else {
    if (maxB <= 0 || NB <= 0) return PA_ERR_INVALID;
    if (uint64_t(NB) * uint64_t(H) > 0xFFFFFFFFull) return PA_ERR_UNSUPPORTED;  // 32-bit tile index
  }
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out))
    return PA_ERR_INVALID;
  if (shared && (kSharedPartTokens % bs != 0 || !sched.group_members)) return PA_ERR_INVALID;
  // counters first (the reserved region, at least one per row), then the partials
  const bool split = plan.ws_bytes > 0;
  const size_t cbytes = counter_bytes_rows(std::max<int64_t>(int64_t(S) * H, sched.counter_rows));
  const size_t ws_need = split ? plan.ws_bytes - counter_bytes(S, H) + cbytes : 0;
  if (split) {
    if (!workspace || workspace_bytes < ws_need) return PA_ERR_WORKSPACE;
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
  p.counters = (split && (what & kFused)) ? reinterpret_cast<int*>(ws) : nullptr;
  p.ws_ml = split ? reinterpret_cast<float*>(ws + cbytes) : nullptr;
  p.ws_o = split ? p.ws_ml + ml_floats(S, H, plan.max_parts) : nullptr;
  p.items = sched.items;
  p.group_items = sched.group_items;
  p.group_members = sched.group_members;
  p.H = H;
  p.maxB = maxB;
  p.log2_bs = log2_exact(bs);
  p.part_tokens = plan.part_tokens;
  p.window_tokens = plan.part_tokens;
  p.max_parts = plan.max_parts;
  p.qk_scale = scale * kLog2e;
  p.contig = cg.on;
  p.stride_s = cg.stride_s;
  p.stride_t = cg.stride_t;
  p.stride_h = cg.stride_h;
  p.max_tokens = cg.max_tokens;
  p.num_blocks = NB;
  p.num_seqs = S;
  p.ws_o_bytes = split ? int64_t(S) * H * plan.max_parts * D * int64_t(sizeof(float)) : 0;
  p.num_group_wgs = 0;
  const NewTokens& nt = sched.new_tokens;
  p.new_k = nt.k;
  p.new_v = nt.v;
  p.new_slots = nt.slots;
  p.num_item_wgs = 0;
  p.num_units = 0;
  p.order_offset = 0;
  p.num_group_pos = 0;
  if (nt.k || nt.v || nt.slots) {
    // the single items' last partitions hold the new tokens (the caller
    // guarantees that every row has one: no new token lies in a shared range)
    if (!nt.k || !nt.v || !nt.slots || !aligned16(nt.k) || !aligned16(nt.v) ||
        !sched.scheduled || !sched.items || sched.num_items <= 0 || cg.on)
      return PA_ERR_INVALID;
  }
  if (shared && !p.counters) return PA_ERR_INVALID;  // groups need the one-launch merge
  if (shared && cg.on) return PA_ERR_INVALID;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // the launches of this call, in order; the timing events go to the first
  // (start) and the last (stop)
  struct Step {
    Launch what;
    const DecodeParams* params;
    int n;
  };
  Step steps[3];
  int nsteps = 0;
  DecodeParams pg = p;
  if (what & kDoPartitions) {
    if (shared && dtype != PA_F32) {
      // one launch: group waves stream the shared tiles while the single
      // waves (short private tails) run beside them
      static_assert(kThreads == kWave, "the fused launch has one wave per workgroup");
      p.num_group_wgs = sched.num_group_items * H;
      steps[nsteps++] = {Launch::kShared, &p, sched.items ? sched.num_items : 0};
    } else {
      if (shared) {
        pg.window_tokens = kSharedPartTokens;
        steps[nsteps++] = {Launch::kGroups, &pg, sched.num_group_items};
      }
      if (!sched.scheduled)
        steps[nsteps++] = {Launch::kSingles, &p, 0};
      else if (sched.num_items > 0 && sched.items)
        steps[nsteps++] = {Launch::kSingles, &p, sched.num_items};
    }
  }
  if ((what & kDoReduce) && !(what & kFused) && plan.max_parts > 1)
    steps[nsteps++] = {Launch::kReduce, &p, 0};
  for (int i = 0; i < nsteps; ++i) {
    Timing t;
    if (i == 0) t.start = sched.timing.start;
    if (i == nsteps - 1) t.stop = sched.timing.stop;
    dispatch(steps[i].what, dtype, D, *steps[i].params, S, steps[i].n, st, t);
  }
  return launch_status();
}

// ---- host schedule -------------------------------------------------------

// Work of one decode, built on the host from the context lengths (and, when
// the block tables are given, the shared prefixes):
//  * Sequences whose tables start with the same physical blocks share those
//    blocks' K/V ([C] 6.4.2-6.4.3).  A group (up to kGroup members per group
//    item) covers the longest run of shared blocks common to its members, in
//    partitions of kSharedPartTokens, with one group item per partition.
//  * Every sequence's remaining tokens are cut into partitions of
//    part_tokens.  Single items are ordered longest first: every full
//    partition, then the partial last partitions from longest to shortest,
//    then one item per empty sequence (which only zeroes its row).
int min_schedule_partition_tokens() { return std::min(256, kSharedPartTokens); }

int build_schedule(const int32_t* ctx, int32_t S, int32_t H, int32_t D, int32_t bs,
                   int32_t dtype, int32_t requested, const int32_t* tables, int32_t maxB,
                   HostSchedule* hs) {
  int rc = check_shape(D, bs, dtype);
  if (rc != PA_OK) return rc;
  if (!ctx || S < 0 || H <= 0 || (tables && maxB <= 0)) return PA_ERR_INVALID;
  int32_t max_ctx = 0;
  for (int32_t s = 0; s < S; ++s) {
    if (ctx[s] < 0) return PA_ERR_INVALID;
    max_ctx = std::max(max_ctx, ctx[s]);
  }
  std::vector<int32_t> shared(static_cast<size_t>(S), 0);
  std::vector<std::vector<int32_t>> groups;
  // members per group wave: the matrix-core kernel takes 16 queries, the
  // float32 (vector ALU) kernel 8
  const size_t max_members = dtype == PA_F32 ? size_t(kGroup) : size_t(kGroupMfma);
  if (tables && kSharedPartTokens % bs == 0) {
    std::unordered_map<int32_t, int32_t> bucket_of;  // first block -> bucket index
    std::vector<std::vector<int32_t>> buckets;
    for (int32_t s = 0; s < S; ++s) {
      if (ctx[s] < kSharedPartTokens) continue;
      const int32_t first = tables[size_t(s) * maxB];
      auto ins = bucket_of.emplace(first, int32_t(buckets.size()));
      if (ins.second) buckets.emplace_back();
      buckets[ins.first->second].push_back(s);
    }
    for (auto& b : buckets) {
      if (b.size() < 2) continue;
      const int32_t lead = b[0];
      const int32_t* tl = tables + size_t(lead) * maxB;
      std::vector<int32_t> mem;
      int32_t common = ctx[lead];
      for (int32_t s : b) {
        const int32_t* ts = tables + size_t(s) * maxB;
        const int32_t nb = std::min({(ctx[lead] + bs - 1) / bs, (ctx[s] + bs - 1) / bs, maxB});
        int32_t lcp = 0;
        while (lcp < nb && ts[lcp] == tl[lcp]) ++lcp;
        const int32_t tok = std::min({lcp * bs, ctx[lead], ctx[s]});
        if (tok < kSharedPartTokens) continue;
        mem.push_back(s);
        common = std::min(common, tok);
      }
      if (mem.size() < 2) continue;
      // Every member keeps at least one token outside the shared run, so each
      // row ends in a single item (group waves also count and merge the rows
      // they complete, so the order of the two kinds does not matter).
      for (int32_t s : mem) common = std::min(common, ctx[s] - 1);
      const int32_t sh = common / kSharedPartTokens * kSharedPartTokens;
      if (sh < kSharedPartTokens) continue;
      for (int32_t s : mem) shared[s] = sh;
      groups.push_back(std::move(mem));
    }
  }
  // Automatic partitions are balanced: a row's tokens after its shared run
  // are cut into ceil(rest / pt) partitions of nearly equal length (whole
  // units of q tokens, so every partition starts on a block and chunk
  // boundary; at most pt tokens each), where pt is the smallest size (from 256
  // up, in steps of q) whose launch fits kSchedTargetWaves waves.  All waves
  // of such a launch start together and, with equal work, end together; a
  // launch that does not fit even at the largest size runs several rounds,
  // longest items first.  A requested size cuts full partitions of exactly
  // that size and one shorter last partition per row.
  const bool balanced = requested == 0;
  const int32_t q = std::max<int32_t>(32, bs);
  int32_t pt = requested;
  if (balanced) {
    const int max_pt = std::min(64 * bs, 1024);
    int64_t gwaves = 0;
    for (auto& g : groups)
      gwaves += int64_t((g.size() + max_members - 1) / max_members) *
                (shared[g[0]] / kSharedPartTokens);
    pt = max_pt;
    for (int32_t t = std::min(256, max_pt); t <= max_pt; t += q) {
      int64_t waves = gwaves;
      for (int32_t s = 0; s < S; ++s) waves += (ctx[s] - shared[s] + t - 1) / t;
      if (waves * H <= kSchedTargetWaves) {
        pt = t;
        break;
      }
    }
  }
  Plan plan;
  rc = make_plan(S, H, D, bs, max_ctx, dtype, pt, &plan, groups.empty() ? 0 : kSharedPartTokens);
  if (rc != PA_OK) return rc;
  pt = plan.part_tokens;
  hs->part_tokens = pt;
  hs->max_ctx = max_ctx;
  hs->ws_bytes = plan.ws_bytes;
  std::vector<int32_t> nparts(static_cast<size_t>(S), 0);
  for (int32_t s = 0; s < S; ++s) {
    const int32_t rest = ctx[s] - shared[s];
    nparts[s] = shared[s] / kSharedPartTokens + (rest + pt - 1) / pt;
  }
  auto push = [](std::vector<int32_t>& v, std::initializer_list<int32_t> x) {
    v.insert(v.end(), x.begin(), x.end());
  };
  hs->items.clear();
  hs->groups.clear();
  hs->members.clear();
  if (balanced) {
    // n = ceil(rest / pt) partitions of u / n or u / n + 1 units (u = units
    // of the rest; the first u % n partitions take the extra unit), so none
    // is longer than pt; the last one ends at the context.
    std::vector<int32_t> single;  // items before ordering
    for (int32_t s = 0; s < S; ++s) {
      const int32_t rest = ctx[s] - shared[s];
      if (rest <= 0) continue;
      const int32_t n = (rest + pt - 1) / pt;
      const int32_t u = (rest + q - 1) / q;
      const int32_t base = shared[s] / kSharedPartTokens;
      int32_t t0 = shared[s];
      for (int32_t p = 0; p < n; ++p) {
        const int32_t units = u / n + (p < u % n ? 1 : 0);
        const int32_t len = std::min(units * q, ctx[s] - t0);
        push(single, {s, base + p, t0, len, nparts[s]});
        t0 += len;
      }
    }
    // longest first (stable: ties keep sequence and partition order)
    const size_t n_single = single.size() / kItemInts;
    std::vector<size_t> order(n_single);
    for (size_t i = 0; i < n_single; ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) {
      return single[a * kItemInts + 3] > single[b * kItemInts + 3];
    });
    for (size_t i : order)
      hs->items.insert(hs->items.end(), single.begin() + i * kItemInts,
                       single.begin() + (i + 1) * kItemInts);
  } else {
    for (int32_t s = 0; s < S; ++s) {
      const int32_t base = shared[s] / kSharedPartTokens;
      for (int32_t p = 0; p < (ctx[s] - shared[s]) / pt; ++p)
        push(hs->items, {s, base + p, shared[s] + p * pt, pt, nparts[s]});
    }
    std::vector<int32_t> partial;
    for (int32_t s = 0; s < S; ++s)
      if ((ctx[s] - shared[s]) % pt != 0) partial.push_back(s);
    std::stable_sort(partial.begin(), partial.end(), [&](int32_t a, int32_t b) {
      return (ctx[a] - shared[a]) % pt > (ctx[b] - shared[b]) % pt;
    });
    for (int32_t s : partial) {
      const int32_t rest = ctx[s] - shared[s];
      const int32_t full = rest / pt;
      push(hs->items, {s, shared[s] / kSharedPartTokens + full, shared[s] + full * pt,
                       rest % pt, nparts[s]});
    }
  }
  for (int32_t s = 0; s < S; ++s)
    if (ctx[s] == 0) push(hs->items, {s, 0, 0, 0, 0});
  for (auto& g : groups) {
    const int32_t parts = shared[g[0]] / kSharedPartTokens;
    // chunks of at most max_members, balanced so that none is a lone member
    const size_t nchunks = (g.size() + max_members - 1) / max_members;
    for (size_t c = 0, c0 = 0; c < nchunks; ++c) {
      const int32_t moff = int32_t(hs->members.size() / kMemberInts);
      const int32_t cnt = int32_t((g.size() - c0) / (nchunks - c));
      for (int32_t i = 0; i < cnt; ++i) push(hs->members, {g[c0 + i], nparts[g[c0 + i]]});
      for (int32_t p = 0; p < parts; ++p)
        push(hs->groups, {moff, cnt, p, p * kSharedPartTokens, kSharedPartTokens});
      c0 += size_t(cnt);
    }
  }
  return PA_OK;
}

}  // namespace pa

namespace pa {

// ---- the decode without a workspace argument ------------------------------
// For callers that cannot allocate device memory (code under graph capture,
// tight serving loops): the decode's scratch (row counters and partials)
// lives in one file-scope device array, which each GPU the library runs on
// holds until the process ends.
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
// The counters keep this fixed prefix of the array (131072 rows), zeroed once
// per device; the partials of every call come after it.
constexpr size_t kNoAllocCounterBytes = kNoAllocScratchBytes / 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, size_t n) {
  for (size_t i = size_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += size_t(gridDim.x) * 256)
    p[i] = 0u;
}

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

// Device address of the current device's scratch array.  The first call on a
// device looks the address up (the array's name is only a host-side stand-in)
// and clears the counter prefix with a kernel on `st`, so the counters start
// at zero however the module was loaded; every completed decode leaves them
// zero again.
static int noalloc_scratch(hipStream_t st, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return PA_ERR_HIP;
    }
    (void)hipGetLastError();
    hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, st,
                       static_cast<uint32_t*>(ptr), kNoAllocCounterBytes / 4);
    if (launch_status() != PA_OK) return PA_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return PA_OK;
}

}  // namespace pa

namespace pa {
uint32_t debug_take_decode() { return debug_take_word(); }

int decode_scheduled_timed(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                           int32_t max_context_len, int32_t dtype, void* out, void* workspace,
                           size_t workspace_bytes, int32_t partition_tokens, void* stream,
                           const int32_t* items, int32_t num_items, const int32_t* group_items,
                           int32_t num_group_items, const int32_t* members, hipEvent_t start,
                           hipEvent_t stop, int64_t counter_rows, const NewTokens& new_tokens) {
  if (num_seqs > 0 && ((num_items > 0 && !items) || num_items < 0 || num_group_items < 0 ||
                       (num_group_items > 0 && (!group_items || !members)) ||
                       num_items + num_group_items <= 0))
    return PA_ERR_INVALID;
  Schedule sc;
  sc.scheduled = true;
  sc.items = items;
  sc.num_items = num_items;
  sc.group_items = group_items;
  sc.num_group_items = num_group_items;
  sc.group_members = members;
  sc.timing.start = start;
  sc.timing.stop = stop;
  sc.counter_rows = counter_rows;
  sc.new_tokens = new_tokens;
  return decode_impl(kDoPartitions | kDoReduce | kFused, q, k_cache, v_cache, block_tables,
                     max_blocks_per_seq, context_lens, num_seqs, num_heads, head_dim,
                     block_size, num_blocks, scale, max_context_len, dtype, out, workspace,
                     workspace_bytes, partition_tokens, stream, sc);
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

static int copy_out(const std::vector<int32_t>& v, int32_t per, int32_t* dst, int32_t cap,
                    int32_t* n) {
  if (n) *n = int32_t(v.size() / size_t(per));
  if (int64_t(v.size() / size_t(per)) > cap) return PA_ERR_CAPACITY;
  if (!v.empty()) std::copy(v.begin(), v.end(), dst);
  return PA_OK;
}

int pa_decode_schedule(const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                       int32_t head_dim, int32_t block_size, int32_t dtype,
                       int32_t partition_tokens, int32_t* items, int32_t capacity,
                       int32_t* num_items, int32_t* partition_tokens_out,
                       int32_t* max_context_len_out) {
  if (!num_items || (capacity > 0 && !items)) return PA_ERR_INVALID;
  pa::HostSchedule hs;
  int rc = pa::build_schedule(context_lens, num_seqs, num_heads, head_dim, block_size, dtype,
                              partition_tokens, nullptr, 0, &hs);
  if (rc != PA_OK) return rc;
  if (partition_tokens_out) *partition_tokens_out = hs.part_tokens;
  if (max_context_len_out) *max_context_len_out = hs.max_ctx;
  return copy_out(hs.items, pa::kItemInts, items, capacity, num_items);
}

int pa_decode_schedule_shared(const int32_t* context_lens, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_heads,
                              int32_t head_dim, int32_t block_size, int32_t dtype,
                              int32_t partition_tokens, int32_t* items, int32_t items_capacity,
                              int32_t* num_items, int32_t* group_items, int32_t group_capacity,
                              int32_t* num_group_items, int32_t* members,
                              int32_t members_capacity, int32_t* num_members,
                              int32_t* partition_tokens_out, int32_t* max_context_len_out,
                              size_t* workspace_bytes_out) {
  if (!block_tables || !num_items || !num_group_items || !num_members ||
      (items_capacity > 0 && !items) || (group_capacity > 0 && !group_items) ||
      (members_capacity > 0 && !members))
    return PA_ERR_INVALID;
  pa::HostSchedule hs;
  int rc = pa::build_schedule(context_lens, num_seqs, num_heads, head_dim, block_size, dtype,
                              partition_tokens, block_tables, max_blocks_per_seq, &hs);
  if (rc != PA_OK) return rc;
  if (partition_tokens_out) *partition_tokens_out = hs.part_tokens;
  if (max_context_len_out) *max_context_len_out = hs.max_ctx;
  if (workspace_bytes_out) *workspace_bytes_out = hs.ws_bytes;
  int rc1 = copy_out(hs.items, pa::kItemInts, items, items_capacity, num_items);
  int rc2 = copy_out(hs.groups, pa::kItemInts, group_items, group_capacity, num_group_items);
  int rc3 = copy_out(hs.members, pa::kMemberInts, members, members_capacity, num_members);
  return rc1 != PA_OK ? rc1 : (rc2 != PA_OK ? rc2 : rc3);
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
int pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                      int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                      int32_t max_context_len, int32_t dtype, void* out,
                      int32_t partition_tokens, void* stream) {
  pa::Plan plan;
  int rc = pa::make_plan(num_seqs, num_heads, head_dim, block_size, max_context_len, dtype,
                         partition_tokens, &plan);
  if (rc != PA_OK) return rc;
  // The counters keep the array's fixed prefix whatever the call's size (a
  // smaller call's partials never lie where a later call's counters are);
  // the partials follow it.
  constexpr int64_t kRows = int64_t(pa::kNoAllocCounterBytes / sizeof(int));
  void* ws = nullptr;
  if (plan.ws_bytes > 0 && num_seqs > 0) {
    if (int64_t(num_seqs) * num_heads > kRows ||
        plan.ws_bytes - pa::counter_bytes(num_seqs, num_heads) + pa::kNoAllocCounterBytes >
            pa::kNoAllocScratchBytes)
      return PA_ERR_WORKSPACE;
    rc = pa::noalloc_scratch(reinterpret_cast<hipStream_t>(stream), &ws);
    if (rc != PA_OK) return rc;
  }
  pa::Schedule sc;
  sc.counter_rows = kRows;
  return pa::decode_impl(pa::kDoPartitions | pa::kDoReduce | pa::kFused, q, k_cache, v_cache,
                         block_tables, max_blocks_per_seq, context_lens, num_seqs, num_heads,
                         head_dim, block_size, num_blocks, scale, max_context_len, dtype, out,
                         ws, ws ? pa::kNoAllocScratchBytes : 0, partition_tokens, stream, sc);
}

int pa_decode_partitions(PA_DECODE_ARGS) {
  return pa::decode_impl(pa::kDoPartitions, PA_DECODE_PASS);
}
int pa_decode_reduce(PA_DECODE_ARGS) { return pa::decode_impl(pa::kDoReduce, PA_DECODE_PASS); }

int pa_decode_scheduled(PA_DECODE_ARGS, const int32_t* items, int32_t num_items) {
  if (num_seqs > 0 && (!items || num_items <= 0)) return PA_ERR_INVALID;
  return pa::decode_scheduled_timed(PA_DECODE_PASS, items, num_items, nullptr, 0, nullptr,
                                    nullptr, nullptr, 0);
}

int pa_decode_scheduled_shared(PA_DECODE_ARGS, const int32_t* items, int32_t num_items,
                               const int32_t* group_items, int32_t num_group_items,
                               const int32_t* members) {
  return pa::decode_scheduled_timed(PA_DECODE_PASS, items, num_items, group_items,
                                    num_group_items, members, nullptr, nullptr, 0);
}

// Contiguous (non-paged) K/V: the same decode with token rows addressed by
// strides instead of the block table.  Partitions follow the rules of a
// 16-token block size (multiples of 32 up to 1024 tokens).
int pa_decode_contiguous(const void* q, const void* k, const void* v, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                         int64_t stride_seq, int64_t stride_token, int64_t stride_head,
                         int64_t max_tokens, float scale, int32_t max_context_len, int32_t dtype,
                         void* out, void* workspace, size_t workspace_bytes,
                         int32_t partition_tokens, void* stream, const int32_t* items,
                         int32_t num_items) {
  if (num_seqs > 0 && ((items && num_items <= 0) || (!items && num_items != 0)))
    return PA_ERR_INVALID;
  if (max_context_len > max_tokens) return PA_ERR_INVALID;
  pa::Schedule sc;
  sc.scheduled = items != nullptr;
  sc.items = items;
  sc.num_items = num_items;
  sc.contig.on = true;
  sc.contig.stride_s = stride_seq;
  sc.contig.stride_t = stride_token;
  sc.contig.stride_h = stride_head;
  sc.contig.max_tokens = max_tokens;
  return pa::decode_impl(pa::kDoPartitions | pa::kDoReduce | pa::kFused, q, k, v, nullptr, 1,
                         context_lens, num_seqs, num_heads, head_dim, 16, 1, scale,
                         max_context_len, dtype, out, workspace, workspace_bytes,
                         partition_tokens, stream, sc);
}

}  // extern "C"

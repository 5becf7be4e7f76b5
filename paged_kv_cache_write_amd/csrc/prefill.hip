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
// How (MI355X design): with many queries of one sequence against each key
// tile, q.K and P.V are dense products for the matrix cores.  A workgroup of
// 4 waves owns (sequence, head, 128 consecutive queries), 32 per wave in two
// column sets of 16 (each K or V operand read from LDS feeds both), and
// streams keys 0 .. its last query's position in steps of 64: the step's K
// and V rows are loaded once for the workgroup (coalesced 16-byte loads; the
// block id of each wave's group of rows is one scalar table load) into
// registers while the previous step is computed, then stored into one of two
// LDS buffers.  Each wave computes
//   S^T[t][q] = sum_d K[t][d] Q[q][d]        (v_mfma_f32_16x16x32, A = K rows)
//   O^T[d][q] += sum_t V^T[d][t] P^T[t][q]   (P^T is S^T's layout; V^T comes
//                                             from transposed LDS reads)
// with the online softmax per query column (base 2, lazy rescale), the causal
// mask (key t > query position -> weight 0) only on the steps that cross the
// wave's own positions, and l = sum P from one more product against ones.
// Float16 weights are rounded once; bfloat16 weights keep a hi + lo pair.  A
// wave skips the steps after its last query.  Rows past the workgroup's last
// key are read from their group's block (allocated memory), their scores are
// masked and their V rows are stored as zeros.
#include <type_traits>

#include "launch_common.hpp"
#include "pa_device.hpp"

namespace pa {

namespace {

constexpr float kPfLog2e = 1.4426950408889634f;
constexpr float kPfNegBig = -1.0e30f;  // running-max start: finite
constexpr float kPfSlack = 8.0f;       // lazy rescale threshold, log2 units

struct PrefillParams {
  const void* q;       // [T, H, D] queries of all sequences, packed
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;  // [S, maxB]
  const int32_t* cu_q;          // [S + 1] query offsets
  const int32_t* context_lens;  // [S] tokens in the cache, the new ones included
  void* out;                    // [T, H, D]
  int H;
  int S;
  int num_tiles;  // query tiles per sequence (of the longest chunk)
  int maxB;
  int64_t num_blocks;  // pool size (checked against table entries in debug builds)
  int log2_bs;
  float qk_scale;  // scale * log2(e)
};

constexpr int kPfWaves = 4;                 // waves per workgroup
constexpr int kPfKeys = 64;                 // keys per step
constexpr int kPfTiles = kPfKeys / 16;      // 16-key tiles of S^T per step

// LDS layout of one step.  K: key rows of D elements; the 16-byte chunk c
// of row r sits at chunk c ^ f(r), f(r) = (r >> (1 for D = 64)) mod
// chunks-per-row, so the 16 lanes of every K operand read (16 rows of one
// chunk) and of the cooperative stores (consecutive chunks of a row) fall on
// different banks.  V: key rows padded by 32 bytes, no swizzle: the
// transposed reads that build V^T operands then sit at constant offsets from
// a per-lane base, and the 32 lanes of each half of such a read (8 rows x 32
// bytes) cover the 64 banks once.
template <int D>
struct PfLds {
  static constexpr int kRow = D * 2;
  static constexpr int kChunksPerRow = kRow / 16;
  static constexpr int kShift = D == 64 ? 1 : 0;
  static constexpr int kMat = kPfKeys * kRow;  // one K step
  static constexpr int kVRow = kRow + 32;
  static constexpr int kVMat = kPfKeys * kVRow;  // one V step
  static __device__ __forceinline__ int at(int row, int chunk) {
    return row * kRow + ((chunk ^ ((row >> kShift) & (kChunksPerRow - 1))) << 4);
  }
};

// Transposed LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// 4a + b receives element b of the 4-element vectors read by lanes a, a + 4,
// a + 8 and a + 12 of the group.  When lane s of the group reads row s / 4,
// columns 4 (s % 4) .. + 3 of a row-major tile, lane i thus receives column i
// of rows 0..3: four keys of one head-dimension column.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s4 LdsS4;
  const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (LdsS4*)((__attribute__((address_space(3))) const char*)p));
  return __builtin_bit_cast(u32x2, v);
}

// MFMA operand of 16 x 32 ones (the sums of P^T's columns)
__device__ __forceinline__ u32x4 ones_operand(F16) {
  return u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};
}
__device__ __forceinline__ u32x4 ones_operand(BF16) {
  return u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
}

// Maximum over the 4 rows of 16 lanes (v_permlane16_swap / v_permlane32_swap:
// the rows that pair up in each swap exchange values).
__device__ __forceinline__ float max_over_rows(float v) {
  const uint32_t u = __builtin_bit_cast(uint32_t, v);
  auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(bits_as<float>(a[0]), bits_as<float>(a[1]));
  const uint32_t w = __builtin_bit_cast(uint32_t, v);
  auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(bits_as<float>(b[0]), bits_as<float>(b[1]));
}

template <class DT, int D, int NS>
__global__ __launch_bounds__(kPfWaves * kWave, 2) void prefill_mfma_kernel(
    PrefillParams P) {
  using T = typename DT::T;
  using L = PfLds<D>;
  constexpr int NK = D / 32;
  constexpr int NJ = D / 16;
  constexpr int kWaveQueries = 16 * NS;             // queries per wave (NS sets of 16)
  constexpr int kWgQueries = kWaveQueries * kPfWaves;
  constexpr uint32_t kRowBytes = uint32_t(D) * sizeof(T);
  constexpr int kLog2Row = __builtin_ctz(kRowBytes);
  constexpr int kChunks = kPfKeys * (D / 8);             // 16-byte chunks of one step's K
  constexpr int kPerThread = kChunks / (kPfWaves * kWave);  // of K, and as many of V
  static_assert(sizeof(T) == 2 && (NJ == 8 || NJ == 4), "16-bit storage, D 64 or 128");
  static_assert(kPerThread >= 1 && kChunks % (kPfWaves * kWave) == 0, "load split");
  __shared__ __align__(16) char lds_k[2][L::kMat];   // [buffer]
  __shared__ __align__(16) char lds_v[2][L::kVMat];

  const int tid = threadIdx.x;
  const int wave = wave_uniform(tid / kWave);
  const int lane = tid & (kWave - 1);
  // Workgroups are dealt to the 8 XCDs in turn (workgroup i to XCD i mod 8).
  // All query tiles of one (sequence, head) go to one XCD, whose L2 then
  // holds the keys they share; over the grid the last (longest, under the
  // causal mask) tiles go first, so that the short ones fill the end.
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int groups_per_xcd = (P.S * P.H + 7) / 8;
  const int grp = xcd + 8 * (slot % groups_per_xcd);
  const int qt = P.num_tiles - 1 - slot / groups_per_xcd;
  if (grp >= P.S * P.H) return;
  const int h = grp % P.H, s = grp / P.H;
  const int H = P.H;
  const int q_begin = P.cu_q[s];
  const int q_len = P.cu_q[s + 1] - q_begin;
  const int q0 = qt * kWgQueries;
  if (q0 >= q_len) return;  // whole workgroup: no barrier is skipped by part of it
  const int ctx = P.context_lens[s];
  const int pos0 = ctx - q_len + q0;
  if (pos0 < 0) return;  // inconsistent lengths: nothing is read
  const int nq_wg = min(kWgQueries, q_len - q0);
  const int kv_end = pos0 + nq_wg;  // keys [0, kv_end) for the workgroup
  const int last = kv_end - 1;
  const int qi = lane & 15;
  const int g = lane >> 4;
  // set k of this wave: queries q0 + wave * kWaveQueries + 16 k + (0..15)
  const int wq0 = wave * kWaveQueries;
  const int nq_w = max(0, min(kWaveQueries, nq_wg - wq0));
  const int wpos0 = pos0 + wq0;
  const int w_end = nq_w > 0 ? wpos0 + nq_w : 0;  // keys this wave needs
  bool has_q[NS];
  int my_pos[NS];
  size_t qrow[NS];
  u32x4 qv[NS][NK];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    has_q[k] = 16 * k + qi < nq_w;
    my_pos[k] = wpos0 + 16 * k + qi;
    qrow[k] = size_t(q_begin + q0 + wq0 + 16 * k + (has_q[k] ? qi : 0)) * H + h;
#pragma unroll
    for (int j = 0; j < NK; ++j)
      qv[k][j] = has_q[k]
                     ? *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(P.q) +
                                                       qrow[k] * kRowBytes +
                                                       (32 * j + 8 * g) * sizeof(T))
                     : u32x4{0, 0, 0, 0};
  }

  const int log2_bs = P.log2_bs;
  const int bs_mask = (1 << log2_bs) - 1;
  const int log2_tile = kLog2Row + log2_bs;
  const int32_t* trow = P.block_tables + size_t(s) * P.maxB;
  const char* kc = reinterpret_cast<const char*>(P.k_cache);
  const char* vc = reinterpret_cast<const char*>(P.v_cache);

  // Cooperative load of one step: thread tid moves chunks tid, tid + 256, ...
  // of K and of V (row = chunk / (D/8), 16-byte column = chunk % (D/8)).  A
  // wave's rows of one chunk group are 64 / (D/8) consecutive rows aligned to
  // that count (<= 8 <= bs), so they lie in one block: its id is one scalar
  // load from the table, read through the constant address space (the table
  // is not written here).  A group that starts past the last key reads the
  // last key's block instead; rows past the last key are read from their
  // group's block (allocated memory, any content), their K scores are masked
  // and their V rows are stored to LDS as zeros.
  constexpr int kRowsPerGroup = kPfWaves * kWave / (D / 8);  // rows per chunk group
  using ConstI32 = const __attribute__((address_space(4))) int32_t;
  ConstI32* trow_c = (ConstI32*)trow;
  struct Ids { int b[kPerThread]; };
  auto load_ids = [&](int base, Ids& ids) {
#pragma unroll
    for (int c = 0; c < kPerThread; ++c) {
      const int r0 = c * kRowsPerGroup + wave * (kWave / (D / 8));  // first row of the wave
      const int t = wave_uniform(min(base + r0, last));
      ids.b[c] = trow_c[t >> log2_bs];
      if (debug_bad(ids.b[c], P.num_blocks, PA_DEBUG_TABLE)) ids.b[c] = 0;  // t is in the context
    }
  };
  // Row base + r of a step lies at (base & bs_mask) + (r & bs_mask) in its
  // block (base is a multiple of 64 and bs a power of two: for bs <= 64 the
  // first term is 0, for bs >= 64 the second is r), so a load's address is a
  // wave-uniform block address plus a per-thread offset fixed for the kernel.
  uint32_t lane_off[kPerThread];
#pragma unroll
  for (int c = 0; c < kPerThread; ++c) {
    const int chunk = tid + c * kPfWaves * kWave;
    const int r = chunk / (D / 8), col = chunk % (D / 8);
    lane_off[c] = uint32_t(r & bs_mask) * kRowBytes + uint32_t(col) * 16;
  }
  struct Regs { u32x4 k[kPerThread], v[kPerThread]; };
  auto load_step = [&](int base, const Ids& ids, Regs& g_) {
    const size_t in_block = size_t(base & bs_mask) * kRowBytes;
#pragma unroll
    for (int c = 0; c < kPerThread; ++c) {
      const size_t blk = (size_t(uint32_t(ids.b[c]) * uint32_t(H) + uint32_t(h)) << log2_tile) +
                         in_block;
      g_.k[c] = *reinterpret_cast<const u32x4*>(kc + blk + lane_off[c]);
      g_.v[c] = *reinterpret_cast<const u32x4*>(vc + blk + lane_off[c]);
    }
  };
  auto store_step = [&](int buf, int base, const Regs& g_) {
    // V rows past the last key become zeros (their weights are 0, their
    // memory may hold anything); only a step that reaches past it has any
    const bool tail = base + kPfKeys - 1 > last;  // workgroup-uniform
#pragma unroll
    for (int c = 0; c < kPerThread; ++c) {
      const int chunk = tid + c * kPfWaves * kWave;
      const int r = chunk / (D / 8), col = chunk % (D / 8);
      *reinterpret_cast<u32x4*>(&lds_k[buf][L::at(r, col)]) = g_.k[c];
      *reinterpret_cast<u32x4*>(&lds_v[buf][r * L::kVRow + col * 16]) = g_.v[c];
    }
    if (tail) {  // overwrite those rows (same thread, program order)
#pragma unroll
      for (int c = 0; c < kPerThread; ++c) {
        const int chunk = tid + c * kPfWaves * kWave;
        const int r = chunk / (D / 8), col = chunk % (D / 8);
        if (base + r > last)
          *reinterpret_cast<u32x4*>(&lds_v[buf][r * L::kVRow + col * 16]) = u32x4{0, 0, 0, 0};
      }
    }
  };

  float m[NS];
  f32x4 o[NS][NJ];
  f32x4 ol[NS];  // row sums of the weights, from the matrix cores (a V^T tile of ones)
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    m[k] = kPfNegBig;
    ol[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jd = 0; jd < NJ; ++jd) o[k][jd] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float qk_scale = P.qk_scale;
  // float16 weights are rounded once (relative error <= 2^-11, weights <= 2^8);
  // bfloat16 weights keep a low part so that they stay close to float32.
  constexpr bool kSplitP = !std::is_same<DT, F16>::value;
  // this lane's part of the transposed V reads: row 4 g + qi / 4, 4 columns
  // from 4 (qi % 4); the other key half is 16 rows further
  const int v_lane = (4 * g + (qi >> 2)) * L::kVRow + 8 * (qi & 3);

  auto compute = [&](int buf, int base) {
    const char* lk = lds_k[buf];
    const char* lv = lds_v[buf] + v_lane;
    // one K operand read from LDS serves the NS query sets
    f32x4 sc[NS][kPfTiles];  // S^T tile a: keys 16 a + 4 g + r, query qi
#pragma unroll
    for (int a = 0; a < kPfTiles; ++a) {
#pragma unroll
      for (int k = 0; k < NS; ++k) sc[k][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        const u32x4 kr = *reinterpret_cast<const u32x4*>(lk + L::at(16 * a + qi, 4 * j + g));
#pragma unroll
        for (int k = 0; k < NS; ++k) sc[k][a] = mma16x16x32(DT{}, kr, qv[k][j], sc[k][a]);
      }
    }
    // P^T per 32-key chunk b (one MFMA k-extent): k-slot 8 g + 4 a' + r holds
    // key 32 b + 16 a' + 4 g + r
    constexpr int NB = kPfKeys / 32;
    u32x4 phi[NS][NB], plo[NS][NB];
#pragma unroll
    for (int k = 0; k < NS; ++k) {
      float x[4 * kPfTiles];  // raw scores q.k of keys base + 16 (e / 4) + 4 g + e % 4
#pragma unroll
      for (int e = 0; e < 4 * kPfTiles; ++e) x[e] = sc[k][e >> 2][e & 3];
      if (base + kPfKeys > wpos0 + 16 * k) {  // wave-uniform: a step on this set's diagonal
#pragma unroll
        for (int e = 0; e < 4 * kPfTiles; ++e)
          if (base + 16 * (e >> 2) + 4 * g + (e & 3) > my_pos[k]) x[e] = -__builtin_inff();
      }
      float mx = x[0];
#pragma unroll
      for (int e = 1; e < 4 * kPfTiles; ++e) mx = fmaxf(mx, x[e]);
      mx = max_over_rows(mx);
      // The running reference m moves only when a column's maximum passes it by
      // more than kPfSlack (log2 units): weights stay <= 2^kPfSlack, and the
      // rescale of O and l is skipped on most steps.  o / l does not depend on m.
      const float ms = mx * qk_scale;
      if (__builtin_amdgcn_ballot_w64(ms > m[k] + kPfSlack) != 0) {
        const float mn = fmaxf(m[k], ms);
        const float alpha = fast_exp2(m[k] - mn);
        m[k] = mn;
        ol[k][0] *= alpha;  // only element 0 is read
#pragma unroll
        for (int jd = 0; jd < NJ; ++jd) o[k][jd] *= alpha;
      }
      const float neg_m = -m[k];
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int p2 = 0; p2 < 4; ++p2) {
          const float p0 = fast_exp2(fmaf(x[8 * b + 2 * p2], qk_scale, neg_m));
          const float p1 = fast_exp2(fmaf(x[8 * b + 2 * p2 + 1], qk_scale, neg_m));
          if constexpr (kSplitP) {
            uint32_t hw, lw;
            split_pair(DT{}, p0, p1, hw, lw);
            phi[k][b][p2] = hw;
            plo[k][b][p2] = lw;
          } else {
            phi[k][b][p2] = round_pair(DT{}, p0, p1);
          }
        }
    }
    // O^T += V^T P^T: the V^T operand of head-dimension tile jd (rows d =
    // 16 jd + 0..15, k-slots = this lane group's keys 4 g + 0..3 and
    // 16 + 4 g + 0..3 of chunk b, matching P^T's slots) is two transposed
    // reads.
    const u32x4 ones = ones_operand(DT{});
#pragma unroll
    for (int b = 0; b < NB; ++b) {
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        ol[k] = mma16x16x32(DT{}, ones, phi[k][b], ol[k]);
        if constexpr (kSplitP) ol[k] = mma16x16x32(DT{}, ones, plo[k][b], ol[k]);
      }
#pragma unroll
      for (int jd = 0; jd < NJ; ++jd) {
        const u32x2 v0 = lds_read_tr16(lv + 32 * b * L::kVRow + 32 * jd);
        const u32x2 v1 = lds_read_tr16(lv + (32 * b + 16) * L::kVRow + 32 * jd);
        const u32x4 va = {v0[0], v0[1], v1[0], v1[1]};
#pragma unroll
        for (int k = 0; k < NS; ++k) {
          o[k][jd] = mma16x16x32(DT{}, va, phi[k][b], o[k][jd]);
          if constexpr (kSplitP) o[k][jd] = mma16x16x32(DT{}, va, plo[k][b], o[k][jd]);
        }
      }
    }
  };

  // Steps: LDS double buffer; the next step's rows are loaded into registers
  // while this step is computed, then stored into the other buffer.  One
  // barrier per step makes the stores visible and keeps a buffer from being
  // overwritten while another wave still reads it.  Unrolled by two so that
  // buffers are fixed per position; block ids are read one step before their
  // loads; loads are issued unconditionally (steps past the end read in-bounds
  // rows again): a load issued on one path only would make the compiler wait
  // for every load where the paths join.
  const int nsteps = (kv_end + kPfKeys - 1) / kPfKeys;
  Ids ida, idb;
  Regs r;
  load_ids(0, ida);
  load_step(0, ida, r);
  load_ids(kPfKeys, idb);
  store_step(0, 0, r);
  load_ids(2 * kPfKeys, ida);
  __syncthreads();
  for (int c = 0; c < nsteps; c += 2) {
    // step c (buffer 0): idb holds step c + 1's ids, ida step c + 2's
    load_step((c + 1) * kPfKeys, idb, r);
    if (c * kPfKeys < w_end) compute(0, c * kPfKeys);  // wave-uniform: keys this wave needs
    if (c + 1 < nsteps) store_step(1, (c + 1) * kPfKeys, r);
    load_ids((c + 3) * kPfKeys, idb);
    __syncthreads();
    // step c + 1 (buffer 1)
    load_step((c + 2) * kPfKeys, ida, r);
    if (c + 1 < nsteps && (c + 1) * kPfKeys < w_end) compute(1, (c + 1) * kPfKeys);
    if (c + 2 < nsteps) store_step(0, (c + 2) * kPfKeys, r);
    load_ids((c + 4) * kPfKeys, ida);
    __syncthreads();
  }

#pragma unroll
  for (int k = 0; k < NS; ++k) {
    if (!has_q[k]) continue;
    const float inv = 1.0f / ol[k][0];  // >= 1: the reference key's weight is 2^0 or more
    T* out = reinterpret_cast<T*>(P.out) + qrow[k] * D + 4 * g;
#pragma unroll
    for (int jd = 0; jd < NJ; ++jd) {
      const u32x2 w = {pack_store(DT{}, o[k][jd][0] * inv, o[k][jd][1] * inv),
                       pack_store(DT{}, o[k][jd][2] * inv, o[k][jd][3] * inv)};
      *reinterpret_cast<u32x2*>(out + 16 * jd) = w;  // d = 16 jd + 4 g + 0..3
    }
  }
}

constexpr int kPfSets = 2;  // 16-query sets per wave
constexpr int kPfWgQueries = 16 * kPfSets * kPfWaves;  // queries per workgroup

template <class DT, int D>
void launch_prefill(const PrefillParams& p, int S, hipStream_t st) {
  // 8 XCDs x (sequence, head) groups per XCD x query tiles; see the kernel
  const int64_t groups_per_xcd = (int64_t(S) * p.H + 7) / 8;
  const dim3 grid(unsigned(8 * groups_per_xcd * p.num_tiles));
  hipLaunchKernelGGL((prefill_mfma_kernel<DT, D, kPfSets>), grid, dim3(kPfWaves * kWave), 0, st,
                     p);
}

}  // namespace

}  // namespace pa

namespace pa {
uint32_t debug_take_prefill() { return debug_take_word(); }
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
  p.S = num_seqs;
  p.num_tiles = (max_q_len + pa::kPfWgQueries - 1) / pa::kPfWgQueries;
  // the 1-D grid's work-items (256 per workgroup) must stay below 2^32
  if (int64_t(p.num_tiles) * ((int64_t(num_seqs) * num_heads + 7) / 8) * 8 * 256 > 0xFFFFFFFFll)
    return PA_ERR_UNSUPPORTED;
  p.maxB = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.log2_bs = pa::log2_exact(block_size);
  p.qk_scale = scale * pa::kPfLog2e;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (dtype == PA_F16) {
    if (head_dim == 64) pa::launch_prefill<pa::F16, 64>(p, num_seqs, st);
    else pa::launch_prefill<pa::F16, 128>(p, num_seqs, st);
  } else {
    if (head_dim == 64) pa::launch_prefill<pa::BF16, 64>(p, num_seqs, st);
    else pa::launch_prefill<pa::BF16, 128>(p, num_seqs, st);
  }
  return pa::launch_status();
}

}  // extern "C"

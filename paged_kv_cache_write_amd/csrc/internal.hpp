// Library-internal entry points shared between translation units.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <vector>

namespace pa {

// Decode work of one call, built on the host (see build_schedule in
// decode.hip): single items and group items of 5 int32 each, members of 2.
struct HostSchedule {
  std::vector<int32_t> items;
  std::vector<int32_t> groups;
  std::vector<int32_t> members;
  int part_tokens = 0;
  int max_ctx = 0;
  size_t ws_bytes = 0;
};

// `tables` (host [S, maxB], may be NULL) enables shared-prefix groups.
// Smallest partition (tokens) that build_schedule uses on its own: the
// automatic size and the shared-prefix partitions never go below it.
int min_schedule_partition_tokens();

int build_schedule(const int32_t* ctx, int32_t S, int32_t H, int32_t D, int32_t bs,
                   int32_t dtype, int32_t requested, const int32_t* tables, int32_t maxB,
                   HostSchedule* hs);

// One launch at the start of an engine step: copy `copy_bytes` (a multiple of
// 16) of staging from pinned host memory (device-visible address `host_src`)
// to `dev_dst`, and write the n new tokens' K/V into the pools with the slots
// read from the host staging `host_slots`.  Returns a pa_status.
int launch_step_prologue(const void* host_src, void* dev_dst, size_t copy_bytes,
                         const int64_t* host_slots, const void* k, const void* v, int64_t n,
                         void* k_cache, void* v_cache, int64_t num_blocks, int32_t num_heads,
                         int32_t head_dim, int32_t block_size, int32_t dtype,
                         hipStream_t stream);

// pa_decode_scheduled (num_group_items == 0) or pa_decode_scheduled_shared,
// with optional HIP events recorded by the dispatch itself at the start of
// the decode's first kernel and the end of its last (no marker packets), and
// counter_rows row counters reserved at the start of the workspace (0: one
// per row of this call; the engine reserves its largest batch's rows, so the
// counters stay in place when the batch grows).
// New tokens that a scheduled decode of single items reads and writes into
// the pool (see DecodeParams): K and V [S, H, D], each row's token being the
// last of its context, and their slots (int64 [S]).
struct NewTokens {
  const void* k = nullptr;
  const void* v = nullptr;
  const int64_t* slots = nullptr;
};

int decode_scheduled_timed(const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks, float scale,
                           int32_t max_context_len, int32_t dtype, void* out, void* workspace,
                           size_t workspace_bytes, int32_t partition_tokens, void* stream,
                           const int32_t* items, int32_t num_items, const int32_t* group_items,
                           int32_t num_group_items, const int32_t* members, hipEvent_t start,
                           hipEvent_t stop, int64_t counter_rows,
                           const NewTokens& new_tokens = NewTokens());

// Device error words of the translation units with kernels (debug builds:
// table entries, slots and copy pairs out of range; release builds: 0), each
// read and cleared.  Synchronous.
uint32_t debug_take_decode();
uint32_t debug_take_prefill();
uint32_t debug_take_cache_ops();

}  // namespace pa

// Host block manager: shared pool, FIFO free list, per-block reference counts,
// per-sequence block tables and copy-on-write planning.  No device memory.
//
// Method (comfyai.app "6.4 PagedAttention" 6.4.1-6.4.3; polomodov.tech
// "vLLM and PagedAttention" slides 10-14):
//   * logical block j of a sequence maps to a physical block of one shared
//     pool; a free block goes to whichever sequence needs it next;
//   * a block is taken only when the previous one is full;
//   * forked sequences share blocks; a block's reference count is the number
//     of table entries that name it;
//   * writing into a shared last block first copies it: the writer gets a new
//     block (count 1), the old block's count drops by one;
//   * preemption by swapping (slide 15): a request's blocks move to a second
//     pool in host memory and back, all or nothing, shared blocks once.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "bm_internal.hpp"
#include "pa.h"

struct SeqState {
  std::vector<int32_t> table;
  int64_t len = 0;
};

struct pa_bm {
  int64_t num_blocks = 0;
  int32_t bs = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, SeqState> seqs;      // resident: tables name GPU blocks
  // host pool for swapped-out sequences (tables name host blocks)
  int64_t num_host = 0;
  std::deque<int32_t> host_free;
  std::vector<int32_t> host_ref;
  std::unordered_map<int64_t, SeqState> swapped;
};

namespace {

bool pop_free(pa_bm* bm, int32_t* out) {
  if (bm->free_list.empty()) return false;
  *out = bm->free_list.front();
  bm->free_list.pop_front();
  bm->ref[*out] = 1;
  return true;
}

using Undo = pa::AppendUndo;

int append_one(pa_bm* bm, int64_t seq, int64_t* slot, int32_t* cow_src,
               int32_t* cow_dst, Undo* undo = nullptr) {
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  SeqState& st = it->second;
  const int64_t t = st.len;
  int copied = 0;
  if (undo) *undo = Undo{seq, 0, -1, -1};
  if (t % bm->bs == 0) {
    int32_t b;
    if (!pop_free(bm, &b)) return PA_ERR_NO_BLOCKS;
    st.table.push_back(b);
    if (undo) *undo = Undo{seq, 1, -1, b};
  } else {
    int32_t last = st.table.back();
    if (bm->ref[last] > 1) {
      int32_t b;
      if (!pop_free(bm, &b)) return PA_ERR_NO_BLOCKS;
      bm->ref[last] -= 1;
      st.table.back() = b;
      if (cow_src) *cow_src = last;
      if (cow_dst) *cow_dst = b;
      if (undo) *undo = Undo{seq, 2, last, b};
      copied = 1;
    }
  }
  if (slot) *slot = int64_t(st.table[t / bm->bs]) * bm->bs + t % bm->bs;
  st.len = t + 1;
  return copied;
}

// Undo appends in reverse order: lengths, tables, refcounts and the free list
// (popped blocks go back to its front) are exactly as before them.
void undo_appends(pa_bm* bm, const std::vector<Undo>& log) {
  for (auto u = log.rbegin(); u != log.rend(); ++u) {
    SeqState& st = bm->seqs.find(u->seq)->second;
    st.len -= 1;
    if (u->kind == 1) {
      st.table.pop_back();
      bm->ref[u->dst] = 0;
      bm->free_list.push_front(u->dst);
    } else if (u->kind == 2) {
      st.table.back() = u->src;
      bm->ref[u->src] += 1;
      bm->ref[u->dst] = 0;
      bm->free_list.push_front(u->dst);
    }
  }
}

void export_row(const SeqState& st, int32_t* row, int32_t width, int32_t pad) {
  const int32_t n = int32_t(st.table.size());
  for (int32_t j = 0; j < width; ++j) row[j] = j < n ? st.table[j] : pad;
}

}  // namespace

extern "C" {

int pa_bm_create(int64_t num_blocks, int32_t block_size,
                 const int32_t* free_order, int64_t num_free, pa_bm** out) {
  if (!out || num_blocks <= 0 || num_blocks > INT32_MAX || block_size <= 0)
    return PA_ERR_INVALID;
  *out = nullptr;
  pa_bm* bm = new (std::nothrow) pa_bm;
  if (!bm) return PA_ERR_INVALID;
  bm->num_blocks = num_blocks;
  bm->bs = block_size;
  bm->ref.assign(size_t(num_blocks), 0);
  if (free_order) {
    if (num_free < 0 || num_free > num_blocks) {
      delete bm;
      return PA_ERR_INVALID;
    }
    std::vector<char> seen(size_t(num_blocks), 0);
    for (int64_t i = 0; i < num_free; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        return PA_ERR_INVALID;
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
  } else {
    for (int64_t b = 0; b < num_blocks; ++b) bm->free_list.push_back(int32_t(b));
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int pa_bm_add_seq(pa_bm* bm, int64_t seq, int64_t num_tokens) {
  if (!bm || num_tokens < 0) return PA_ERR_INVALID;
  if (bm->seqs.count(seq) || bm->swapped.count(seq)) return PA_ERR_EXISTS;
  const int64_t need = (num_tokens + bm->bs - 1) / bm->bs;
  if (need > int64_t(bm->free_list.size())) return PA_ERR_NO_BLOCKS;
  SeqState st;
  st.table.reserve(size_t(need));
  for (int64_t j = 0; j < need; ++j) {
    int32_t b;
    pop_free(bm, &b);
    st.table.push_back(b);
  }
  st.len = num_tokens;
  bm->seqs.emplace(seq, std::move(st));
  return PA_OK;
}

int pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return PA_ERR_INVALID;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  if (bm->seqs.count(child) || bm->swapped.count(child)) return PA_ERR_EXISTS;
  SeqState st = it->second;
  for (int32_t b : st.table) bm->ref[b] += 1;
  bm->seqs.emplace(child, std::move(st));
  return PA_OK;
}

int pa_bm_append_slot(pa_bm* bm, int64_t seq, int64_t* slot, int32_t* cow_src,
                      int32_t* cow_dst) {
  if (!bm) return PA_ERR_INVALID;
  return append_one(bm, seq, slot, cow_src, cow_dst);
}

}  // extern "C"

namespace {

// All or nothing: on failure the appends before the failing one are undone
// and `log` is left empty.
int append_slots_logged(pa_bm* bm, const int64_t* seqs, int32_t n, int64_t* slots,
                        int32_t* cow_pairs, int32_t* num_cow, int32_t* num_done,
                        std::vector<Undo>& log) {
  if (num_done) *num_done = 0;
  if (num_cow) *num_cow = 0;
  log.clear();
  if (!bm || n < 0 || (n > 0 && (!seqs || !slots || !cow_pairs)))
    return PA_ERR_INVALID;
  int32_t ncow = 0;
  log.reserve(size_t(n));
  for (int32_t i = 0; i < n; ++i) {
    int32_t src = -1, dst = -1;
    Undo u;
    int rc = append_one(bm, seqs[i], &slots[i], &src, &dst, &u);
    if (rc < 0) {
      undo_appends(bm, log);
      log.clear();
      return rc;
    }
    log.push_back(u);
    if (rc == 1) {
      cow_pairs[2 * ncow] = src;
      cow_pairs[2 * ncow + 1] = dst;
      ++ncow;
    }
  }
  if (num_cow) *num_cow = ncow;
  if (num_done) *num_done = n;
  return PA_OK;
}

}  // namespace

namespace pa {

int bm_step_logged(pa_bm* bm, const int64_t* seqs, int32_t n, int64_t* slots,
                   int32_t* cow_pairs, int32_t* num_cow, int32_t* tables, int32_t max_blocks,
                   int32_t pad, int32_t* context_lens, std::vector<AppendUndo>* log) {
  int32_t done = 0;
  int rc = append_slots_logged(bm, seqs, n, slots, cow_pairs, num_cow, &done, *log);
  if (rc != PA_OK) return rc;
  rc = pa_bm_block_tables(bm, seqs, n, tables, max_blocks, pad, context_lens);
  if (rc != PA_OK) {  // a table wider than max_blocks: nothing stays changed
    undo_appends(bm, *log);
    log->clear();
  }
  return rc;
}

void bm_undo(pa_bm* bm, const std::vector<AppendUndo>& log) { undo_appends(bm, log); }

}  // namespace pa

extern "C" {

int pa_bm_append_slots(pa_bm* bm, const int64_t* seqs, int32_t n,
                       int64_t* slots, int32_t* cow_pairs, int32_t* num_cow,
                       int32_t* num_done) {
  std::vector<Undo> log;
  return append_slots_logged(bm, seqs, n, slots, cow_pairs, num_cow, num_done, log);
}

int pa_bm_block_tables(const pa_bm* bm, const int64_t* seqs, int32_t n,
                       int32_t* tables, int32_t max_blocks, int32_t pad,
                       int32_t* context_lens) {
  if (!bm || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !tables)))
    return PA_ERR_INVALID;
  int rc = PA_OK;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
    const SeqState& st = it->second;
    if (int64_t(st.table.size()) > max_blocks) rc = PA_ERR_CAPACITY;
    export_row(st, tables + int64_t(i) * max_blocks, max_blocks, pad);
    if (context_lens) context_lens[i] = int32_t(st.len);
  }
  return rc;
}

int pa_bm_step(pa_bm* bm, const int64_t* seqs, int32_t n, int64_t* slots,
               int32_t* cow_pairs, int32_t* num_cow, int32_t* tables,
               int32_t max_blocks, int32_t pad, int32_t* context_lens) {
  std::vector<Undo> log;
  return pa::bm_step_logged(bm, seqs, n, slots, cow_pairs, num_cow, tables, max_blocks, pad,
                            context_lens, &log);
}

int pa_bm_select(pa_bm* bm, const int64_t* parents, const int64_t* children, int32_t n,
                 const int64_t* retire, int32_t m) {
  if (!bm || n < 0 || m < 0 || (n > 0 && (!parents || !children)) || (m > 0 && !retire))
    return PA_ERR_INVALID;
  // every check before any change: parents exist, children are new and
  // distinct, retired sequences exist and are distinct
  std::unordered_map<int64_t, int> seen;
  for (int32_t i = 0; i < n; ++i) {
    if (!bm->seqs.count(parents[i])) return PA_ERR_NOT_FOUND;
    if (bm->seqs.count(children[i]) || bm->swapped.count(children[i]) ||
        !seen.emplace(children[i], 1).second)
      return PA_ERR_EXISTS;
  }
  std::unordered_map<int64_t, int> gone;
  for (int32_t j = 0; j < m; ++j) {
    if (!bm->seqs.count(retire[j])) return PA_ERR_NOT_FOUND;
    if (!gone.emplace(retire[j], 1).second) return PA_ERR_INVALID;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int rc = pa_bm_fork(bm, parents[i], children[i]);
    if (rc != PA_OK) return rc;  // cannot happen after the checks
  }
  for (int32_t j = 0; j < m; ++j) {
    const int rc = pa_bm_free_seq(bm, retire[j]);
    if (rc != PA_OK) return rc;
  }
  return PA_OK;
}

int pa_bm_free_seq(pa_bm* bm, int64_t seq) {
  if (!bm) return PA_ERR_INVALID;
  auto sw = bm->swapped.find(seq);
  if (sw != bm->swapped.end()) {  // a swapped-out sequence releases host blocks
    for (int32_t b : sw->second.table) {
      bm->host_ref[b] -= 1;
      if (bm->host_ref[b] == 0) bm->host_free.push_back(b);
    }
    bm->swapped.erase(sw);
    return PA_OK;
  }
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  for (int32_t b : it->second.table) {
    bm->ref[b] -= 1;
    if (bm->ref[b] == 0) bm->free_list.push_back(b);
  }
  bm->seqs.erase(it);
  return PA_OK;
}

int pa_bm_slots(const pa_bm* bm, int64_t seq, int64_t start, int64_t n,
                int64_t* out) {
  if (!bm || start < 0 || n < 0 || (n > 0 && !out)) return PA_ERR_INVALID;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
  const SeqState& st = it->second;
  if (start + n > st.len) return PA_ERR_INVALID;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t t = start + i;
    out[i] = int64_t(st.table[t / bm->bs]) * bm->bs + t % bm->bs;
  }
  return PA_OK;
}

int pa_bm_block_table(const pa_bm* bm, int64_t seq, int32_t* out, int32_t cap,
                      int32_t* n) {
  if (!bm || cap < 0 || (cap > 0 && !out)) return PA_ERR_INVALID;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) {
    it = bm->swapped.find(seq);  // a swapped-out sequence: host block ids
    if (it == bm->swapped.end()) return PA_ERR_NOT_FOUND;
  }
  const auto& tab = it->second.table;
  if (n) *n = int32_t(tab.size());
  if (int64_t(tab.size()) > cap) return PA_ERR_CAPACITY;
  if (!tab.empty()) std::memcpy(out, tab.data(), tab.size() * sizeof(int32_t));
  return PA_OK;
}

int64_t pa_bm_seq_len(const pa_bm* bm, int64_t seq) {
  if (!bm) return PA_ERR_INVALID;
  auto it = bm->seqs.find(seq);
  if (it != bm->seqs.end()) return it->second.len;
  it = bm->swapped.find(seq);  // a swapped-out sequence keeps its length
  return it == bm->swapped.end() ? int64_t(PA_ERR_NOT_FOUND) : it->second.len;
}

int32_t pa_bm_refcount(const pa_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return PA_ERR_INVALID;
  return bm->ref[block];
}

int64_t pa_bm_num_free(const pa_bm* bm) {
  return bm ? int64_t(bm->free_list.size()) : int64_t(PA_ERR_INVALID);
}

int64_t pa_bm_num_seqs(const pa_bm* bm) {
  return bm ? int64_t(bm->seqs.size() + bm->swapped.size()) : int64_t(PA_ERR_INVALID);
}

int pa_bm_set_host_pool(pa_bm* bm, int64_t num_host_blocks, const int32_t* free_order,
                        int64_t num_free) {
  if (!bm || num_host_blocks < 0 || num_host_blocks > INT32_MAX || !bm->swapped.empty())
    return PA_ERR_INVALID;
  std::deque<int32_t> fl;
  if (free_order) {
    if (num_free < 0 || num_free > num_host_blocks) return PA_ERR_INVALID;
    std::vector<char> seen(size_t(num_host_blocks), 0);
    for (int64_t i = 0; i < num_free; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_host_blocks || seen[b]) return PA_ERR_INVALID;
      seen[b] = 1;
      fl.push_back(b);
    }
  } else {
    for (int64_t b = 0; b < num_host_blocks; ++b) fl.push_back(int32_t(b));
  }
  bm->num_host = num_host_blocks;
  bm->host_free = std::move(fl);
  bm->host_ref.assign(size_t(num_host_blocks), 0);
  return PA_OK;
}

namespace {

// Move the tables of `seqs` (distinct, all in `from`) to the other pool, all
// or nothing.  Every block they name must be held by them alone (its
// reference count equals the number of their references): a group that
// shares blocks moves as a whole.  Each distinct block gets one block of the
// destination pool (taken from the front of its free list in first-use
// order: sequences in the order given, logical blocks in order) with the same
// reference count; the source block returns to the back of its free list.
// pairs[2i], pairs[2i+1] = (source block, destination block).
int move_seqs(std::unordered_map<int64_t, SeqState>& from,
              std::unordered_map<int64_t, SeqState>& to, std::vector<int32_t>& src_ref,
              std::deque<int32_t>& src_free, std::vector<int32_t>& dst_ref,
              std::deque<int32_t>& dst_free, const int64_t* seqs, int32_t n, int32_t* pairs,
              int32_t cap, int32_t* num_pairs) {
  if (num_pairs) *num_pairs = 0;
  if (n <= 0 || !seqs || cap < 0 || (cap > 0 && !pairs)) return PA_ERR_INVALID;
  std::unordered_map<int64_t, int> seen;
  std::unordered_map<int32_t, int32_t> uses;  // block -> references from the set
  std::vector<int32_t> order;
  for (int32_t i = 0; i < n; ++i) {
    if (!seen.emplace(seqs[i], 1).second) return PA_ERR_INVALID;
    auto it = from.find(seqs[i]);
    if (it == from.end()) return PA_ERR_NOT_FOUND;
    for (int32_t b : it->second.table)
      if (uses[b]++ == 0) order.push_back(b);
  }
  for (int32_t b : order)
    if (uses[b] != src_ref[b]) return PA_ERR_INVALID;  // shared with a sequence outside
  const int32_t d = int32_t(order.size());
  if (num_pairs) *num_pairs = d;
  if (size_t(d) > dst_free.size()) return PA_ERR_NO_BLOCKS;
  if (d > cap) return PA_ERR_CAPACITY;
  std::unordered_map<int32_t, int32_t> map;
  for (int32_t k = 0; k < d; ++k) {
    const int32_t b = order[k];
    const int32_t nb = dst_free.front();
    dst_free.pop_front();
    dst_ref[nb] = src_ref[b];
    src_ref[b] = 0;
    src_free.push_back(b);
    map[b] = nb;
    pairs[2 * k] = b;
    pairs[2 * k + 1] = nb;
  }
  for (int32_t i = 0; i < n; ++i) {
    auto it = from.find(seqs[i]);
    SeqState st = std::move(it->second);
    from.erase(it);
    for (auto& b : st.table) b = map[b];
    to.emplace(seqs[i], std::move(st));
  }
  return PA_OK;
}

}  // namespace

int pa_bm_swap_out(pa_bm* bm, const int64_t* seqs, int32_t n, int32_t* pairs, int32_t cap,
                   int32_t* num_pairs) {
  if (!bm) return PA_ERR_INVALID;
  return move_seqs(bm->seqs, bm->swapped, bm->ref, bm->free_list, bm->host_ref, bm->host_free,
                   seqs, n, pairs, cap, num_pairs);
}

int pa_bm_swap_in(pa_bm* bm, const int64_t* seqs, int32_t n, int32_t* pairs, int32_t cap,
                  int32_t* num_pairs) {
  if (!bm) return PA_ERR_INVALID;
  return move_seqs(bm->swapped, bm->seqs, bm->host_ref, bm->host_free, bm->ref, bm->free_list,
                   seqs, n, pairs, cap, num_pairs);
}

int pa_bm_is_swapped(const pa_bm* bm, int64_t seq) {
  if (!bm) return PA_ERR_INVALID;
  if (bm->swapped.count(seq)) return 1;
  return bm->seqs.count(seq) ? 0 : PA_ERR_NOT_FOUND;
}

int64_t pa_bm_num_free_host(const pa_bm* bm) {
  return bm ? int64_t(bm->host_free.size()) : int64_t(PA_ERR_INVALID);
}

int64_t pa_bm_host_free_list(const pa_bm* bm, int32_t* out, int64_t cap) {
  if (!bm) return PA_ERR_INVALID;
  const int64_t n = int64_t(bm->host_free.size());
  if (out)
    for (int64_t i = 0; i < std::min(n, cap); ++i) out[i] = bm->host_free[size_t(i)];
  return n;
}

int32_t pa_bm_host_refcount(const pa_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_host) return PA_ERR_INVALID;
  return bm->host_ref[size_t(block)];
}

int64_t pa_bm_blocks_needed(const pa_bm* bm, const int64_t* seqs, int32_t n) {
  // the appends of pa_bm_append_slots(seqs) simulated without the pool: a
  // new block at a block boundary, a copy when the last block is shared
  if (!bm || n < 0 || (n > 0 && !seqs)) return PA_ERR_INVALID;
  std::unordered_map<int64_t, int64_t> len;
  std::unordered_map<int64_t, int> own_last;      // last block private after a copy/new block
  std::unordered_map<int32_t, int32_t> ref_drop;  // references moved off a block by copies
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PA_ERR_NOT_FOUND;
    const SeqState& st = it->second;
    auto ins = len.emplace(seqs[i], st.len);
    int64_t& t = ins.first->second;
    if (t % bm->bs == 0) {
      ++need;
      own_last[seqs[i]] = 1;
    } else if (!own_last[seqs[i]]) {
      const int32_t last = st.table.back();
      if (bm->ref[last] - ref_drop[last] > 1) {
        ++need;
        ref_drop[last] += 1;
      }
      own_last[seqs[i]] = 1;  // private now (copied, or the last holder)
    }
    t += 1;
  }
  return need;
}

int64_t pa_bm_free_list(const pa_bm* bm, int32_t* out, int64_t cap) {
  if (!bm || cap < 0 || (cap > 0 && !out)) return PA_ERR_INVALID;
  int64_t i = 0;
  for (int32_t b : bm->free_list) {
    if (i < cap) out[i] = b;
    ++i;
  }
  return i;
}

}  // extern "C"

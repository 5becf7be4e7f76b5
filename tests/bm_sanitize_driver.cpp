// Randomised workload for the host block manager, built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_block_manager_sanitize.py (CPU
// only).  Every pa_bm_* call of the C ABI runs many times, successes and
// failures alike, and after each operation the pool's invariants are checked
// through the ABI alone: a block's reference count equals the number of
// table entries naming it, free + referenced blocks = the pool, a failed
// call changes nothing, and blocks_needed predicts what an append takes.
// Engine steps are also undone through the library-internal undo log (what
// the engine does when a launch after the appends fails): the state,
// free-list order included, must be exactly as before.
// Exit status 0 = all checks held (the sanitizers abort on any memory or UB
// error).
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <string>
#include <vector>

#include "bm_internal.hpp"
#include "pa.h"

namespace {

constexpr int32_t kTableCap = 128;  // > the longest table the pool allows
constexpr size_t kMaxLive = 40;     // forks take no blocks: bound the population

int fail(const char* what, long step) {
  std::fprintf(stderr, "invariant failed at op %ld: %s\n", step, what);
  std::exit(1);
}

struct Snapshot {
  int64_t free_dev = 0, free_host = 0, seqs = 0;
  std::map<int64_t, std::vector<int32_t>> tables;
  std::map<int64_t, int64_t> lens;
  std::vector<int32_t> free_list;
  bool operator==(const Snapshot& o) const {
    return free_dev == o.free_dev && free_host == o.free_host && seqs == o.seqs &&
           tables == o.tables && lens == o.lens && free_list == o.free_list;
  }
};

Snapshot snap(pa_bm* bm, const std::set<int64_t>& live) {
  Snapshot s;
  s.free_dev = pa_bm_num_free(bm);
  s.free_host = pa_bm_num_free_host(bm);
  s.seqs = pa_bm_num_seqs(bm);
  s.free_list.resize(size_t(s.free_dev) + 1);
  s.free_list.resize(size_t(pa_bm_free_list(bm, s.free_list.data(), int64_t(s.free_list.size()))));
  for (int64_t q : live) {
    int32_t n = 0;
    std::vector<int32_t> t(kTableCap);
    if (pa_bm_block_table(bm, q, t.data(), int32_t(t.size()), &n) != PA_OK) fail("table", -1);
    t.resize(size_t(n));
    s.tables[q] = t;
    s.lens[q] = pa_bm_seq_len(bm, q);
  }
  return s;
}

void check(pa_bm* bm, const std::set<int64_t>& live, int64_t NB, int64_t NH, int32_t bs,
           long step) {
  std::map<int32_t, int64_t> dev_refs, host_refs;
  for (int64_t q : live) {
    int32_t n = 0;
    std::vector<int32_t> t(kTableCap);
    if (pa_bm_block_table(bm, q, t.data(), int32_t(t.size()), &n) != PA_OK) fail("table", step);
    const int64_t len = pa_bm_seq_len(bm, q);
    if (len < 0 || n != (len + bs - 1) / bs) fail("table length", step);
    const bool swapped = pa_bm_is_swapped(bm, q) == 1;
    for (int i = 0; i < n; ++i) (swapped ? host_refs : dev_refs)[t[size_t(i)]]++;
  }
  if (pa_bm_num_seqs(bm) != int64_t(live.size())) fail("sequence count", step);
  for (auto& kv : dev_refs) {
    if (kv.first < 0 || kv.first >= NB) fail("device block id", step);
    if (pa_bm_refcount(bm, kv.first) != kv.second) fail("device refcount", step);
  }
  for (auto& kv : host_refs) {
    if (kv.first < 0 || kv.first >= NH) fail("host block id", step);
    if (pa_bm_host_refcount(bm, kv.first) != kv.second) fail("host refcount", step);
  }
  if (pa_bm_num_free(bm) + int64_t(dev_refs.size()) != NB) fail("device free + used", step);
  if (pa_bm_num_free_host(bm) + int64_t(host_refs.size()) != NH) fail("host free + used", step);
  std::vector<int32_t> fl(size_t(NB) + 1);
  const int64_t nf = pa_bm_free_list(bm, fl.data(), int64_t(fl.size()));
  std::set<int32_t> seen;
  for (int64_t i = 0; i < nf; ++i) {
    if (dev_refs.count(fl[size_t(i)]) || !seen.insert(fl[size_t(i)]).second)
      fail("free list", step);
  }
}

}  // namespace

int main(int argc, char** argv) {
  const long steps = argc > 1 ? std::atol(argv[1]) : 20000;
  const int32_t bs = 8;
  const int64_t NB = 96, NH = 64;
  std::mt19937_64 rng(20251203);
  auto pick = [&](int64_t n) { return int64_t(rng() % uint64_t(n)); };
  std::vector<int32_t> order(static_cast<size_t>(NB));
  for (int64_t i = 0; i < NB; ++i) order[size_t(i)] = int32_t((i * 37) % NB);
  pa_bm* bm = nullptr;
  if (pa_bm_create(NB, bs, order.data(), NB, &bm) != PA_OK) return fail("create", 0);
  if (pa_bm_set_host_pool(bm, NH, nullptr, 0) != PA_OK) return fail("host pool", 0);
  std::set<int64_t> live;  // resident and swapped
  std::map<std::string, long> seen;  // outcomes exercised
  int64_t next_id = 1;
  auto any_live = [&](bool want_swapped) -> int64_t {
    std::vector<int64_t> c;
    for (int64_t q : live)
      if ((pa_bm_is_swapped(bm, q) == 1) == want_swapped) c.push_back(q);
    return c.empty() ? -1 : c[size_t(pick(int64_t(c.size())))];
  };
  for (long step = 0; step < steps; ++step) {
    const Snapshot before = snap(bm, live);
    const int op = int(pick(10));
    int rc = PA_OK;
    bool changed = true;
    if (op == 0 || live.size() < 2) {  // add
      const int64_t id = next_id++;
      rc = pa_bm_add_seq(bm, id, 1 + pick(60));
      seen[rc == PA_OK ? "add" : "add_full"]++;
      if (rc == PA_OK) live.insert(id);
      else if (rc != PA_ERR_NO_BLOCKS) fail("add status", step);
    } else if (op == 1) {  // fork
      const int64_t p = live.size() < kMaxLive ? any_live(false) : -1;
      if (p >= 0) {
        const int64_t id = next_id++;
        rc = pa_bm_fork(bm, p, id);
        if (rc != PA_OK) fail("fork", step);
        seen["fork"]++;
        live.insert(id);
      }
    } else if (op == 2 || op == 3) {  // batch append (sequences may repeat)
      std::vector<int64_t> seqs;
      for (int i = 0, n = int(1 + pick(6)); i < n; ++i) {
        const int64_t q = any_live(false);
        if (q >= 0) seqs.push_back(q);
      }
      if (!seqs.empty()) {
        const int64_t need = pa_bm_blocks_needed(bm, seqs.data(), int32_t(seqs.size()));
        std::vector<int64_t> slots(seqs.size());
        std::vector<int32_t> cow(2 * seqs.size());
        int32_t ncow = -1, done = -1;
        rc = pa_bm_append_slots(bm, seqs.data(), int32_t(seqs.size()), slots.data(), cow.data(),
                                &ncow, &done);
        if (rc == PA_OK) {
          seen[ncow > 0 ? "append_cow" : "append"]++;
          if (before.free_dev - pa_bm_num_free(bm) != need) fail("blocks_needed", step);
          if (done != int32_t(seqs.size())) fail("num_done", step);
          for (size_t i = 0; i < seqs.size(); ++i)
            if (slots[i] < 0 || slots[i] >= NB * bs) fail("slot range", step);
        } else if (rc == PA_ERR_NO_BLOCKS) {
          seen["append_full"]++;
          if (need <= before.free_dev) fail("blocks_needed vs failure", step);
          changed = false;
        } else {
          fail("append status", step);
        }
      }
    } else if (op == 4) {  // free (resident or swapped)
      if (!live.empty()) {
        auto it = live.begin();
        std::advance(it, pick(int64_t(live.size())));
        seen[pa_bm_is_swapped(bm, *it) == 1 ? "free_swapped" : "free"]++;
        if (pa_bm_free_seq(bm, *it) != PA_OK) fail("free", step);
        live.erase(it);
      }
    } else if (op == 5) {  // beam selection: children of repeated parents, retire some
      std::vector<int64_t> parents, children, retire;
      const int64_t p = live.size() < kMaxLive ? any_live(false) : -1;
      if (p >= 0) {
        for (int i = 0, n = int(1 + pick(3)); i < n; ++i) {
          parents.push_back(p);
          children.push_back(next_id++);
        }
        if (pick(2)) retire.push_back(p);
        rc = pa_bm_select(bm, parents.data(), children.data(), int32_t(parents.size()),
                          retire.data(), int32_t(retire.size()));
        if (rc != PA_OK) fail("select", step);
        seen["select"]++;
        for (int64_t c : children) live.insert(c);
        for (int64_t r : retire) live.erase(r);
      }
    } else if (op == 6) {  // swap out one sequence (fails unless it holds its blocks alone)
      const int64_t q = any_live(false);
      if (q >= 0) {
        std::vector<int32_t> pairs(2 * kTableCap);
        int32_t np = -1;
        rc = pa_bm_swap_out(bm, &q, 1, pairs.data(), kTableCap, &np);
        seen[rc == PA_OK ? "swap_out" : "swap_out_refused"]++;
        if (rc == PA_OK) {
          for (int32_t i = 0; i < np; ++i)
            if (pairs[size_t(2 * i)] >= NB || pairs[size_t(2 * i + 1)] >= NH) fail("pair", step);
        } else if (rc == PA_ERR_INVALID || rc == PA_ERR_NO_BLOCKS) {
          changed = false;
        } else {
          fail("swap out status", step);
        }
      }
    } else if (op == 7) {  // swap in
      const int64_t q = any_live(true);
      if (q >= 0) {
        std::vector<int32_t> pairs(2 * kTableCap);
        int32_t np = -1;
        rc = pa_bm_swap_in(bm, &q, 1, pairs.data(), kTableCap, &np);
        seen[rc == PA_OK ? "swap_in" : "swap_in_full"]++;
        if (rc == PA_ERR_NO_BLOCKS) changed = false;
        else if (rc != PA_OK) fail("swap in status", step);
      }
    } else if (op == 8) {  // error paths change nothing
      int64_t slot = 0;
      int32_t a = 0, b = 0, n = 0;
      int32_t small[1];
      if (pa_bm_append_slot(bm, -5, &slot, &a, &b) != PA_ERR_NOT_FOUND) fail("unknown", step);
      if (pa_bm_fork(bm, -5, next_id) != PA_ERR_NOT_FOUND) fail("fork unknown", step);
      const int64_t q = any_live(false);
      if (q >= 0 && pa_bm_add_seq(bm, q, 3) != PA_ERR_EXISTS) fail("exists", step);
      if (q >= 0 && pa_bm_seq_len(bm, q) > bs &&
          pa_bm_block_table(bm, q, small, 1, &n) != PA_ERR_CAPACITY)
        fail("capacity", step);
      changed = false;
    } else {  // engine-style step over every resident sequence
      std::vector<int64_t> seqs;
      for (int64_t q : live)
        if (pa_bm_is_swapped(bm, q) == 0) seqs.push_back(q);
      if (!seqs.empty()) {
        std::vector<int64_t> slots(seqs.size());
        std::vector<int32_t> cow(2 * seqs.size()), tables(seqs.size() * kTableCap),
            lens(seqs.size());
        int32_t ncow = 0;
        const int kind = int(pick(4));
        if (kind == 0) {  // a step whose later launch fails: the engine undoes it
          std::vector<pa::AppendUndo> log;
          rc = pa::bm_step_logged(bm, seqs.data(), int32_t(seqs.size()), slots.data(), cow.data(),
                                  &ncow, tables.data(), kTableCap, -1, lens.data(), &log);
          if (rc == PA_OK) {
            if (log.size() != seqs.size()) fail("undo log length", step);
            pa::bm_undo(bm, log);
            seen["step_undone"]++;
          } else if (rc == PA_ERR_NO_BLOCKS) {
            if (!log.empty()) fail("log of a failed step", step);
            seen["step_full"]++;
          } else {
            fail("logged step status", step);
          }
          changed = false;
        } else if (kind == 1) {  // tables wider than the caller's rows: nothing changes
          rc = pa_bm_step(bm, seqs.data(), int32_t(seqs.size()), slots.data(), cow.data(), &ncow,
                          tables.data(), 1, -1, lens.data());
          int64_t longest = 0;
          for (int64_t q : seqs) longest = std::max(longest, pa_bm_seq_len(bm, q));
          if (rc == PA_ERR_CAPACITY) seen["step_capacity"]++;
          else if (rc == PA_OK && longest <= bs) seen["step"]++;
          else if (rc == PA_OK || rc != PA_ERR_NO_BLOCKS) fail("narrow step status", step);
          changed = rc != PA_OK ? false : true;
        } else {
          rc = pa_bm_step(bm, seqs.data(), int32_t(seqs.size()), slots.data(), cow.data(), &ncow,
                          tables.data(), kTableCap, -1, lens.data());
          seen[rc == PA_OK ? "step" : "step_full"]++;
          if (rc == PA_ERR_NO_BLOCKS) changed = false;
          else if (rc != PA_OK) fail("step status", step);
        }
      }
    }
    if (!changed && !(snap(bm, live) == before)) fail("a failed call changed the state", step);
    check(bm, live, NB, NH, bs, step);
  }
  pa_bm_destroy(bm);
  std::printf("ok %ld operations\n", steps);
  for (auto& kv : seen) std::printf("%s %ld\n", kv.first.c_str(), kv.second);
  return 0;
}

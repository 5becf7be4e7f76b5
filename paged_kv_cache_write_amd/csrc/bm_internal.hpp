// Block-manager calls used by the engine step (library-internal; host only).
#pragma once

#include <stdint.h>

#include <vector>

#include "pa.h"

namespace pa {

// What one append did, for undoing it: kind 0 in place, 1 a new block (dst),
// 2 a copy on write (src -> dst).
struct AppendUndo {
  int64_t seq;
  int kind;
  int32_t src, dst;
};

// pa_bm_step that also returns the log of the appends it made (cleared
// first; empty when it fails: a failed step changes nothing).
int bm_step_logged(pa_bm* bm, const int64_t* seqs, int32_t n, int64_t* slots,
                   int32_t* cow_pairs, int32_t* num_cow, int32_t* tables, int32_t max_blocks,
                   int32_t pad, int32_t* context_lens, std::vector<AppendUndo>* log);

// Undo a logged step: lengths, tables, reference counts and the free list are
// exactly as before it.  The log must be the manager's most recent change.
void bm_undo(pa_bm* bm, const std::vector<AppendUndo>& log);

}  // namespace pa

// One decode engine step in native code: host slot assignment, schedule,
// table shipment, copy-on-write copies, slot-mapped cache write and
// scheduled PagedAttention decode, all enqueued on the caller's stream.
//
// The step is the serving loop of the pages: the scheduler's block manager
// gives each running sequence the slot of its new token (a new block when
// the last is full, a copy when it is shared; comfyai.app "6.4 PagedAttention"
// 6.4.3, polomodov.tech "vLLM and PagedAttention" slides 11-13), and the
// block tables travel to the GPU workers every step (slide 16).
//
// Staging: the caller gives `ring` pinned host slots and one device slot of
// pa_engine_staging_bytes() each.  A step fills host slot i (slots, context
// lengths, CoW pairs, block tables, work items); the step prologue kernel
// reads exactly the used bytes from the mapped host slot into the device slot
// (or one hipMemcpyAsync does, where the host memory is not mapped).  Events
// guard the host slots in groups: with an even ring the slots form two halves
// and one event is recorded after the last step of each half, so a marker
// packet sits between only every ring/2-th pair of steps; a host slot is
// rewritten only after the event of its group.  The device slot is reused in
// stream order.
//
// Where the device's memory is mapped for the host (a large PCIe BAR), the
// engine also keeps `ring` slots of uncached device memory: the host copies
// the used bytes of its slot straight into the matching device slot, so no
// kernel reads host memory, and a step without copies on write is one
// launch: the decode, whose wave of each row's last partition reads the new
// token from k_new / v_new while extra workgroups of the launch write the
// tokens into their slots.  The device slots follow the host slots' guard
// events.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "bm_internal.hpp"
#include "internal.hpp"
#include "pa.h"

struct pa_engine {
  pa_bm* bm = nullptr;
  void* k_cache = nullptr;
  void* v_cache = nullptr;
  int64_t num_blocks = 0;
  int32_t H = 0, D = 0, bs = 0, dtype = 0;
  int32_t max_batch = 0, max_blocks = 0, pad = 0;
  char* host = nullptr;
  char* host_dev = nullptr;  // device-visible address of `host` (NULL: use hipMemcpyAsync)
  char* dev = nullptr;
  char* mapped = nullptr;     // ring slots of host-written device memory (NULL: none)
  bool use_mapped = true;     // steps use `mapped` when present
  size_t slot_bytes = 0;
  int32_t ring = 0, next = 0;
  int32_t group = 1;       // host slots per guarding event (the event sits on the group's last)
  bool unguarded = false;  // steps enqueued since the last recorded guard event
  std::vector<hipEvent_t> events;
  std::vector<char> pending;
  std::vector<int32_t> ctx_pre;
  hipEvent_t ev_start = nullptr, ev_end = nullptr;  // optional: the decode kernel's start / end
  bool sharing = true;  // detect shared prefixes in the tables each step
  pa::HostSchedule hs;
  std::vector<pa::AppendUndo> undo;  // the block manager's appends of the current step
  std::vector<char> covered;         // rows whose last token lies in a single item
};

namespace {

// Work items (5 int32 each) are bounded by one per 32 tokens (the smallest
// partition) plus one per sequence, for single and for group items; members
// (2 int32) by one per sequence.
int64_t item_ints(int32_t max_batch, int32_t max_blocks, int32_t bs) {
  const int64_t tokens = int64_t(max_blocks) * bs;
  return 2 * 5 * int64_t(max_batch) * ((tokens + 31) / 32 + 1) + 2 * int64_t(max_batch);
}

size_t align16(size_t x) { return (x + 15) & ~size_t(15); }

// Uncached device memory that the host writes through the BAR mapping.  The
// device reads it from memory every time (no cache holds a line of it), so a
// slot the host rewrites is never read stale.  Once a kernel has read such
// memory it is not returned to the runtime: chunks are kept for the life of
// the process and reused, smallest fit first, by later engines of the same
// device.
struct MappedChunk {
  int device;
  char* ptr;
  size_t bytes;
  bool used;
};
std::mutex g_mapped_mu;
std::vector<MappedChunk> g_mapped;

// Whether [p, p + bytes) is covered by readable and writable mappings of
// this process without a gap (/proc/self/maps lists them in address order).
bool host_mapped_rw(const void* p, size_t bytes) {
  std::FILE* f = std::fopen("/proc/self/maps", "r");
  if (!f) return false;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p), hi = lo + bytes;
  uintptr_t covered = lo;  // [lo, covered) is known to be mapped rw
  char line[512];
  while (covered < hi && std::fgets(line, sizeof(line), f)) {
    unsigned long a = 0, b = 0;
    char perm[8] = {0};
    if (std::sscanf(line, "%lx-%lx %7s", &a, &b, perm) != 3 || b <= covered) continue;
    if (a > covered || perm[0] != 'r' || perm[1] != 'w') break;  // a gap, or not rw
    covered = b;
  }
  std::fclose(f);
  return covered >= hi;
}

char* mapped_take(int device, size_t bytes) {
  std::lock_guard<std::mutex> lock(g_mapped_mu);
  MappedChunk* best = nullptr;
  for (auto& c : g_mapped)
    if (!c.used && c.device == device && c.bytes >= bytes && (!best || c.bytes < best->bytes))
      best = &c;
  if (best) {
    best->used = true;
    return best->ptr;
  }
  int large_bar = 0;
  if (hipDeviceGetAttribute(&large_bar, hipDeviceAttributeIsLargeBar, device) != hipSuccess ||
      !large_bar) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = nullptr;
  if (hipExtMallocWithFlags(&p, bytes, hipDeviceMallocUncached) != hipSuccess || !p) {
    (void)hipGetLastError();
    return nullptr;
  }
  // The host writes the chunk at the device address: that range must be a
  // readable and writable mapping of this process.  Otherwise the chunk is
  // returned (no kernel has read it yet) and the engine keeps its prologue.
  if (size_t(p) % 16 || !host_mapped_rw(p, bytes)) {
    (void)hipFree(p);
    (void)hipGetLastError();
    return nullptr;
  }
  g_mapped.push_back({device, static_cast<char*>(p), bytes, true});
  return static_cast<char*>(p);
}

void mapped_give(char* p) {
  std::lock_guard<std::mutex> lock(g_mapped_mu);
  for (auto& c : g_mapped)
    if (c.ptr == p) c.used = false;
}

// Copy the used staging bytes into a mapped device slot so that the next
// launch sees them: the fence drains the CPU's write-combining buffers, and
// the read of the last word, which travels behind the writes over the link,
// returns only once they have reached the device.
void mapped_publish(char* dst, const char* src, size_t used) {
  std::memcpy(dst, src, used);
  std::atomic_thread_fence(std::memory_order_seq_cst);
  (void)*reinterpret_cast<volatile const uint32_t*>(dst + used - 4);
}

}  // namespace

extern "C" {

size_t pa_engine_staging_bytes(int32_t max_batch, int32_t max_blocks_per_seq,
                               int32_t block_size) {
  if (max_batch <= 0 || max_blocks_per_seq <= 0 || block_size <= 0) return 0;
  const size_t B = size_t(max_batch);
  return align16(8 * B + 4 * B + 8 * B + 4 * B * size_t(max_blocks_per_seq) +
                4 * size_t(item_ints(max_batch, max_blocks_per_seq, block_size)));
}

int pa_engine_create(pa_bm* bm, void* k_cache, void* v_cache, int64_t num_blocks,
                     int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                     int32_t max_batch, int32_t max_blocks_per_seq, int32_t pad_block,
                     void* host_staging, int32_t ring, void* dev_staging, pa_engine** out) {
  if (!out) return PA_ERR_INVALID;
  *out = nullptr;
  if (!bm || !k_cache || !v_cache || !host_staging || !dev_staging || ring <= 0 ||
      num_blocks <= 0 || num_heads <= 0 || max_batch <= 0 || max_blocks_per_seq <= 0)
    return PA_ERR_INVALID;
  // the decode and the step prologue launch at most 65535 sequences
  if (max_batch > 65535) return PA_ERR_UNSUPPORTED;
  if (size_t(host_staging) % 16 || size_t(dev_staging) % 16) return PA_ERR_INVALID;
  size_t ws;
  int rc = pa_decode_plan(1, num_heads, head_dim, block_size, 0, dtype, 0, nullptr, nullptr, &ws);
  if (rc != PA_OK) return rc;
  pa_engine* e = new (std::nothrow) pa_engine;
  if (!e) return PA_ERR_INVALID;
  e->bm = bm;
  e->k_cache = k_cache;
  e->v_cache = v_cache;
  e->num_blocks = num_blocks;
  e->H = num_heads;
  e->D = head_dim;
  e->bs = block_size;
  e->dtype = dtype;
  e->max_batch = max_batch;
  e->max_blocks = max_blocks_per_seq;
  e->pad = pad_block;
  e->host = static_cast<char*>(host_staging);
  e->dev = static_cast<char*>(dev_staging);
  e->slot_bytes = pa_engine_staging_bytes(max_batch, max_blocks_per_seq, block_size);
  e->ring = ring;
  e->group = (ring % 2 == 0) ? ring / 2 : 1;
  {
    // Pinned host memory is mapped for the device: the step prologue kernel
    // reads the staging straight from it instead of a DMA copy.
    void* dptr = nullptr;
    if (hipHostGetDevicePointer(&dptr, host_staging, 0) == hipSuccess && dptr &&
        size_t(dptr) % 16 == 0 && size_t(host_staging) % 16 == 0)
      e->host_dev = static_cast<char*>(dptr);
    else
      (void)hipGetLastError();
  }
  {
    int device = 0;
    if (hipGetDevice(&device) == hipSuccess)
      e->mapped = mapped_take(device, e->slot_bytes * size_t(ring));
    else
      (void)hipGetLastError();
  }
  e->events.assign(size_t(ring), nullptr);
  e->pending.assign(size_t(ring), 0);
  // The ring events only order work (the host waits on one before it reuses a
  // staging slot the GPU has read): no timing, and no system-scope fence
  // (which would write back and invalidate the caches at every record).
  const unsigned order_only = hipEventDisableTiming | hipEventDisableSystemFence;
  for (auto& ev : e->events) {
    if (hipEventCreateWithFlags(&ev, order_only) != hipSuccess) {
      pa_engine_destroy(e);
      return PA_ERR_HIP;
    }
  }
  *out = e;
  return PA_OK;
}

void pa_engine_destroy(pa_engine* e) {
  if (!e) return;
  // steps after the last guard event may still read the host staging, which
  // the caller frees after this call
  if (e->unguarded) (void)hipDeviceSynchronize();
  for (size_t i = 0; i < e->events.size(); ++i) {
    if (e->events[i]) {
      if (e->pending[i]) (void)hipEventSynchronize(e->events[i]);
      (void)hipEventDestroy(e->events[i]);
    }
  }
  if (e->mapped) mapped_give(e->mapped);  // no step that reads it is pending
  delete e;
}

size_t pa_engine_workspace_bytes(const pa_engine* e, int32_t partition_tokens) {
  if (!e) return size_t(-1);
  // the schedule's own partitions (automatic and shared-prefix) never go
  // below this size; an explicit smaller size is used as given
  const int32_t floor_pt = pa::min_schedule_partition_tokens();
  int32_t pt = partition_tokens == 0 ? floor_pt : std::min<int32_t>(partition_tokens, floor_pt);
  return pa_decode_workspace_size(e->max_batch, e->H, e->D, e->bs, e->max_blocks * e->bs,
                                  e->dtype, pt);
}

int pa_engine_step(pa_engine* e, const int64_t* seqs, int32_t n, const void* q,
                   const void* k_new, const void* v_new, float scale, void* out,
                   void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                   void* stream, pa_step_info* info) {
  if (!e || n < 0 || n > e->max_batch || (n > 0 && !seqs)) return PA_ERR_INVALID;
  if (info) std::memset(info, 0, sizeof(*info));
  if (n == 0) return PA_OK;
  // Every argument the launches check is checked here, before the block
  // manager commits the appends.
  for (const void* p : {q, k_new, v_new, static_cast<const void*>(out)})
    if (!p || size_t(p) % 16) return PA_ERR_INVALID;
  if (workspace && size_t(workspace) % 16) return PA_ERR_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);

  // 1. Checks that need no change of state: known, distinct sequences whose
  //    contexts fit the tables, and a workspace that covers any step.
  e->ctx_pre.resize(size_t(n));
  for (int32_t i = 0; i < n; ++i) {
    const int64_t len = pa_bm_seq_len(e->bm, seqs[i]);
    if (len < 0) return int(len);
    if (len + 1 > int64_t(e->max_blocks) * e->bs) return PA_ERR_CAPACITY;
    e->ctx_pre[i] = int32_t(len + 1);
  }
  {
    std::vector<int64_t> sorted(seqs, seqs + n);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end()) return PA_ERR_INVALID;
  }
  const size_t ws_bound = pa_engine_workspace_bytes(e, partition_tokens);
  if (ws_bound == size_t(-1)) return PA_ERR_INVALID;
  if (ws_bound > workspace_bytes || (ws_bound > 0 && !workspace)) return PA_ERR_WORKSPACE;

  // 2. Host staging slot.
  const int32_t slot = e->next;
  const int32_t guard = slot / e->group * e->group + e->group - 1;  // the group's event
  if (e->pending[guard]) {
    if (hipEventSynchronize(e->events[guard]) != hipSuccess) return PA_ERR_HIP;
    e->pending[guard] = 0;
  }
  char* h = e->host + size_t(slot) * e->slot_bytes;
  const size_t off_slots = 0, off_ctx = 8 * size_t(n), off_cow = off_ctx + 4 * size_t(n);
  const size_t off_tab = off_cow + 8 * size_t(n);
  const size_t off_items = off_tab + 4 * size_t(n) * size_t(e->max_blocks);
  int64_t* h_slots = reinterpret_cast<int64_t*>(h + off_slots);
  int32_t* h_ctx = reinterpret_cast<int32_t*>(h + off_ctx);
  int32_t* h_cow = reinterpret_cast<int32_t*>(h + off_cow);
  int32_t* h_tab = reinterpret_cast<int32_t*>(h + off_tab);

  // 3. Commit the appends, then schedule from the new tables and lengths.
  //    From here on a failure undoes the appends (all or nothing).  If some
  //    of the step's device work was already enqueued, the host slot counts
  //    as used: it is rewritten only after its guard event, as for a step
  //    that succeeded.
  int32_t ncow = 0;
  int rc = pa::bm_step_logged(e->bm, seqs, n, h_slots, h_cow, &ncow, h_tab, e->max_blocks, e->pad,
                              h_ctx, &e->undo);
  if (rc != PA_OK) return rc;
  bool enqueued = false;
  auto advance = [&]() -> int {
    e->unguarded = true;
    int status = PA_OK;
    if (slot == guard) {
      if (hipEventRecord(e->events[slot], st) == hipSuccess) {
        e->pending[slot] = 1;
        e->unguarded = false;
      } else {
        status = PA_ERR_HIP;
      }
    }
    e->next = (slot + 1) % e->ring;
    return status;
  };
  auto fail = [&](int code) -> int {
    pa::bm_undo(e->bm, e->undo);
    e->undo.clear();
    if (enqueued) (void)advance();
    return code;
  };
  rc = pa::build_schedule(h_ctx, n, e->H, e->D, e->bs, e->dtype, partition_tokens,
                          e->sharing ? h_tab : nullptr, e->max_blocks, &e->hs);
  if (rc != PA_OK) return fail(rc);
  const pa::HostSchedule& hs = e->hs;
  const int32_t n_items = int32_t(hs.items.size() / 5);
  const int32_t n_groups = int32_t(hs.groups.size() / 5);
  const size_t off_groups = off_items + 4 * hs.items.size();
  const size_t off_members = off_groups + 4 * hs.groups.size();
  if (!hs.items.empty()) std::memcpy(h + off_items, hs.items.data(), 4 * hs.items.size());
  if (!hs.groups.empty()) std::memcpy(h + off_groups, hs.groups.data(), 4 * hs.groups.size());
  if (!hs.members.empty()) std::memcpy(h + off_members, hs.members.data(), 4 * hs.members.size());
  const int32_t pt = hs.part_tokens, max_ctx = hs.max_ctx;

  // 4. Ship the used bytes, copy shared last blocks, write the new tokens.
  //    Copies must land before the writes into the copied blocks.  Mapped
  //    device staging: the host writes the device slot, and the decode launch
  //    writes the new tokens.  Otherwise, without copies, one prologue launch
  //    ships the staging and writes the tokens.
  const size_t used = (off_members + 4 * hs.members.size() + 15) & ~size_t(15);
  char* d = e->dev;
  const bool mapped = e->mapped != nullptr && e->use_mapped;
  const bool fused = !mapped && e->host_dev != nullptr && ncow == 0;
  // mapped staging: the decode launch writes the new tokens itself when
  // every row's last token lies in a single item (its last partition; never
  // in a shared range, whose last block is private after copy on write)
  bool write_in_decode = mapped && n_items > 0;
  if (write_in_decode && n_groups > 0) {
    e->covered.assign(size_t(n), 0);
    for (size_t i = 0; i + 4 < hs.items.size(); i += 5) {
      const int32_t s = hs.items[i], part = hs.items[i + 1], ntok = hs.items[i + 3];
      if (s >= 0 && s < n && ntok > 0 && part == hs.items[i + 4] - 1) e->covered[size_t(s)] = 1;
    }
    write_in_decode = std::all_of(e->covered.begin(), e->covered.end(), [](char c) { return c; });
  }
  if (mapped) {
    d = e->mapped + size_t(slot) * e->slot_bytes;
    mapped_publish(d, h, used);
    enqueued = true;
    if (ncow > 0) {
      rc = pa_copy_blocks(e->k_cache, e->v_cache, reinterpret_cast<const int32_t*>(d + off_cow),
                          ncow, e->num_blocks, e->H, e->D, e->bs, e->dtype, stream);
      if (rc != PA_OK) return fail(rc);
    }
    if (!write_in_decode) {
      rc = pa_cache_write(k_new, v_new, reinterpret_cast<const int64_t*>(d + off_slots), n,
                          e->k_cache, e->v_cache, e->num_blocks, e->H, e->D, e->bs, e->dtype,
                          stream);
      if (rc != PA_OK) return fail(rc);
    }
  } else if (fused) {
    char* hd = e->host_dev + size_t(slot) * e->slot_bytes;
    rc = pa::launch_step_prologue(hd, d, used, reinterpret_cast<const int64_t*>(hd + off_slots),
                                  k_new, v_new, n, e->k_cache, e->v_cache, e->num_blocks, e->H,
                                  e->D, e->bs, e->dtype, st);
    enqueued = true;
    if (rc != PA_OK) return fail(rc);
  } else {
    if (hipMemcpyAsync(d, h, used, hipMemcpyHostToDevice, st) != hipSuccess) {
      enqueued = true;
      return fail(PA_ERR_HIP);
    }
    enqueued = true;
    if (ncow > 0) {
      rc = pa_copy_blocks(e->k_cache, e->v_cache, reinterpret_cast<const int32_t*>(d + off_cow),
                          ncow, e->num_blocks, e->H, e->D, e->bs, e->dtype, stream);
      if (rc != PA_OK) return fail(rc);
    }
    rc = pa_cache_write(k_new, v_new, reinterpret_cast<const int64_t*>(d + off_slots), n,
                        e->k_cache, e->v_cache, e->num_blocks, e->H, e->D, e->bs, e->dtype,
                        stream);
    if (rc != PA_OK) return fail(rc);
  }
  const int32_t* d_tab = reinterpret_cast<const int32_t*>(d + off_tab);
  const int32_t* d_ctx = reinterpret_cast<const int32_t*>(d + off_ctx);
  const int32_t* d_items = reinterpret_cast<const int32_t*>(d + off_items);
  // ev_start / ev_end (if set) are recorded by the decode kernel's own dispatch
  rc = pa::decode_scheduled_timed(q, e->k_cache, e->v_cache, d_tab, e->max_blocks, d_ctx, n,
                                  e->H, e->D, e->bs, e->num_blocks, scale, max_ctx, e->dtype,
                                  out, workspace, workspace_bytes, pt, stream,
                                  n_items ? d_items : nullptr, n_items,
                                  n_groups ? reinterpret_cast<const int32_t*>(d + off_groups)
                                           : nullptr,
                                  n_groups,
                                  n_groups ? reinterpret_cast<const int32_t*>(d + off_members)
                                           : nullptr,
                                  e->ev_start, e->ev_end, int64_t(e->max_batch) * e->H,
                                  write_in_decode
                                      ? pa::NewTokens{k_new, v_new,
                                                      reinterpret_cast<const int64_t*>(
                                                          d + off_slots)}
                                      : pa::NewTokens());
  if (rc != PA_OK) return fail(rc);
  e->undo.clear();
  // The host slots of this group may be rewritten once this step has run
  // (recorded at the end of the group's last step: no marker between the
  // prologue and the decode, and none after the group's other steps).
  rc = advance();
  if (info) {
    info->num_cow = ncow;
    info->max_context_len = max_ctx;
    info->partition_tokens = pt;
    info->num_items = n_items;
    info->num_group_items = n_groups;
    int64_t sum = 0;
    for (int32_t i = 0; i < n; ++i) sum += h_ctx[i];
    info->sum_context_len = sum;
  }
  // a failed guard record leaves the step done (the decode is enqueued); the
  // host slot then waits for the next guard event
  return rc;
}

int pa_engine_set_sharing(pa_engine* e, int32_t enable) {
  if (!e) return PA_ERR_INVALID;
  e->sharing = enable != 0;
  return PA_OK;
}

int pa_engine_set_mapped_staging(pa_engine* e, int32_t enable) {
  if (!e) return PA_ERR_INVALID;
  if (enable && !e->mapped) return PA_ERR_UNSUPPORTED;
  e->use_mapped = enable != 0;
  return PA_OK;
}

int32_t pa_engine_has_mapped_staging(const pa_engine* e) { return e && e->mapped ? 1 : 0; }

int pa_engine_set_decode_events(pa_engine* e, void* start_event, void* end_event) {
  if (!e) return PA_ERR_INVALID;
  e->ev_start = static_cast<hipEvent_t>(start_event);
  e->ev_end = static_cast<hipEvent_t>(end_event);
  return PA_OK;
}

int pa_engine_last_step(const pa_engine* e, int32_t n, int64_t* slots, int32_t* context_lens,
                        int32_t* cow_pairs, int32_t num_cow) {
  if (!e || n < 0 || n > e->max_batch) return PA_ERR_INVALID;
  const int32_t slot = (e->next + e->ring - 1) % e->ring;
  const char* h = e->host + size_t(slot) * e->slot_bytes;
  if (slots) std::memcpy(slots, h, 8 * size_t(n));
  if (context_lens) std::memcpy(context_lens, h + 8 * size_t(n), 4 * size_t(n));
  if (cow_pairs && num_cow > 0)
    std::memcpy(cow_pairs, h + 12 * size_t(n), 8 * size_t(num_cow));
  return PA_OK;
}

}  // extern "C"

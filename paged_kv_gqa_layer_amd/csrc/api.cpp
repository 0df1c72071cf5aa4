// C ABI of libpkv (declared in include/pkv.h): argument checks, device-side
// pool state, per-call descriptor upload, kernel launches and kernel timing.
//
// Device-side state of a pool (besides the caller's K/V storage):
//  - a mirror of every sequence's page table, int32 [max_seqs][stride], kept
//    current by patch lists (one entry per page-table write on the host,
//    applied by a small kernel before the next kernel that reads the mirror);
//  - per batch row, one RowDesc (length, mirror offset, decode split range),
//    uploaded together with the pending patches once per pool version and
//    batch, so every layer of a step reuses the same upload.
// Uploads go through a ring of pinned staging slots; a slot is rewritten only
// after the event recorded behind its previous copy has completed.  All
// copies and kernels of a pool go to the caller's stream, in call order.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>
#include <type_traits>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "device.hpp"
#include "pkv.h"
#include "pool_meta.hpp"

namespace {

using pkv::AttnArgs;
using pkv::ContigMap;
using pkv::PagedMap;
using pkv::RowDesc;

constexpr double kLog2e = 1.4426950408889634074;
constexpr int kStageSlots = 8;
// Timing events made when profiling is switched on (two per timed launch).
constexpr size_t kProfReserve = 256;

enum Buf { kRows = 0, kCow = 1, kNumBufs = 2 };

inline int32_t ceil_div(int64_t a, int64_t b) {
  return static_cast<int32_t>((a + b - 1) / b);
}

int32_t dev_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_DEVICE; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Pinned staging ring, small device buffers, timing.
struct DeviceCtx {
  struct Slot {
    void* host = nullptr;
    const void* dev = nullptr;  // the same memory as kernels address it
    size_t cap = 0;
    bool used = false;  // read by an enqueued launch or copy not known done
  };
  // Slot guard events, one per group of kSlotGroup consecutive slots: the
  // event of a group is recorded after the launch or copy that reads the
  // group's last slot, so (the stream being in order) it completes after
  // every earlier reader of the group's slots; a used slot is rewritten only
  // after that.  One record per group rather than per use: each record is a
  // system-scope release in the stream (an L2 write-back before the signal),
  // several microseconds of GPU time that the next launch waits behind.
  static constexpr int kSlotGroup = 4;
  static constexpr int kSlotGroups = kStageSlots / kSlotGroup;
  hipEvent_t group_ev[kSlotGroups] = {};
  bool group_rec[kSlotGroups] = {};  // recorded since the group was last freed
  struct DevBuf {
    void* ptr = nullptr;
    size_t cap = 0;
    bool valid = false;  // holds the blob described by `key`
    std::vector<int64_t> key;
  };
  Slot slot[kStageSlots];
  int next = 0;
  int last_slot = 0;  // the slot take_slot returned last
  DevBuf buf[kNumBufs];
  hipStream_t last_stream = nullptr;
  bool used = false;

  bool prof_on = false;
  uint32_t prof_mask = ~0u;  // kernel ids timed while prof_on
  // while set, timing uses only events made earlier (none are created)
  bool no_new_events = false;
  // the kernel form (template instance) last launched under each kernel id
  std::string form[PKV_K_COUNT];
  std::vector<std::pair<hipEvent_t, hipEvent_t>> prof_ev[PKV_K_COUNT];
  // Timing events of earlier profiling runs, reused (creating timing events
  // can cost the host more than a short step).
  std::vector<hipEvent_t> ev_pool;

  ~DeviceCtx() { release(); }

  void release() {
    if (used) (void)hipStreamSynchronize(last_stream);
    for (int g = 0; g < kSlotGroups; ++g) {
      if (group_ev[g]) (void)hipEventSynchronize(group_ev[g]), (void)hipEventDestroy(group_ev[g]);
      group_ev[g] = nullptr;
      group_rec[g] = false;
    }
    for (auto& s : slot) {
      if (s.host) (void)hipHostFree(s.host);
      s = Slot();
    }
    for (auto& b : buf) {
      if (b.ptr) (void)hipFree(b.ptr);
      b = DevBuf();
    }
    clear_prof();
    for (hipEvent_t e : ev_pool) (void)hipEventDestroy(e);
    ev_pool.clear();
    used = false;
  }

  // Callers synchronise the stream first, so every recorded event is done.
  void clear_prof() {
    for (auto& v : prof_ev) {
      for (auto& e : v) {
        ev_pool.push_back(e.first);
        ev_pool.push_back(e.second);
      }
      v.clear();
    }
  }

  // Timing events for the next profiled launches, made before they are
  // needed: creating one can cost the host hundreds of microseconds.
  hipError_t reserve_events(size_t n, hipStream_t st) {
    const size_t had = ev_pool.size();
    while (ev_pool.size() < n) {
      hipEvent_t e = nullptr;
      hipError_t r = hipEventCreate(&e);
      if (r != hipSuccess) return r;
      ev_pool.push_back(e);
      if ((r = hipEventRecord(e, st)) != hipSuccess) return r;
    }
    return ev_pool.size() > had ? hipStreamSynchronize(st) : hipSuccess;
  }

  hipEvent_t take_event() {
    if (!ev_pool.empty()) {
      const hipEvent_t e = ev_pool.back();
      ev_pool.pop_back();
      return e;
    }
    if (no_new_events) return nullptr;
    hipEvent_t e = nullptr;
    return hipEventCreate(&e) == hipSuccess ? e : nullptr;
  }

  // All device work of a context goes to one stream at a time.
  hipError_t use_stream(hipStream_t st) {
    if (used && st != last_stream) {
      hipError_t e = hipStreamSynchronize(last_stream);
      if (e != hipSuccess) return e;
    }
    last_stream = st;
    used = true;
    return hipSuccess;
  }

  // Device buffer `b` with room for `bytes` (its old content is dropped).
  hipError_t reserve(int b, size_t bytes, hipStream_t st) {
    DevBuf& d = buf[b];
    if (bytes <= d.cap) return hipSuccess;
    hipError_t e = hipStreamSynchronize(st);  // old buffer may still be read
    if (e != hipSuccess) return e;
    if (d.ptr) (void)hipFree(d.ptr);
    d = DevBuf();
    const size_t cap = bytes < 65536 ? 65536 : bytes + bytes / 2;
    if ((e = hipMalloc(&d.ptr, cap)) != hipSuccess) return e;
    d.cap = cap;
    return hipSuccess;
  }

  // The next staging slot, free for rewriting (its previous reader done),
  // with room for `bytes`.
  hipError_t take_slot(size_t bytes, Slot** out) {
    Slot& s = slot[next];
    const int g = next / kSlotGroup;
    last_slot = next;
    next = (next + 1) % kStageSlots;
    hipError_t e;
    if (s.used) {
      // the group's event follows every use of its slots; without one (a
      // reader whose launch failed after the slot was filled) wait for the
      // whole stream
      e = group_rec[g] ? hipEventSynchronize(group_ev[g]) : hipStreamSynchronize(last_stream);
      if (e != hipSuccess) return e;
      for (int j = g * kSlotGroup; j < (g + 1) * kSlotGroup; ++j) slot[j].used = false;
      group_rec[g] = false;
    }
    if (!group_ev[g] &&
        (e = hipEventCreateWithFlags(&group_ev[g], hipEventDisableTiming)) != hipSuccess)
      return e;
    if (bytes > s.cap) {
      if (s.host) (void)hipHostFree(s.host);
      s.host = nullptr;
      s.dev = nullptr;
      s.cap = 0;
      const size_t cap = bytes < 65536 ? 65536 : bytes + bytes / 2;
      // coherent: kernels read the slot directly and must see every rewrite
      if ((e = hipHostMalloc(&s.host, cap, hipHostMallocMapped | hipHostMallocCoherent)) !=
          hipSuccess)
        return e;
      void* dp = nullptr;
      if ((e = hipHostGetDevicePointer(&dp, s.host, 0)) != hipSuccess) return e;
      s.dev = dp;
      s.cap = cap;
    }
    *out = &s;
    return hipSuccess;
  }

  // Copy `blob` into device buffer `b` (skipped if it already holds `key`;
  // an empty key never matches).
  hipError_t upload(int b, const std::vector<int32_t>& blob,
                    const std::vector<int64_t>& key, hipStream_t st,
                    int32_t** dev) {
    DevBuf& d = buf[b];
    if (!key.empty() && d.valid && d.key == key) {
      *dev = static_cast<int32_t*>(d.ptr);
      return hipSuccess;
    }
    d.valid = false;
    const size_t bytes = std::max<size_t>(blob.size(), 1) * sizeof(int32_t);
    hipError_t e = reserve(b, bytes, st);
    if (e != hipSuccess) return e;
    Slot* s = nullptr;
    if ((e = take_slot(bytes, &s)) != hipSuccess) return e;
    if (!blob.empty()) {
      std::memcpy(s->host, blob.data(), blob.size() * sizeof(int32_t));
      if ((e = hipMemcpyAsync(d.ptr, s->host, blob.size() * sizeof(int32_t),
                              hipMemcpyHostToDevice, st)) != hipSuccess)
        return e;
      if ((e = staged(st)) != hipSuccess) return e;
    }
    d.key = key;
    d.valid = !key.empty();
    *dev = static_cast<int32_t*>(d.ptr);
    return hipSuccess;
  }

  // As upload, but the copy into device buffer `b` is left to the caller's
  // next kernel: the blob goes to a pinned staging slot which that kernel
  // reads (*src, a device-readable address) and copies to *dev.  *src is
  // null when buffer b already holds `key` (nothing to copy).  After the
  // kernel is enqueued, staged(st) marks the slot busy until it has run.
  hipError_t stage(int b, const std::vector<int32_t>& blob,
                   const std::vector<int64_t>& key, hipStream_t st,
                   const int32_t** src, int32_t** dev) {
    DevBuf& d = buf[b];
    *src = nullptr;
    if (!key.empty() && d.valid && d.key == key) {
      *dev = static_cast<int32_t*>(d.ptr);
      return hipSuccess;
    }
    d.valid = false;
    const size_t bytes = std::max<size_t>(blob.size(), 1) * sizeof(int32_t);
    hipError_t e = reserve(b, bytes, st);
    if (e != hipSuccess) return e;
    Slot* s = nullptr;
    if ((e = take_slot(bytes, &s)) != hipSuccess) return e;
    if (!blob.empty()) std::memcpy(s->host, blob.data(), blob.size() * sizeof(int32_t));
    d.key = key;
    d.valid = !key.empty();
    *src = static_cast<const int32_t*>(s->dev);
    *dev = static_cast<int32_t*>(d.ptr);
    return hipSuccess;
  }
  // Buffer b holds the blob `key` names (an upload of it would copy nothing).
  bool holds(int b, const std::vector<int64_t>& key) const {
    return !key.empty() && buf[b].valid && buf[b].key == key;
  }

  // Device buffer b sized for `bytes` and marked as holding `key`, for a
  // launch that writes the blob there itself (its argument copy).
  hipError_t claim(int b, size_t bytes, const std::vector<int64_t>& key, hipStream_t st,
                   int32_t** dev) {
    DevBuf& d = buf[b];
    d.valid = false;
    const hipError_t e = reserve(b, std::max<size_t>(bytes, 1), st);
    if (e != hipSuccess) return e;
    d.key = key;
    d.valid = !key.empty();
    *dev = static_cast<int32_t*>(d.ptr);
    return hipSuccess;
  }

  hipError_t staged(hipStream_t st) {
    slot[last_slot].used = true;
    if (last_slot % kSlotGroup != kSlotGroup - 1) return hipSuccess;
    const int g = last_slot / kSlotGroup;
    const hipError_t e = hipEventRecord(group_ev[g], st);
    if (e == hipSuccess) group_rec[g] = true;
    return e;
  }

  // Timing brackets around one launch.
  struct ProfScope {
    DeviceCtx* c;
    int k;
    hipStream_t st;
    hipEvent_t a = nullptr, b = nullptr;
    ProfScope(DeviceCtx* c_, int k_, hipStream_t st_) : c(c_), k(k_), st(st_) {
      if (!c->prof_on || !((c->prof_mask >> k) & 1u)) return;
      if (!(a = c->take_event())) return;
      if (!(b = c->take_event())) {
        c->ev_pool.push_back(a);
        a = nullptr;
        return;
      }
      (void)hipEventRecord(a, st);
    }
    ~ProfScope() {
      if (!a) return;
      (void)hipEventRecord(b, st);
      c->prof_ev[k].emplace_back(a, b);
    }
  };
};

// Shared by the contiguous-twin calls (no pool object to hang state on).
DeviceCtx& contig_ctx() {
  static DeviceCtx* c = new DeviceCtx();  // lives until process exit
  return *c;
}
std::mutex& contig_mutex() {
  static std::mutex m;
  return m;
}

// What a row blob holds beyond the RowDescs (see device.hpp).
struct RowPlan {
  int32_t n_items = 0;      // split decode items (the rows' own key splits)
  int32_t n_slots = 0;      // partial-result slots (own splits + prefix splits)
  int32_t max_parts = 0;    // most partial results of one row
  int32_t max_split = 0;    // longest split (keys)
  size_t item_off = 0;      // int32 offset of the (row, split) item list
  // shared-prefix decode (empty otherwise): int32 offsets in the blob
  int32_t n_pre_items = 0;
  size_t pre_off = 0, group_off = 0, member_off = 0;
};

// One batch row as the plan sees it: cached rows, page-table offset, first
// own key and prefix partial slots (both 0 unless a shared prefix is used).
struct RowIn {
  int32_t start = 0, pt_off = 0, k_off = 0, n_pre = 0;
  int32_t append_block = -1;  // paged: block of page start / block_size
};

// Row blob: RowDesc[M], then the split items as (row, split) pairs, longest
// first (the hardware starts workgroups in grid order, so the short items
// fill the slots that free up last): full splits of the longest split size,
// row by row, then shorter sizes, with each partial last split placed before
// the first size it is longer than.  The split plan is for n_q new rows per
// sequence (total_k = start + n_q): the row's own keys [k_off, total_k) are
// cut into split_keys(own, n_q, shared)-key splits (shared: a shared-prefix
// decode plan).
template <class F>
RowPlan build_rows(std::vector<int32_t>& v, int32_t M, int32_t n_q, bool shared,
                   F rowinfo) {
  RowPlan pl;
  v.assign(static_cast<size_t>(M) * pkv::kRowInts, 0);
  std::vector<std::pair<int32_t, int32_t>> tails;  // (partial keys, row)
  std::vector<int32_t> sizes;                      // distinct split sizes
  pl.item_off = v.size();
  for (int32_t r = 0; r < M; ++r) {
    const RowIn in = rowinfo(r);
    const int64_t own = static_cast<int64_t>(in.start) + n_q - in.k_off;
    const int32_t split = pkv::split_keys(own, n_q, shared);
    const int32_t nsp = ceil_div(own, split);
    const int32_t rem = static_cast<int32_t>(own % split);
    int32_t* d = v.data() + static_cast<size_t>(r) * pkv::kRowInts;
    d[0] = in.start;
    d[1] = in.pt_off;
    d[2] = nsp;
    d[3] = pl.n_slots + in.n_pre;
    d[4] = in.k_off;
    d[5] = in.n_pre;
    d[6] = in.append_block;
    d[7] = split;
    pl.n_items += nsp;
    pl.n_slots += in.n_pre + nsp;
    pl.max_parts = std::max(pl.max_parts, in.n_pre + nsp);
    pl.max_split = std::max(pl.max_split, split);
    if (rem) tails.emplace_back(rem, r);
    if (std::find(sizes.begin(), sizes.end(), split) == sizes.end()) sizes.push_back(split);
  }
  std::stable_sort(tails.begin(), tails.end(),
                   [](const std::pair<int32_t, int32_t>& x,
                      const std::pair<int32_t, int32_t>& y) { return x.first > y.first; });
  std::sort(sizes.begin(), sizes.end(), std::greater<int32_t>());
  size_t ti = 0;
  auto emit_tails_above = [&](int32_t keys) {
    for (; ti < tails.size() && tails[ti].first > keys; ++ti) {
      const int32_t r = tails[ti].second;
      v.push_back(r);
      v.push_back(v[static_cast<size_t>(r) * pkv::kRowInts + 2] - 1);
    }
  };
  for (const int32_t size : sizes) {
    emit_tails_above(size);
    for (int32_t r = 0; r < M; ++r) {
      const int32_t* d = v.data() + static_cast<size_t>(r) * pkv::kRowInts;
      if (d[7] != size) continue;
      const int64_t own = static_cast<int64_t>(d[0]) + n_q - d[4];
      const int32_t n_full = static_cast<int32_t>(own / size);
      for (int32_t sp = 0; sp < n_full; ++sp) {
        v.push_back(r);
        v.push_back(sp);
      }
    }
  }
  emit_tails_above(0);
  return pl;
}

// Shared prefixes of a decode batch ("nx_paged_kv_gate.nx source", fork:
// forked sequences hold the same blocks, by reference count, for their
// common rows).  Rows are grouped when their page tables begin with the same
// full pages -- at least kMinSharedPages of them -- and a group's prefix is
// the full pages all its members share.  Groups are found in batch order
// (bucketed by the first block), so the plan depends only on the batch.
constexpr int32_t kMinSharedPages = 16;

struct SharedPlan {
  std::vector<int32_t> k_off, n_pre;        // per row
  std::vector<int32_t> groups, members, items;
};

void find_shared(const pkv::PoolMeta& m, const int32_t* seqs, int32_t M,
                 int32_t group_heads, SharedPlan* sp) {
  const int32_t B = m.block_size();
  sp->k_off.assign(M, 0);
  sp->n_pre.assign(M, 0);
  sp->groups.clear();
  sp->members.clear();
  sp->items.clear();
  std::unordered_map<int64_t, std::vector<int32_t>> by_first;
  std::vector<int64_t> order;
  for (int32_t r = 0; r < M; ++r) {
    const pkv::SeqMeta* q = m.seq(seqs[r]);
    if (q->seq_len / B < kMinSharedPages) continue;
    auto it = by_first.find(q->pages[0]);
    if (it == by_first.end()) {
      order.push_back(q->pages[0]);
      by_first[q->pages[0]].push_back(r);
    } else {
      it->second.push_back(r);
    }
  }
  std::vector<int32_t> mem;
  for (const int64_t first : order) {
    const std::vector<int32_t>& bucket = by_first[first];
    if (bucket.size() < 2) continue;
    const pkv::SeqMeta* rep = m.seq(seqs[bucket[0]]);
    int32_t P = rep->seq_len / B;
    mem.assign(1, bucket[0]);
    for (size_t i = 1; i < bucket.size(); ++i) {
      const pkv::SeqMeta* q = m.seq(seqs[bucket[i]]);
      const int32_t lim = std::min(q->seq_len / B, rep->seq_len / B);
      int32_t l = 0;
      while (l < lim && q->pages[l] == rep->pages[l]) ++l;
      if (l < kMinSharedPages) continue;
      mem.push_back(bucket[i]);
      P = std::min(P, l);
    }
    if (mem.size() < 2) continue;
    const int32_t keys = P * B;
    const int32_t n_pre = ceil_div(keys, pkv::kPrefixSplit);
    const int32_t g = static_cast<int32_t>(sp->groups.size() / 4);
    sp->groups.insert(sp->groups.end(),
                      {mem[0], static_cast<int32_t>(sp->members.size()),
                       static_cast<int32_t>(mem.size()), keys});
    for (const int32_t r : mem) {
      sp->members.push_back(r);
      sp->k_off[r] = keys;
      sp->n_pre[r] = n_pre;
    }
    const int32_t n_rb = ceil_div(static_cast<int64_t>(mem.size()) * group_heads,
                                  pkv::kPrefixRows);
    for (int32_t s = 0; s < n_pre; ++s)
      for (int32_t b = 0; b < n_rb; ++b) sp->items.insert(sp->items.end(), {g, s, b, 0});
  }
}

// Append the shared-prefix tables to a row blob (16-byte aligned entries).
void append_shared(std::vector<int32_t>& v, const SharedPlan& sp, RowPlan* pl) {
  auto align4 = [&]() { while (v.size() % 4) v.push_back(0); };
  align4();
  pl->pre_off = v.size();
  v.insert(v.end(), sp.items.begin(), sp.items.end());
  pl->group_off = v.size();
  v.insert(v.end(), sp.groups.begin(), sp.groups.end());
  pl->member_off = v.size();
  v.insert(v.end(), sp.members.begin(), sp.members.end());
  pl->n_pre_items = static_cast<int32_t>(sp.items.size() / 4);
}

}  // namespace

// ---------------------------------------------------------------------------

// Rotary table on the device: (cos, sin) in double per (position, pair).
struct pkv_rope {
  int32_t head_dim = 0;
  int32_t max_positions = 0;
  double log_base = 0.0;
  double2* table = nullptr;  // [max_positions][head_dim / 2]
  ~pkv_rope() {
    if (table) (void)hipFree(table);
  }
};

struct pkv_pool {
  pkv::PoolMeta meta;
  float* storage = nullptr;
  size_t storage_bytes = 0;
  int64_t block_floats = 0;
  DeviceCtx dev;
  int32_t* mirror = nullptr;  // [max_seqs][stride]
  int64_t stride = 0;
  // A launch that was to apply page-table patches (taken off the pending
  // list) failed: the next call re-patches every entry of every table.
  bool mirror_stale = false;
  // the row blob currently in dev.buf[kRows]
  std::vector<int32_t> rows;
  std::vector<int32_t> na_rows;  // the last zero-allocation decode's blob
  RowPlan plan;
  std::vector<int64_t> rows_key;
  size_t patch_off = 0;  // patches follow the rows in the blob
  std::unordered_set<int64_t> seen;
  const pkv_rope* rope = nullptr;  // borrowed; null = no rotary embedding
  int32_t checks = 0;              // debug state checks (pkv_pool_set_checks)
  bool last_shared = false;        // the last attention call grouped prefixes
  int32_t shared_heads = 0;        // ... with this many query heads per kv head
  SharedPlan shared;

  pkv_pool(int32_t nb, int32_t bs, int32_t nl, int32_t g, int32_t d, int32_t ms)
      : meta(nb, bs, nl, g, d, ms) {}
  ~pkv_pool() {
    dev.release();
    if (mirror) (void)hipFree(mirror);
  }
};

namespace {

// Every page-table entry of every sequence as a pending patch (a new or
// stale mirror), replacing the pending list.
void queue_all_pages(pkv_pool* p) {
  auto& m = p->meta;
  p->mirror_stale = false;
  p->rows_key.clear();  // row descriptors hold mirror offsets
  auto& pt = m.patches();
  pt.clear();
  for (int32_t s = 0; s < m.max_seqs(); ++s) {
    const pkv::SeqMeta* q = m.seq(s);
    if (!q) continue;
    for (int32_t i = 0; i < static_cast<int32_t>(q->pages.size()); ++i)
      pt.push_back({s, i, q->pages[i]});
  }
}

// (Re)allocate the page-table mirror when a sequence may outgrow its stride;
// a new or stale mirror is filled from every live page-table entry.
hipError_t size_mirror(pkv_pool* p, hipStream_t st) {
  auto& m = p->meta;
  const int64_t stride = pkv::PoolMeta::mirror_stride(m.max_pages_seen());
  const bool grow = !p->mirror || stride > p->stride;
  if (!grow && !p->mirror_stale) return hipSuccess;
  if (grow) {
    hipError_t e;
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
    if (p->mirror) (void)hipFree(p->mirror);
    p->mirror = nullptr;
    if ((e = hipMalloc(&p->mirror, static_cast<size_t>(m.max_seqs()) * stride *
                                       sizeof(int32_t))) != hipSuccess)
      return e;
    p->stride = stride;
  }
  queue_all_pages(p);
  return hipSuccess;
}

// The row blob of a batch (n new rows per sequence; with shared_heads > 0 --
// the query heads per kv head -- grouped by shared prefix) for the mirror's
// current stride, followed by the pending page-table patches (from int32
// offset *patch_off on, three ints each).
void build_blob(pkv_pool* p, const int32_t* seqs, int32_t M, int32_t n,
                int32_t shared_heads, std::vector<int32_t>& blob, RowPlan* plan,
                size_t* patch_off) {
  const bool shared = shared_heads > 0;
  if (shared) find_shared(p->meta, seqs, M, shared_heads, &p->shared);
  const int32_t B = p->meta.block_size();
  const bool grouped = shared && !p->shared.groups.empty();
  *plan = build_rows(blob, M, n, grouped, [&](int32_t r) {
    const pkv::SeqMeta* q = p->meta.seq(seqs[r]);
    RowIn in;
    in.start = q->seq_len;
    in.pt_off = static_cast<int32_t>(seqs[r] * p->stride);
    const size_t pg = static_cast<size_t>(q->seq_len / B);
    in.append_block = pg < q->pages.size() ? static_cast<int32_t>(q->pages[pg]) : -1;
    if (shared) {
      in.k_off = p->shared.k_off[r];
      in.n_pre = p->shared.n_pre[r];
    }
    return in;
  });
  if (shared) append_shared(blob, p->shared, plan);
  // The patch kernel writes entries in parallel, so keep only the last
  // write of each (sequence, page) entry (a fork's share followed by a
  // copy-on-append replacement, for example).
  *patch_off = blob.size();
  p->seen.clear();
  const auto& pt = p->meta.patches();
  for (auto it = pt.rbegin(); it != pt.rend(); ++it) {
    if (!p->seen.insert(static_cast<int64_t>(it->seq) * p->stride + it->page).second)
      continue;
    blob.push_back(it->seq);
    blob.push_back(it->page);
    blob.push_back(it->block);
  }
}

// pool_rows: row descriptors of this batch (see build_blob) on the device,
// with the pending page-table patches applied to the mirror first.  Rows and
// patches travel in one upload, which is skipped when the device copy
// already describes this batch at this pool version (no patches can be
// pending then: every page-table change bumps the version).
// With `fused` (the one-row append), both the upload and the patches are
// left to the caller's kernel: *rows_dev is then the copy that kernel reads
// (the pinned staging copy when an upload is due), *fused says what it must
// copy and patch, and the caller calls p->dev.staged(st) after the launch
// when fused->n_copy > 0.
//
// Its first half: the mirror sized for every sequence and the row blob of
// this batch in p->rows / p->plan (rebuilt unless the last one already
// describes this batch at this pool version); *key names it.
hipError_t plan_rows(pkv_pool* p, const int32_t* seqs, int32_t M, int32_t n,
                     int32_t shared_heads, hipStream_t st, std::vector<int64_t>* key) {
  const hipError_t e = size_mirror(p, st);
  if (e != hipSuccess) return e;
  key->clear();
  key->reserve(M + 4);
  key->push_back(static_cast<int64_t>(p->meta.version()));
  key->push_back(p->stride);
  key->push_back(n);
  key->push_back(shared_heads);
  key->insert(key->end(), seqs, seqs + M);
  if (*key != p->rows_key || !p->meta.patches().empty()) {
    build_blob(p, seqs, M, n, shared_heads, p->rows, &p->plan, &p->patch_off);
    p->rows_key.clear();  // the blob below is new
  }
  return hipSuccess;
}

// Second half: the blob plan_rows left in p->rows (named by key) to the
// device.
hipError_t rows_to_device(pkv_pool* p, const std::vector<int64_t>& key, hipStream_t st,
                          const int32_t** rows_dev, pkv::PatchArgs* fused) {
  hipError_t e;
  auto& pt = p->meta.patches();
  const int32_t n_patch = static_cast<int32_t>((p->rows.size() - p->patch_off) / 3);
  int32_t* d = nullptr;
  if (fused) {
    const int32_t* src = nullptr;
    if ((e = p->dev.stage(kRows, p->rows, key, st, &src, &d)) != hipSuccess) return e;
    const int32_t* from = src ? src : d;
    *fused = pkv::PatchArgs{p->mirror, from + p->patch_off, 0, p->stride, src, d,
                            src ? static_cast<int32_t>(p->rows.size()) : 0};
    if (!pt.empty()) {
      pt.clear();
      fused->n = n_patch;  // the caller's launch applies them
    }
    p->rows_key = key;
    *rows_dev = from;
    return hipSuccess;
  }
  if ((e = p->dev.upload(kRows, p->rows, key, st, &d)) != hipSuccess) return e;
  if (!pt.empty()) {
    pt.clear();
    if ((e = pkv::launch_patch(p->mirror, d + p->patch_off, n_patch, p->stride, st)) !=
        hipSuccess) {
      p->mirror_stale = true;
      return e;
    }
  }
  p->rows_key = key;
  *rows_dev = d;
  return hipSuccess;
}

hipError_t pool_rows(pkv_pool* p, const int32_t* seqs, int32_t M, int32_t n,
                     int32_t shared_heads, hipStream_t st, const int32_t** rows_dev,
                     pkv::PatchArgs* fused = nullptr) {
  std::vector<int64_t> key;
  const hipError_t e = plan_rows(p, seqs, M, n, shared_heads, st, &key);
  if (e != hipSuccess) return e;
  return rows_to_device(p, key, st, rows_dev, fused);
}

// Floats per head unit of the append scatter (half a head with a rotary
// table: a thread takes a value and its rotation partner).
int32_t span_of(const pkv_pool* p) {
  return p->rope ? p->meta.head_dim() / 2 : p->meta.head_dim();
}

PagedMap make_paged_map(const pkv_pool* p, int32_t layer) {
  const auto& m = p->meta;
  const int64_t G = m.n_kv_heads(), B = m.block_size(), D = m.head_dim();
  PagedMap pm;
  pm.base = p->storage;
  pm.pages = p->mirror;
  pm.block_stride = p->block_floats;
  pm.layer_off = static_cast<int64_t>(layer) * 2 * G * B * D;
  pm.head_stride = B * D;
  pm.v_off = G * B * D;
  pm.block_size = m.block_size();
  return pm;
}

// Debug state checks (pkv_pool_set_checks).  Host state a launch for the
// rows of `seqs` relies on: the pages covering seq_len + n rows exist, every
// page id is in range, each block's count is at least the page-table entries
// naming it (and those are at least one), and with `writes` every page the
// n new rows land in is held by this sequence alone.
int32_t check_state(const pkv_pool* p, const int32_t* seqs, int32_t M, int32_t n,
                    bool writes) {
  const auto& m = p->meta;
  const auto& ref = m.refcounts();
  const auto& held = m.holders();
  const int32_t B = m.block_size();
  for (int32_t r = 0; r < M; ++r) {
    const pkv::SeqMeta* q = m.seq(seqs[r]);
    const int64_t end = static_cast<int64_t>(q->seq_len) + n;
    if (end > static_cast<int64_t>(q->pages.size()) * B) return PKV_ERR_STATE;
    for (size_t i = 0; i < q->pages.size(); ++i) {
      const int32_t b = q->pages[i];
      if (b < 0 || b >= m.n_blocks() || held[b] < 1 || ref[b] < held[b]) return PKV_ERR_STATE;
      const int64_t first = static_cast<int64_t>(i) * B;
      if (writes && first + B > q->seq_len && first < end && ref[b] != 1) return PKV_ERR_STATE;
    }
  }
  return PKV_OK;
}

// The row blob as built for `seqs` (n rows each) against the host state:
// every row descriptor names its sequence's length, mirror offset and append
// block; every page-table patch addresses an entry inside the mirror and a
// block in range, and a live sequence's patch carries the block its page
// table holds now.
int32_t check_blob(const pkv_pool* p, const int32_t* seqs, int32_t M,
                   const std::vector<int32_t>& blob, size_t patch_off) {
  const auto& m = p->meta;
  const int32_t B = m.block_size();
  if (blob.size() < static_cast<size_t>(M) * pkv::kRowInts || patch_off > blob.size() ||
      (blob.size() - patch_off) % 3 != 0)
    return PKV_ERR_STATE;
  for (int32_t r = 0; r < M; ++r) {
    const pkv::SeqMeta* q = m.seq(seqs[r]);
    const int32_t* d = blob.data() + static_cast<size_t>(r) * pkv::kRowInts;
    const size_t pg = static_cast<size_t>(q->seq_len / B);
    const int32_t ab = pg < q->pages.size() ? q->pages[pg] : -1;
    if (d[0] != q->seq_len || d[1] != seqs[r] * p->stride || d[6] != ab) return PKV_ERR_STATE;
  }
  for (size_t i = patch_off; i < blob.size(); i += 3) {
    const int32_t s = blob[i], page = blob[i + 1], b = blob[i + 2];
    if (s < 0 || s >= m.max_seqs() || page < 0 || page >= p->stride || b < 0 ||
        b >= m.n_blocks())
      return PKV_ERR_STATE;
    const pkv::SeqMeta* q = m.seq(s);
    if (q && static_cast<size_t>(page) < q->pages.size() && q->pages[page] != b)
      return PKV_ERR_STATE;
  }
  return PKV_OK;
}

// The device page-table mirror rows of the batch against the host page
// tables (synchronizes the stream: the pending patches have been applied by
// the launches enqueued so far).
int32_t check_mirror(const pkv_pool* p, const int32_t* seqs, int32_t M, hipStream_t st) {
  if (hipStreamSynchronize(st) != hipSuccess) return PKV_ERR_DEVICE;
  std::vector<int32_t> row;
  for (int32_t r = 0; r < M; ++r) {
    const pkv::SeqMeta* q = p->meta.seq(seqs[r]);
    row.resize(q->pages.size());
    if (row.empty()) continue;
    if (hipMemcpy(row.data(), p->mirror + static_cast<int64_t>(seqs[r]) * p->stride,
                  row.size() * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
      return PKV_ERR_DEVICE;
    if (row != q->pages) return PKV_ERR_STATE;
  }
  return PKV_OK;
}

bool contig_valid(const pkv_contig* c) {
  return c && c->base_dev && c->n_slots > 0 && c->n_layers > 0 &&
         c->n_kv_heads > 0 && c->max_seq > 0 && c->head_dim > 0 &&
         c->block_size > 0 && (!c->rope || c->rope->head_dim == c->head_dim);
}

ContigMap make_contig_map(const pkv_contig* c, int32_t layer) {
  const int64_t G = c->n_kv_heads, S = c->max_seq, D = c->head_dim;
  ContigMap cm;
  cm.base = static_cast<float*>(c->base_dev);
  cm.head_stride = S * D;
  cm.v_off = G * S * D;
  cm.slot_stride = static_cast<int64_t>(c->n_layers) * 2 * G * S * D;
  cm.layer_off = static_cast<int64_t>(layer) * 2 * G * S * D;
  cm.page_stride = static_cast<int64_t>(c->block_size) * D;
  cm.block_size = c->block_size;
  return cm;
}

// Split partial results a batch needs (for n_q queries per row).
size_t partial_bytes(const RowPlan& pl, int32_t n_q, int32_t n_heads,
                     int32_t head_dim) {
  if (pl.max_parts <= 1) return 0;
  return static_cast<size_t>(pl.n_slots) * n_q * n_heads * (head_dim + 2) *
         sizeof(float);
}

// Which attention entry point: decode (one query per row), shared-prefix
// decode, verify (a few offset-causal queries per row, split over keys),
// prefill (a chunk).
enum class Kind { kDecode, kDecodeShared, kVerify, kPrefill };

// Whether this call runs a split kernel (and so needs a workspace).
bool uses_splits(Kind k, int32_t head_dim, int32_t group, int32_t block,
                 int32_t n_q) {
  if (k == Kind::kPrefill) return false;
  if (n_q == 1 && pkv::fast_decode_ok(head_dim, group, block)) return true;
  return k == Kind::kVerify && pkv::fast_verify_ok(head_dim, group, block, n_q);
}

// Launch attention.  rows_dev points at a row blob laid out by build_rows
// with plan `pl` for n_q rows.
template <class Map>
int32_t run_attention(DeviceCtx& dev, const Map& map, const int32_t* rows_dev,
                      const RowPlan& pl, const float* Q, float* out, void* ws,
                      int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                      int32_t n_q, int32_t causal, float scale, int32_t M,
                      int32_t block_size, Kind kind, const double2* rope,
                      hipStream_t st) {
  const int32_t group = n_heads / n_kv_heads;
  AttnArgs a;
  a.rows = reinterpret_cast<const RowDesc*>(rows_dev);
  a.items = reinterpret_cast<const int2*>(rows_dev + pl.item_off);
  a.Q = Q;
  a.out = out;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = ws ? static_cast<float*>(ws) +
                       static_cast<size_t>(pl.n_slots) * n_q * n_heads * head_dim
                 : nullptr;
  a.n_rows = M;
  a.n_heads = n_heads;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.n_q = n_q;
  a.causal = causal;
  a.qscale = static_cast<float>(static_cast<double>(scale) * kLog2e);
  a.n_items = pl.n_items;
  a.rope = rope;
  a.pre_items = rows_dev + pl.pre_off;
  a.groups = rows_dev + pl.group_off;
  a.members = rows_dev + pl.member_off;
  a.n_pre_items = pl.n_pre_items;
  hipError_t e;
  const char* mname = std::is_same<Map, PagedMap>::value ? "PagedMap" : "ContigMap";
  auto name = [](const char* kernel, std::initializer_list<std::string> args) {
    std::string n = std::string(kernel) + "<";
    for (const auto& x : args) n += (n.back() == '<' ? "" : ", ") + x;
    return n + ">";
  };
  if (uses_splits(kind, head_dim, group, block_size, n_q)) {
    if (pl.n_pre_items > 0) {
      // shared prefixes: the prefix work and the own-key splits in one launch
      if constexpr (std::is_same<Map, PagedMap>::value) {
        dev.form[PKV_K_PREFIX] = name("shared_decode_kernel", {std::to_string(group)});
        {
          DeviceCtx::ProfScope ps(&dev, PKV_K_PREFIX, st);
          if (pkv::launch_shared_decode(map, a, group, st) != hipSuccess)
            return PKV_ERR_DEVICE;
        }
        dev.form[PKV_K_MERGE] = "merge_kernel";
        DeviceCtx::ProfScope ps(&dev, PKV_K_MERGE, st);
        return dev_status(pkv::launch_merge(a, st));
      }
    }
    {
      const bool one = n_q == 1 && pkv::fast_decode_ok(head_dim, group, block_size);
      const bool deep = pl.max_split >= 4 * pkv::kDecodeSplit;
      const int kid = one ? PKV_K_DECODE : PKV_K_VERIFY;
      dev.form[kid] = one ? name("decode_fast_kernel", {std::to_string(group), mname,
                                                        deep ? "true" : "false"})
                          : name("verify_mfma_kernel",
                                 {n_q * group <= 16 ? "1" : "2", mname});
      DeviceCtx::ProfScope ps(&dev, kid, st);
      e = one ? pkv::launch_decode_fast(map, a, group, deep, st)
              : pkv::launch_verify_mfma(map, a, group, st);
      if (e != hipSuccess) return PKV_ERR_DEVICE;
    }
    if (pl.max_parts <= 1) return PKV_OK;
    dev.form[PKV_K_MERGE] = "merge_kernel";
    DeviceCtx::ProfScope ps(&dev, PKV_K_MERGE, st);
    return dev_status(pkv::launch_merge(a, st));
  }
  const bool decode = kind == Kind::kDecode || kind == Kind::kDecodeShared;
  if (!decode && pkv::fast_prefill_ok(head_dim, group, block_size)) {
    dev.form[PKV_K_PREFILL] = name("prefill_mfma_kernel", {std::to_string(group), mname});
    DeviceCtx::ProfScope ps(&dev, PKV_K_PREFILL, st);
    return dev_status(pkv::launch_prefill_mfma(map, a, group, st));
  }
  if (group > 16) return PKV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(group) * head_dim * 2 + group * 64 > 16384)
    return PKV_ERR_UNSUPPORTED;  // generic kernel keeps q and o in LDS
  dev.form[decode ? PKV_K_DECODE : PKV_K_PREFILL] = name("generic_kernel", {mname});
  DeviceCtx::ProfScope ps(&dev, decode ? PKV_K_DECODE : PKV_K_PREFILL, st);
  return dev_status(pkv::launch_generic(map, a, group, st));
}

// Rows of a call sit at positions seq_len .. seq_len + n - 1; with rotary
// embedding on, every one must have a row in the table.
int32_t pool_rope_check(const pkv_pool* p, const int32_t* seqs, int32_t M,
                        int32_t n) {
  if (!p->rope) return PKV_OK;
  for (int32_t r = 0; r < M; ++r)
    if (static_cast<int64_t>(p->meta.seq(seqs[r])->seq_len) + n >
        p->rope->max_positions)
      return PKV_ERR_CAPACITY;
  return PKV_OK;
}

const double2* rope_table(const pkv_rope* r) { return r ? r->table : nullptr; }

// Common front checks of the attention calls, in the pages' order.
int32_t attn_front_checks(int32_t M, int32_t n_q, int32_t n_heads,
                          int32_t n_kv_heads, int32_t head_dim) {
  if (M <= 0 || n_q <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0)
    return PKV_ERR_BAD_DIM;
  if (n_heads % n_kv_heads != 0) return PKV_ERR_BAD_GQA;
  return PKV_OK;
}

}  // namespace

// ===========================================================================
// Exported functions
// ===========================================================================

extern "C" {

const char* pkv_strerror(int32_t code) {
  switch (code) {
    case PKV_OK: return "ok";
    case PKV_ERR_BAD_DIM: return "bad dimension";
    case PKV_ERR_BAD_GQA: return "query heads not a multiple of kv heads";
    case PKV_ERR_SEQ: return "bad sequence or rows not ensured";
    case PKV_ERR_OOM: return "out of blocks";
    case PKV_ERR_CAPACITY: return "capacity exceeded";
    case PKV_ERR_BAD_ARG: return "bad argument";
    case PKV_ERR_DEVICE: return "HIP runtime error";
    case PKV_ERR_UNSUPPORTED: return "unsupported shape";
    case PKV_ERR_STATE: return "pool state check failed";
    default: return "unknown status";
  }
}

size_t pkv_pool_storage_bytes(int32_t n_blocks, int32_t block_size,
                              int32_t n_layers, int32_t n_kv_heads,
                              int32_t head_dim) {
  if (n_blocks <= 0 || block_size <= 0 || n_layers <= 0 || n_kv_heads <= 0 ||
      head_dim <= 0)
    return 0;
  return static_cast<size_t>(n_blocks) * n_layers * 2 * n_kv_heads *
         block_size * head_dim * sizeof(float);
}

pkv_pool* pkv_pool_new(int32_t n_blocks, int32_t block_size, int32_t n_layers,
                       int32_t n_kv_heads, int32_t head_dim, int32_t max_seqs,
                       void* storage_dev, size_t storage_bytes) {
  const size_t need = pkv_pool_storage_bytes(n_blocks, block_size, n_layers,
                                             n_kv_heads, head_dim);
  if (need == 0 || max_seqs <= 0) return nullptr;
  // the page-table mirror holds at least 64 int32-addressed entries per id
  if (static_cast<int64_t>(max_seqs) * pkv::PoolMeta::mirror_stride(1) > INT32_MAX)
    return nullptr;
  if (storage_dev) {
    if (storage_bytes < need) return nullptr;
    if (reinterpret_cast<uintptr_t>(storage_dev) % 256 != 0) return nullptr;
  }
  pkv_pool* p = new (std::nothrow) pkv_pool(n_blocks, block_size, n_layers,
                                            n_kv_heads, head_dim, max_seqs);
  if (!p) return nullptr;
  p->storage = static_cast<float*>(storage_dev);
  p->storage_bytes = storage_bytes;
  p->block_floats = static_cast<int64_t>(n_layers) * 2 * n_kv_heads *
                    block_size * head_dim;
  p->meta.track_patches(storage_dev != nullptr);
  return p;
}

void pkv_pool_free(pkv_pool* pool) { delete pool; }

pkv_rope* pkv_rope_new(int32_t head_dim, double log_base,
                       int32_t max_positions) {
  if (head_dim <= 0 || head_dim % 2 != 0 || !(log_base > 0.0) ||
      !std::isfinite(log_base) || max_positions <= 0)
    return nullptr;
  const int32_t half = head_dim / 2;
  // angle of pair i at position p: p * exp(-(2i / head_dim) * log_base)
  std::vector<double> inv(half);
  for (int32_t i = 0; i < half; ++i)
    inv[i] = std::exp(-(static_cast<double>(2 * i) / head_dim) * log_base);
  std::vector<double> host(static_cast<size_t>(max_positions) * half * 2);
  for (int32_t p = 0; p < max_positions; ++p) {
    double* row = host.data() + static_cast<size_t>(p) * half * 2;
    for (int32_t i = 0; i < half; ++i) {
      const double ang = static_cast<double>(p) * inv[i];
      row[2 * i] = std::cos(ang);
      row[2 * i + 1] = std::sin(ang);
    }
  }
  pkv_rope* r = new (std::nothrow) pkv_rope();
  if (!r) return nullptr;
  r->head_dim = head_dim;
  r->max_positions = max_positions;
  r->log_base = log_base;
  const size_t bytes = host.size() * sizeof(double);
  if (hipMalloc(&r->table, bytes) != hipSuccess) {
    r->table = nullptr;
    delete r;
    return nullptr;
  }
  if (hipMemcpy(r->table, host.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
    delete r;
    return nullptr;
  }
  return r;
}

void pkv_rope_free(pkv_rope* rope) { delete rope; }

int32_t pkv_pool_set_checks(pkv_pool* pool, int32_t level) {
  if (!pool) return PKV_ERR_BAD_ARG;
  if (level < 0 || level > 2) return PKV_ERR_BAD_ARG;
  pool->checks = level;
  return PKV_OK;
}

int32_t pkv_pool_set_rope(pkv_pool* pool, const pkv_rope* rope) {
  if (!pool) return PKV_ERR_BAD_ARG;
  if (rope && rope->head_dim != pool->meta.head_dim()) return PKV_ERR_BAD_DIM;
  pool->rope = rope;
  return PKV_OK;
}

int64_t pkv_alloc_block(pkv_pool* pool) {
  if (!pool) return -1;
  return pool->meta.alloc_block();
}

int32_t pkv_unref_block(pkv_pool* pool, int64_t id) {
  if (!pool) return PKV_ERR_BAD_ARG;
  return pool->meta.unref_block(id);
}

int32_t pkv_pool_set_free_order(pkv_pool* pool, const int64_t* ids, int32_t n) {
  if (!pool) return PKV_ERR_BAD_ARG;
  return pool->meta.set_free_order(ids, n);
}

int32_t pkv_seq_new(pkv_pool* pool, int32_t max_tokens) {
  if (!pool) return -PKV_ERR_BAD_ARG;
  return pool->meta.seq_new(max_tokens);
}

int32_t pkv_seq_free(pkv_pool* pool, int32_t seq) {
  if (!pool) return PKV_ERR_BAD_ARG;
  return pool->meta.seq_free(seq);
}

int32_t pkv_seq_fork(pkv_pool* pool, int32_t seq) {
  if (!pool) return -PKV_ERR_BAD_ARG;
  return pool->meta.seq_fork(seq);
}

int32_t pkv_seq_truncate(pkv_pool* pool, int32_t seq, int32_t new_len) {
  if (!pool) return PKV_ERR_BAD_ARG;
  return pool->meta.seq_truncate(seq, new_len);
}

int32_t pkv_ensure_append(pkv_pool* pool, const int32_t* seqs, int32_t M,
                          int32_t n_new, void* stream) {
  if (!pool) return PKV_ERR_BAD_ARG;
  std::vector<pkv::CowCopy> cows;
  const int32_t rc = pool->meta.ensure_append(seqs, M, n_new, &cows);
  if (rc != PKV_OK) return rc;
  if (pool->checks > 0) {
    if (int32_t c = check_state(pool, seqs, M, n_new, true)) return c;
    for (const auto& c : cows)
      if (c.src < 0 || c.src >= pool->meta.n_blocks() || c.dst < 0 ||
          c.dst >= pool->meta.n_blocks() || pool->meta.refcounts()[c.dst] != 1 ||
          pool->meta.refcounts()[c.src] < 1)
        return PKV_ERR_STATE;
  }
  if (cows.empty() || !pool->storage) return rc;
  // copy the privatised blocks on the stream, before any append
  const hipStream_t st = as_stream(stream);
  if (pool->dev.use_stream(st) != hipSuccess) return PKV_ERR_DEVICE;
  std::vector<int32_t> pairs;
  pairs.reserve(cows.size() * 2);
  for (const auto& c : cows) {
    pairs.push_back(c.src);
    pairs.push_back(c.dst);
  }
  int32_t* dev = nullptr;
  if (pool->dev.upload(kCow, pairs, {}, st, &dev) != hipSuccess) return PKV_ERR_DEVICE;
  pool->dev.form[PKV_K_COW] = pool->block_floats % 4 == 0 ? "cow_kernel<4>" : "cow_kernel<1>";
  DeviceCtx::ProfScope ps(&pool->dev, PKV_K_COW, st);
  return dev_status(pkv::launch_cow(pool->storage, dev,
                                    static_cast<int32_t>(cows.size()),
                                    pool->block_floats, st));
}

int32_t pkv_append_layer(pkv_pool* pool, const int32_t* seqs, int32_t M,
                         int32_t n_new, int32_t layer, const float* K_new_dev,
                         const float* V_new_dev, void* stream) {
  if (!pool) return PKV_ERR_BAD_ARG;
  if (M <= 0 || n_new <= 0) return PKV_ERR_BAD_DIM;
  if (int32_t rc = pool->meta.check_batch(seqs, M)) return rc;
  if (layer < 0 || layer >= pool->meta.n_layers()) return PKV_ERR_BAD_ARG;
  if (int32_t rc = pool->meta.check_append(seqs, M, n_new)) return rc;
  if (int32_t rc = pool_rope_check(pool, seqs, M, n_new)) return rc;
  if (pool->checks > 0)
    if (int32_t rc = check_state(pool, seqs, M, n_new, true)) return rc;
  if (!pool->storage) return PKV_OK;  // metadata-only pool: checks only
  if (!K_new_dev || !V_new_dev) return PKV_ERR_BAD_ARG;
  const hipStream_t st = as_stream(stream);
  if (pool->dev.use_stream(st) != hipSuccess) return PKV_ERR_DEVICE;
  const int32_t* rows = nullptr;
  // build the blob the following attention call will want (shared-prefix
  // groups or not, as the last attention call), so both share one upload
  const int32_t shared_heads =
      pool->last_shared && n_new == 1 ? pool->shared_heads : 0;
  // one row per sequence: the rows name the blocks they land in, so the
  // append kernel also applies the pending page-table patches and brings
  // the step's row blob to the device
  std::vector<int64_t> key;
  if (plan_rows(pool, seqs, M, n_new, shared_heads, st, &key) != hipSuccess)
    return PKV_ERR_DEVICE;
  // after plan_rows: sizing the mirror may have moved it
  const PagedMap pm = make_paged_map(pool, layer);
  const int32_t kv_dim = pool->meta.n_kv_heads() * pool->meta.head_dim();
  if (n_new == 1) {
    // A blob that must go to the device and fits the kernel's arguments
    // travels in them: the launch reads no host memory and needs no
    // staging slot.
    if (pool->rows.size() <= static_cast<size_t>(pkv::kIntChunk) &&
        (!pool->dev.holds(kRows, key) || !pool->meta.patches().empty())) {
      if (pool->checks > 0)
        if (int32_t rc = check_blob(pool, seqs, M, pool->rows, pool->patch_off)) return rc;
      const int32_t n_blob = static_cast<int32_t>(pool->rows.size());
      const int32_t n_patch = static_cast<int32_t>((n_blob - pool->patch_off) / 3);
      int32_t* d = nullptr;
      if (pool->dev.claim(kRows, n_blob * sizeof(int32_t), key, st, &d) != hipSuccess)
        return PKV_ERR_DEVICE;
      pool->meta.patches().clear();
      pool->rows_key = key;
      pool->dev.form[PKV_K_APPEND] = std::string("append_inline_kernel<") +
                                     (span_of(pool) % 4 == 0 ? "4" : "1") + ", " +
                                     (pool->rope ? "true" : "false") + ">";
      hipError_t e;
      {
        DeviceCtx::ProfScope ps(&pool->dev, PKV_K_APPEND, st);
        e = pkv::launch_append_inline(pm, K_new_dev, V_new_dev, M, kv_dim,
                                      pool->meta.head_dim(), rope_table(pool->rope),
                                      pool->mirror, pool->stride, d, pool->rows.data(),
                                      n_blob, static_cast<int32_t>(pool->patch_off), n_patch,
                                      st);
      }
      if (e != hipSuccess) {  // neither the blob nor the patches reached the device
        pool->dev.buf[kRows].valid = false;
        pool->rows_key.clear();
        pool->mirror_stale = true;
      }
      return dev_status(e);
    }
  }
  pkv::PatchArgs pa{};
  if (rows_to_device(pool, key, st, &rows, n_new == 1 ? &pa : nullptr) != hipSuccess)
    return PKV_ERR_DEVICE;
  if (pool->checks > 0)
    if (int32_t rc = check_blob(pool, seqs, M, pool->rows, pool->patch_off)) return rc;
  pool->dev.form[PKV_K_APPEND] = std::string("append_kernel<") +
                                 (span_of(pool) % 4 == 0 ? "4" : "1") + ", PagedMap, " +
                                 (pool->rope ? "true" : "false") + ", " +
                                 (n_new == 1 ? "true" : "false") + ">";
  if (n_new == 1) {
    hipError_t e;
    {
      DeviceCtx::ProfScope ps(&pool->dev, PKV_K_APPEND, st);
      e = pkv::launch_append_one(pm, reinterpret_cast<const RowDesc*>(rows), K_new_dev,
                                 V_new_dev, M, kv_dim, pool->meta.head_dim(),
                                 rope_table(pool->rope), pa, st);
    }
    if (e == hipSuccess && pa.n_copy > 0) e = pool->dev.staged(st);
    if (e != hipSuccess) {  // neither the blob nor the patches reached the device
      pool->dev.buf[kRows].valid = false;
      pool->rows_key.clear();
      if (pa.n > 0) pool->mirror_stale = true;
    }
    return dev_status(e);
  }
  DeviceCtx::ProfScope ps(&pool->dev, PKV_K_APPEND, st);
  return dev_status(pkv::launch_append(
      pm, reinterpret_cast<const RowDesc*>(rows), K_new_dev, V_new_dev, M, n_new,
      kv_dim, pool->meta.head_dim(), rope_table(pool->rope), st));
}

int32_t pkv_advance(pkv_pool* pool, const int32_t* seqs, int32_t M, int32_t n) {
  if (!pool) return PKV_ERR_BAD_ARG;
  return pool->meta.advance(seqs, M, n);
}

namespace {

// Query heads per kv head to group shared prefixes with, or 0 (no grouping:
// another kind of call, or a shape the split kernels do not cover).
int32_t shared_heads_for(const pkv_pool* pool, Kind kind, int32_t n_heads) {
  const auto& m = pool->meta;
  const int32_t group = n_heads / m.n_kv_heads();
  if (kind != Kind::kDecodeShared || !pkv::fast_decode_ok(m.head_dim(), group, m.block_size()))
    return 0;
  return group;
}

size_t pool_workspace_bytes(pkv_pool* pool, const int32_t* seqs, int32_t M,
                            int32_t n_q, int32_t n_heads, Kind kind) {
  if (!pool || M <= 0 || n_q <= 0 || n_heads <= 0) return static_cast<size_t>(-1);
  const auto& m = pool->meta;
  if (n_heads % m.n_kv_heads() != 0) return static_cast<size_t>(-1);
  if (m.check_batch(seqs, M) != PKV_OK) return static_cast<size_t>(-1);
  if (!uses_splits(kind, m.head_dim(), n_heads / m.n_kv_heads(), m.block_size(), n_q))
    return 0;
  const int32_t sh = shared_heads_for(pool, kind, n_heads);
  SharedPlan sp;
  if (sh > 0) find_shared(m, seqs, M, sh, &sp);
  std::vector<int32_t> tmp;
  const RowPlan pl = build_rows(tmp, M, n_q, sh > 0 && !sp.groups.empty(), [&](int32_t r) {
    RowIn in;
    in.start = m.seq(seqs[r])->seq_len;
    if (sh > 0) {
      in.k_off = sp.k_off[r];
      in.n_pre = sp.n_pre[r];
    }
    return in;
  });
  return partial_bytes(pl, n_q, n_heads, m.head_dim());
}

// The three paged attention entry points: checks in the pages' order, then
// the rows upload and the launch.
int32_t paged_attention(pkv_pool* pool, const int32_t* seqs, int32_t M,
                        int32_t n_q, int32_t layer, int32_t n_heads,
                        int32_t n_kv_heads, int32_t head_dim, const float* Q_dev,
                        int32_t causal, float scale, float* out_dev, void* ws_dev,
                        size_t ws_bytes, Kind kind, void* stream) {
  if (!pool) return PKV_ERR_BAD_ARG;
  if (int32_t rc = attn_front_checks(M, n_q, n_heads, n_kv_heads, head_dim)) return rc;
  const auto& m = pool->meta;
  if (n_kv_heads != m.n_kv_heads() || head_dim != m.head_dim()) return PKV_ERR_BAD_DIM;
  if (int32_t rc = m.check_batch(seqs, M)) return rc;
  if (layer < 0 || layer >= m.n_layers()) return PKV_ERR_BAD_ARG;
  if (!pool->storage) return PKV_ERR_BAD_ARG;
  if (int32_t rc = m.check_rows(seqs, M, n_q)) return rc;
  if (int32_t rc = pool_rope_check(pool, seqs, M, n_q)) return rc;
  if (!Q_dev || !out_dev) return PKV_ERR_BAD_ARG;
  if (kind != Kind::kPrefill) {
    const size_t need = pool_workspace_bytes(pool, seqs, M, n_q, n_heads, kind);
    if (need > 0 && (!ws_dev || ws_bytes < need)) return PKV_ERR_BAD_ARG;
  }
  const hipStream_t st = as_stream(stream);
  if (pool->dev.use_stream(st) != hipSuccess) return PKV_ERR_DEVICE;
  const int32_t sh = shared_heads_for(pool, kind, n_heads);
  if (kind == Kind::kDecode || kind == Kind::kDecodeShared) {
    pool->last_shared = sh > 0;
    pool->shared_heads = sh;
  }
  if (pool->checks > 0)
    if (int32_t rc = check_state(pool, seqs, M, n_q, false)) return rc;
  const int32_t* rows = nullptr;
  if (pool_rows(pool, seqs, M, n_q, sh, st, &rows) != hipSuccess) return PKV_ERR_DEVICE;
  if (pool->checks > 0)
    if (int32_t rc = check_blob(pool, seqs, M, pool->rows, pool->patch_off)) return rc;
  if (pool->checks > 1)
    if (int32_t rc = check_mirror(pool, seqs, M, st)) return rc;
  const PagedMap pm = make_paged_map(pool, layer);
  return run_attention(pool->dev, pm, rows, pool->plan, Q_dev, out_dev, ws_dev,
                       n_heads, n_kv_heads, head_dim, n_q, causal, scale, M,
                       m.block_size(), kind, rope_table(pool->rope), st);
}

}  // namespace

size_t pkv_decode_workspace_bytes(pkv_pool* pool, const int32_t* seqs,
                                  int32_t M, int32_t n_heads) {
  return pool_workspace_bytes(pool, seqs, M, 1, n_heads, Kind::kDecode);
}

size_t pkv_verify_workspace_bytes(pkv_pool* pool, const int32_t* seqs,
                                  int32_t M, int32_t n_q, int32_t n_heads) {
  return pool_workspace_bytes(pool, seqs, M, n_q, n_heads, Kind::kVerify);
}

size_t pkv_decode_shared_workspace_bytes(pkv_pool* pool, const int32_t* seqs,
                                         int32_t M, int32_t n_heads) {
  return pool_workspace_bytes(pool, seqs, M, 1, n_heads, Kind::kDecodeShared);
}

int32_t pkv_attn_paged_decode_shared(pkv_pool* pool, const int32_t* seqs, int32_t M,
                                     int32_t layer, int32_t n_heads,
                                     int32_t n_kv_heads, int32_t head_dim,
                                     const float* Q_dev, float scale, float* out_dev,
                                     void* ws_dev, size_t ws_bytes, void* stream) {
  return paged_attention(pool, seqs, M, 1, layer, n_heads, n_kv_heads, head_dim,
                         Q_dev, 1, scale, out_dev, ws_dev, ws_bytes,
                         Kind::kDecodeShared, stream);
}

int32_t pkv_attn_paged_decode(pkv_pool* pool, const int32_t* seqs, int32_t M,
                              int32_t layer, int32_t n_heads,
                              int32_t n_kv_heads, int32_t head_dim,
                              const float* Q_dev, float scale, float* out_dev,
                              void* ws_dev, size_t ws_bytes, void* stream) {
  return paged_attention(pool, seqs, M, 1, layer, n_heads, n_kv_heads, head_dim,
                         Q_dev, 1, scale, out_dev, ws_dev, ws_bytes, Kind::kDecode,
                         stream);
}

namespace {

// pkv_attn_with_paged_decode and its shared-prefix form: every check of
// both calls first, in the pages' order, so an error leaves the pool as it
// was; then append_layer's launch and the attention's.
int32_t with_paged_decode(pkv_pool* pool, const int32_t* seqs, int32_t M, int32_t layer,
                          int32_t n_heads, int32_t n_kv_heads, int32_t head_dim,
                          const float* Q_dev, const float* K_new_dev, const float* V_new_dev,
                          float scale, float* out_dev, void* ws_dev, size_t ws_bytes,
                          Kind kind, void* stream) {
  if (!pool) return PKV_ERR_BAD_ARG;
  if (int32_t rc = attn_front_checks(M, 1, n_heads, n_kv_heads, head_dim)) return rc;
  const auto& m = pool->meta;
  if (n_kv_heads != m.n_kv_heads() || head_dim != m.head_dim()) return PKV_ERR_BAD_DIM;
  if (int32_t rc = m.check_batch(seqs, M)) return rc;
  if (layer < 0 || layer >= m.n_layers()) return PKV_ERR_BAD_ARG;
  if (int32_t rc = m.check_append(seqs, M, 1)) return rc;
  if (int32_t rc = pool_rope_check(pool, seqs, M, 1)) return rc;
  if (!pool->storage) return PKV_ERR_BAD_ARG;
  if (!Q_dev || !out_dev || !K_new_dev || !V_new_dev) return PKV_ERR_BAD_ARG;
  const size_t need = pool_workspace_bytes(pool, seqs, M, 1, n_heads, kind);
  if (need > 0 && (!ws_dev || ws_bytes < need)) return PKV_ERR_BAD_ARG;
  if (int32_t rc = pkv_append_layer(pool, seqs, M, 1, layer, K_new_dev, V_new_dev, stream))
    return rc;
  return paged_attention(pool, seqs, M, 1, layer, n_heads, n_kv_heads, head_dim, Q_dev, 1,
                         scale, out_dev, ws_dev, ws_bytes, kind, stream);
}

}  // namespace

int32_t pkv_attn_with_paged_decode(pkv_pool* pool, const int32_t* seqs, int32_t M,
                                   int32_t layer, int32_t n_heads, int32_t n_kv_heads,
                                   int32_t head_dim, const float* Q_dev,
                                   const float* K_new_dev, const float* V_new_dev,
                                   float scale, float* out_dev, void* ws_dev,
                                   size_t ws_bytes, void* stream) {
  return with_paged_decode(pool, seqs, M, layer, n_heads, n_kv_heads, head_dim, Q_dev,
                           K_new_dev, V_new_dev, scale, out_dev, ws_dev, ws_bytes,
                           Kind::kDecode, stream);
}

int32_t pkv_attn_with_paged_decode_shared(pkv_pool* pool, const int32_t* seqs, int32_t M,
                                          int32_t layer, int32_t n_heads,
                                          int32_t n_kv_heads, int32_t head_dim,
                                          const float* Q_dev, const float* K_new_dev,
                                          const float* V_new_dev, float scale,
                                          float* out_dev, void* ws_dev, size_t ws_bytes,
                                          void* stream) {
  return with_paged_decode(pool, seqs, M, layer, n_heads, n_kv_heads, head_dim, Q_dev,
                           K_new_dev, V_new_dev, scale, out_dev, ws_dev, ws_bytes,
                           Kind::kDecodeShared, stream);
}

int32_t pkv_attn_paged_decode_noalloc(pkv_pool* pool, const int32_t* seqs, int32_t M,
                                      int32_t layer, int32_t n_heads, int32_t n_kv_heads,
                                      int32_t head_dim, const float* Q_dev, float scale,
                                      float* out_dev, void* stream) {
  // the checks of pkv_attn_paged_decode, in the same order (no workspace)
  if (!pool) return PKV_ERR_BAD_ARG;
  if (int32_t rc = attn_front_checks(M, 1, n_heads, n_kv_heads, head_dim)) return rc;
  auto& m = pool->meta;
  if (n_kv_heads != m.n_kv_heads() || head_dim != m.head_dim()) return PKV_ERR_BAD_DIM;
  if (int32_t rc = m.check_batch(seqs, M)) return rc;
  if (layer < 0 || layer >= m.n_layers()) return PKV_ERR_BAD_ARG;
  if (!pool->storage) return PKV_ERR_BAD_ARG;
  if (int32_t rc = m.check_rows(seqs, M, 1)) return rc;
  if (int32_t rc = pool_rope_check(pool, seqs, M, 1)) return rc;
  if (!Q_dev || !out_dev) return PKV_ERR_BAD_ARG;
  // growing the page-table mirror would allocate
  if (!pool->mirror || pkv::PoolMeta::mirror_stride(m.max_pages_seen()) > pool->stride)
    return PKV_ERR_UNSUPPORTED;
  if (pool->checks > 0)
    if (int32_t rc = check_state(pool, seqs, M, 1, false)) return rc;
  if (pool->mirror_stale) queue_all_pages(pool);  // host work only
  RowPlan plan;
  size_t patch_off = 0;
  build_blob(pool, seqs, M, 1, 0, pool->na_rows, &plan, &patch_off);
  if (pool->checks > 0)
    if (int32_t rc = check_blob(pool, seqs, M, pool->na_rows, patch_off)) return rc;
  const int32_t group = n_heads / n_kv_heads;
  const size_t part = uses_splits(Kind::kDecode, head_dim, group, m.block_size(), 1)
                          ? partial_bytes(plan, 1, n_heads, head_dim)
                          : 0;
  if (pool->na_rows.size() * sizeof(int32_t) > pkv::kNoAllocBlobBytes ||
      part > pkv::kNoAllocPartBytes)
    return PKV_ERR_CAPACITY;
  void* base = nullptr;
  if (pkv::noalloc_scratch(&base) != hipSuccess) return PKV_ERR_DEVICE;
  const hipStream_t st = as_stream(stream);
  if (pool->dev.use_stream(st) != hipSuccess) return PKV_ERR_DEVICE;
  int32_t* blob = static_cast<int32_t*>(base);
  float* ws = reinterpret_cast<float*>(static_cast<char*>(base) + pkv::kNoAllocBlobBytes);
  if (pkv::launch_write_ints(blob, pool->na_rows.data(), pool->na_rows.size(), st) !=
      hipSuccess)
    return PKV_ERR_DEVICE;
  const int32_t n_patch = static_cast<int32_t>((pool->na_rows.size() - patch_off) / 3);
  if (n_patch > 0) {
    if (pkv::launch_patch(pool->mirror, blob + patch_off, n_patch, pool->stride, st) !=
        hipSuccess)
      return PKV_ERR_DEVICE;
    m.patches().clear();
  }
  if (pool->checks > 1)
    if (int32_t rc = check_mirror(pool, seqs, M, st)) return rc;
  pool->last_shared = false;
  pool->shared_heads = 0;
  pool->dev.no_new_events = true;
  const int32_t rc = run_attention(pool->dev, make_paged_map(pool, layer), blob, plan, Q_dev,
                                   out_dev, ws, n_heads, n_kv_heads, head_dim, 1, 1, scale,
                                   M, m.block_size(), Kind::kDecode, rope_table(pool->rope),
                                   st);
  pool->dev.no_new_events = false;
  return rc;
}

int32_t pkv_attn_paged_verify(pkv_pool* pool, const int32_t* seqs, int32_t M,
                              int32_t n_q, int32_t layer, int32_t n_heads,
                              int32_t n_kv_heads, int32_t head_dim,
                              const float* Q_dev, float scale, float* out_dev,
                              void* ws_dev, size_t ws_bytes, void* stream) {
  return paged_attention(pool, seqs, M, n_q, layer, n_heads, n_kv_heads, head_dim,
                         Q_dev, 1, scale, out_dev, ws_dev, ws_bytes, Kind::kVerify,
                         stream);
}

int32_t pkv_attn_paged_prefill(pkv_pool* pool, const int32_t* seqs, int32_t M,
                               int32_t n_q, int32_t layer, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim,
                               const float* Q_dev, int32_t causal, float scale,
                               float* out_dev, void* stream) {
  return paged_attention(pool, seqs, M, n_q, layer, n_heads, n_kv_heads, head_dim,
                         Q_dev, causal ? 1 : 0, scale, out_dev, nullptr, 0,
                         Kind::kPrefill, stream);
}

// ---------------------------------------------------------------- contiguous

size_t pkv_contig_bytes(int32_t n_slots, int32_t n_layers, int32_t n_kv_heads,
                        int32_t max_seq, int32_t head_dim) {
  if (n_slots <= 0 || n_layers <= 0 || n_kv_heads <= 0 || max_seq <= 0 ||
      head_dim <= 0)
    return 0;
  return static_cast<size_t>(n_slots) * n_layers * 2 * n_kv_heads * max_seq *
         head_dim * sizeof(float);
}

namespace {

// Rows for contiguous calls (pt_off = slot); checks slots and lengths.
int32_t contig_rows(const pkv_contig* c, const int32_t* slots,
                    const int32_t* seq_lens, int32_t M, int32_t n,
                    std::vector<int32_t>& rows, RowPlan* pl) {
  if (!slots || !seq_lens) return PKV_ERR_BAD_ARG;
  for (int32_t r = 0; r < M; ++r) {
    if (slots[r] < 0 || slots[r] >= c->n_slots) return PKV_ERR_SEQ;
    for (int32_t r2 = 0; r2 < r; ++r2)
      if (slots[r2] == slots[r]) return PKV_ERR_SEQ;
    if (seq_lens[r] < 0) return PKV_ERR_BAD_ARG;
    if (static_cast<int64_t>(seq_lens[r]) + n > c->max_seq) return PKV_ERR_SEQ;
    if (c->rope && static_cast<int64_t>(seq_lens[r]) + n > c->rope->max_positions)
      return PKV_ERR_CAPACITY;
  }
  *pl = build_rows(rows, M, n, false, [&](int32_t r) {
    RowIn in;
    in.start = seq_lens[r];
    in.pt_off = slots[r];
    return in;
  });
  return PKV_OK;
}

}  // namespace

int32_t pkv_contig_append(const pkv_contig* cache, const int32_t* slots,
                          const int32_t* seq_lens, int32_t M, int32_t n_new,
                          int32_t layer, const float* K_new_dev,
                          const float* V_new_dev, void* stream) {
  if (!contig_valid(cache)) return PKV_ERR_BAD_ARG;
  if (M <= 0 || n_new <= 0) return PKV_ERR_BAD_DIM;
  if (layer < 0 || layer >= cache->n_layers) return PKV_ERR_BAD_ARG;
  if (!K_new_dev || !V_new_dev) return PKV_ERR_BAD_ARG;
  std::lock_guard<std::mutex> g(contig_mutex());
  std::vector<int32_t> rows;
  RowPlan pl;
  if (int32_t rc = contig_rows(cache, slots, seq_lens, M, n_new, rows, &pl)) return rc;
  DeviceCtx& dev = contig_ctx();
  const hipStream_t st = as_stream(stream);
  if (dev.use_stream(st) != hipSuccess) return PKV_ERR_DEVICE;
  int32_t* d = nullptr;
  if (dev.upload(kRows, rows, {}, st, &d) != hipSuccess) return PKV_ERR_DEVICE;
  const ContigMap cm = make_contig_map(cache, layer);
  return dev_status(pkv::launch_append(cm, reinterpret_cast<const RowDesc*>(d),
                                       K_new_dev, V_new_dev, M, n_new,
                                       cache->n_kv_heads * cache->head_dim,
                                       cache->head_dim, rope_table(cache->rope),
                                       st));
}

namespace {

size_t contig_workspace_bytes(const int32_t* seq_lens, int32_t M, int32_t n_q,
                              int32_t n_heads, int32_t n_kv_heads,
                              int32_t head_dim, int32_t block_size, Kind kind) {
  if (!seq_lens || M <= 0 || n_q <= 0 || n_heads <= 0 || n_kv_heads <= 0 ||
      head_dim <= 0 || n_heads % n_kv_heads != 0)
    return static_cast<size_t>(-1);
  for (int32_t r = 0; r < M; ++r)
    if (seq_lens[r] < 0) return static_cast<size_t>(-1);
  if (!uses_splits(kind, head_dim, n_heads / n_kv_heads, block_size, n_q)) return 0;
  std::vector<int32_t> tmp;
  const RowPlan pl = build_rows(tmp, M, n_q, false, [&](int32_t r) {
    RowIn in;
    in.start = seq_lens[r];
    return in;
  });
  return partial_bytes(pl, n_q, n_heads, head_dim);
}

int32_t contig_attention(const pkv_contig* cache, const int32_t* slots,
                         const int32_t* seq_lens, int32_t M, int32_t n_q,
                         int32_t layer, int32_t n_heads, int32_t n_kv_heads,
                         int32_t head_dim, const float* Q_dev, int32_t causal,
                         float scale, float* out_dev, void* ws_dev,
                         size_t ws_bytes, Kind kind, void* stream) {
  if (int32_t rc = attn_front_checks(M, n_q, n_heads, n_kv_heads, head_dim)) return rc;
  if (!contig_valid(cache)) return PKV_ERR_BAD_ARG;
  if (n_kv_heads != cache->n_kv_heads || head_dim != cache->head_dim) return PKV_ERR_BAD_DIM;
  if (layer < 0 || layer >= cache->n_layers) return PKV_ERR_BAD_ARG;
  if (!Q_dev || !out_dev) return PKV_ERR_BAD_ARG;
  std::lock_guard<std::mutex> g(contig_mutex());
  std::vector<int32_t> rows;
  RowPlan pl;
  if (int32_t rc = contig_rows(cache, slots, seq_lens, M, n_q, rows, &pl)) return rc;
  const int32_t group = n_heads / n_kv_heads;
  if (uses_splits(kind, head_dim, group, cache->block_size, n_q)) {
    const size_t need = partial_bytes(pl, n_q, n_heads, head_dim);
    if (need > 0 && (!ws_dev || ws_bytes < need)) return PKV_ERR_BAD_ARG;
  }
  DeviceCtx& dev = contig_ctx();
  const hipStream_t st = as_stream(stream);
  if (dev.use_stream(st) != hipSuccess) return PKV_ERR_DEVICE;
  int32_t* d = nullptr;
  if (dev.upload(kRows, rows, {}, st, &d) != hipSuccess) return PKV_ERR_DEVICE;
  const ContigMap cm = make_contig_map(cache, layer);
  return run_attention(dev, cm, d, pl, Q_dev, out_dev, ws_dev, n_heads,
                       n_kv_heads, head_dim, n_q, causal, scale, M,
                       cache->block_size, kind, rope_table(cache->rope), st);
}

}  // namespace

size_t pkv_contig_decode_workspace_bytes(const int32_t* seq_lens, int32_t M,
                                         int32_t n_heads, int32_t n_kv_heads,
                                         int32_t head_dim) {
  return contig_workspace_bytes(seq_lens, M, 1, n_heads, n_kv_heads, head_dim, 16,
                                Kind::kDecode);
}

size_t pkv_contig_verify_workspace_bytes(const int32_t* seq_lens, int32_t M,
                                         int32_t n_q, int32_t n_heads,
                                         int32_t n_kv_heads, int32_t head_dim) {
  return contig_workspace_bytes(seq_lens, M, n_q, n_heads, n_kv_heads, head_dim, 16,
                                Kind::kVerify);
}

int32_t pkv_attn_contig_decode(const pkv_contig* cache, const int32_t* slots,
                               const int32_t* seq_lens, int32_t M,
                               int32_t layer, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim,
                               const float* Q_dev, float scale, float* out_dev,
                               void* ws_dev, size_t ws_bytes, void* stream) {
  return contig_attention(cache, slots, seq_lens, M, 1, layer, n_heads,
                          n_kv_heads, head_dim, Q_dev, 1, scale, out_dev,
                          ws_dev, ws_bytes, Kind::kDecode, stream);
}

int32_t pkv_attn_contig_verify(const pkv_contig* cache, const int32_t* slots,
                               const int32_t* seq_lens, int32_t M, int32_t n_q,
                               int32_t layer, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim,
                               const float* Q_dev, float scale, float* out_dev,
                               void* ws_dev, size_t ws_bytes, void* stream) {
  return contig_attention(cache, slots, seq_lens, M, n_q, layer, n_heads,
                          n_kv_heads, head_dim, Q_dev, 1, scale, out_dev,
                          ws_dev, ws_bytes, Kind::kVerify, stream);
}

int32_t pkv_attn_contig_prefill(const pkv_contig* cache, const int32_t* slots,
                                const int32_t* seq_lens, int32_t M,
                                int32_t n_q, int32_t layer, int32_t n_heads,
                                int32_t n_kv_heads, int32_t head_dim,
                                const float* Q_dev, int32_t causal,
                                float scale, float* out_dev, void* stream) {
  return contig_attention(cache, slots, seq_lens, M, n_q, layer, n_heads,
                          n_kv_heads, head_dim, Q_dev, causal ? 1 : 0, scale,
                          out_dev, nullptr, 0, Kind::kPrefill, stream);
}

// ------------------------------------------------------------- introspection

int32_t pkv_seq_len(pkv_pool* pool, int32_t seq) {
  if (!pool) return -PKV_ERR_BAD_ARG;
  const pkv::SeqMeta* q = pool->meta.seq(seq);
  return q ? q->seq_len : -PKV_ERR_SEQ;
}

int32_t pkv_seq_pages(pkv_pool* pool, int32_t seq, int64_t* out, int32_t cap) {
  if (!pool) return -PKV_ERR_BAD_ARG;
  const pkv::SeqMeta* q = pool->meta.seq(seq);
  if (!q) return -PKV_ERR_SEQ;
  const int32_t n = static_cast<int32_t>(q->pages.size());
  for (int32_t i = 0; i < n && i < cap && out; ++i) out[i] = q->pages[i];
  return n;
}

int32_t pkv_pool_refcounts(pkv_pool* pool, int32_t* out) {
  if (!pool) return -PKV_ERR_BAD_ARG;
  const auto& r = pool->meta.refcounts();
  if (out) std::memcpy(out, r.data(), r.size() * sizeof(int32_t));
  return static_cast<int32_t>(r.size());
}

int32_t pkv_pool_free_stack(pkv_pool* pool, int64_t* out, int32_t cap) {
  if (!pool) return -PKV_ERR_BAD_ARG;
  const auto& f = pool->meta.free_stack();
  const int32_t n = static_cast<int32_t>(f.size());
  for (int32_t i = 0; i < n && i < cap && out; ++i) out[i] = f[i];
  return n;
}

// ------------------------------------------------------------------ timing

int32_t pkv_profile_enable(pkv_pool* pool, int32_t on) {
  if (!pool) return PKV_ERR_BAD_ARG;
  if (pool->dev.used && hipStreamSynchronize(pool->dev.last_stream) != hipSuccess)
    return PKV_ERR_DEVICE;
  pool->dev.clear_prof();
  pool->dev.prof_on = on != 0;
  if (on && pool->storage &&
      pool->dev.reserve_events(kProfReserve, pool->dev.last_stream) != hipSuccess)
    return PKV_ERR_DEVICE;
  return PKV_OK;
}

int32_t pkv_profile_kernels(pkv_pool* pool, uint32_t mask) {
  if (!pool) return PKV_ERR_BAD_ARG;
  pool->dev.prof_mask = mask;
  return PKV_OK;
}

int32_t pkv_profile_read(pkv_pool* pool, int32_t kernel, double* total_ms,
                         int64_t* launches) {
  if (!pool || kernel < 0 || kernel >= PKV_K_COUNT || !total_ms || !launches)
    return PKV_ERR_BAD_ARG;
  double sum = 0.0;
  for (auto& e : pool->dev.prof_ev[kernel]) {
    if (hipEventSynchronize(e.second) != hipSuccess) return PKV_ERR_DEVICE;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, e.first, e.second) != hipSuccess) return PKV_ERR_DEVICE;
    sum += ms;
  }
  *total_ms = sum;
  *launches = static_cast<int64_t>(pool->dev.prof_ev[kernel].size());
  return PKV_OK;
}

int32_t pkv_profile_kernel_name(pkv_pool* pool, int32_t kernel, char* out, int32_t cap) {
  if (!pool || kernel < 0 || kernel >= PKV_K_COUNT || (cap > 0 && !out))
    return -PKV_ERR_BAD_ARG;
  const std::string& f = pool->dev.form[kernel];
  if (cap > 0) {
    const size_t n = std::min<size_t>(f.size(), static_cast<size_t>(cap) - 1);
    std::memcpy(out, f.data(), n);
    out[n] = '\0';
  }
  return static_cast<int32_t>(f.size());
}

int32_t pkv_profile_samples(pkv_pool* pool, int32_t kernel, float* out_ms,
                            int32_t cap) {
  if (!pool || kernel < 0 || kernel >= PKV_K_COUNT || (cap > 0 && !out_ms))
    return -PKV_ERR_BAD_ARG;
  const auto& ev = pool->dev.prof_ev[kernel];
  const int32_t n = static_cast<int32_t>(ev.size());
  for (int32_t i = 0; i < n && i < cap; ++i) {
    if (hipEventSynchronize(ev[i].second) != hipSuccess) return -PKV_ERR_DEVICE;
    if (hipEventElapsedTime(&out_ms[i], ev[i].first, ev[i].second) != hipSuccess)
      return -PKV_ERR_DEVICE;
  }
  return n;
}

}  // extern "C"

// C ABI of libpkv (declared in include/pkv.h): argument checks, the
// per-call batch descriptor upload, kernel launches and kernel timing.
//
// Descriptor upload.  Each device call needs its batch's lengths, page ids
// and work list on the GPU.  The host packs them into one int32 blob, copies
// it into a pinned staging slot and enqueues one H2D copy into a
// library-owned device buffer (one per call kind) on the caller's stream,
// so the kernels that follow are stream-ordered after it.  Staging slots
// rotate through a ring; a slot is rewritten only after the event recorded
// behind its previous copy has completed.  A blob that is identical to what
// its kind's device buffer already holds (same pool version, same batch, same
// call shape) is not sent again, so the layers of one step share one upload.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "device.hpp"
#include "pkv.h"
#include "pool_meta.hpp"

namespace {

using pkv::AttnArgs;
using pkv::ContigMap;
using pkv::Item;
using pkv::OutDesc;
using pkv::PagedMap;
using pkv::RowDesc;

constexpr double kLog2e = 1.4426950408889634074;
constexpr int kStageSlots = 8;
constexpr int32_t kNoSplit = 1 << 30;

enum Kind { kAppend = 0, kDecode = 1, kPrefill = 2, kCow = 3, kNumKinds = 4 };

inline int32_t ceil_div(int64_t a, int64_t b) {
  return static_cast<int32_t>((a + b - 1) / b);
}

// Pinned host staging ring + per-kind device buffers + upload cache.
struct DeviceCtx {
  struct Slot {
    void* host = nullptr;
    size_t cap = 0;
    hipEvent_t ev = nullptr;
    bool pending = false;
  };
  struct Buf {
    void* ptr = nullptr;
    size_t cap = 0;
    bool valid = false;  // holds `key`
    std::vector<int64_t> key;
  };
  Slot slot[kStageSlots];
  int next = 0;
  Buf buf[kNumKinds];
  hipStream_t last_stream = nullptr;
  bool used = false;

  // profiling
  bool prof_on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> prof_ev[PKV_K_COUNT];

  ~DeviceCtx() { release(); }

  void release() {
    if (used) (void)hipStreamSynchronize(last_stream);
    for (auto& s : slot) {
      if (s.ev) (void)hipEventSynchronize(s.ev), (void)hipEventDestroy(s.ev);
      if (s.host) (void)hipHostFree(s.host);
      s = Slot();
    }
    for (auto& b : buf) {
      if (b.ptr) (void)hipFree(b.ptr);
      b = Buf();
    }
    clear_prof();
    used = false;
  }

  void clear_prof() {
    for (auto& v : prof_ev) {
      for (auto& e : v) {
        (void)hipEventDestroy(e.first);
        (void)hipEventDestroy(e.second);
      }
      v.clear();
    }
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

  // Copy blob into buffer `kind` (unless it already holds `key`).
  hipError_t upload(int kind, const std::vector<int32_t>& blob,
                    const std::vector<int64_t>& key, hipStream_t st,
                    int32_t** dev) {
    Buf& b = buf[kind];
    const size_t bytes = blob.size() * sizeof(int32_t);
    if (b.valid && b.key == key) {
      *dev = static_cast<int32_t*>(b.ptr);
      return hipSuccess;
    }
    b.valid = false;
    hipError_t e;
    if (bytes > b.cap) {
      // the old buffer may still be read by enqueued kernels
      if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
      if (b.ptr) (void)hipFree(b.ptr);
      b.ptr = nullptr;
      b.cap = 0;
      size_t cap = bytes < 65536 ? 65536 : bytes + bytes / 2;
      if ((e = hipMalloc(&b.ptr, cap)) != hipSuccess) return e;
      b.cap = cap;
    }
    Slot& s = slot[next];
    next = (next + 1) % kStageSlots;
    if (s.pending) {
      if ((e = hipEventSynchronize(s.ev)) != hipSuccess) return e;
      s.pending = false;
    }
    if (!s.ev && (e = hipEventCreateWithFlags(&s.ev, hipEventDisableTiming)) != hipSuccess)
      return e;
    if (bytes > s.cap) {
      if (s.host) (void)hipHostFree(s.host);
      s.host = nullptr;
      s.cap = 0;
      size_t cap = bytes < 65536 ? 65536 : bytes + bytes / 2;
      if ((e = hipHostMalloc(&s.host, cap, hipHostMallocDefault)) != hipSuccess) return e;
      s.cap = cap;
    }
    if (bytes) {
      std::memcpy(s.host, blob.data(), bytes);
      if ((e = hipMemcpyAsync(b.ptr, s.host, bytes, hipMemcpyHostToDevice, st)) != hipSuccess)
        return e;
      if ((e = hipEventRecord(s.ev, st)) != hipSuccess) return e;
      s.pending = true;
    }
    b.key = key;
    b.valid = true;
    *dev = static_cast<int32_t*>(b.ptr);
    return hipSuccess;
  }

  // Timing brackets around one launch.
  struct ProfScope {
    DeviceCtx* c;
    int k;
    hipStream_t st;
    hipEvent_t a = nullptr, b = nullptr;
    ProfScope(DeviceCtx* c_, int k_, hipStream_t st_) : c(c_), k(k_), st(st_) {
      if (!c->prof_on) return;
      if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) {
        a = b = nullptr;
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

int32_t dev_status(hipError_t e) { return e == hipSuccess ? PKV_OK : PKV_ERR_DEVICE; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// Shared by the contiguous-twin calls (no pool object to hang state on).
DeviceCtx& contig_ctx() {
  static DeviceCtx* c = new DeviceCtx();  // lives until process exit
  return *c;
}
std::mutex& contig_mutex() {
  static std::mutex m;
  return m;
}

// Work-list builders -------------------------------------------------------

// Blob layout: RowDesc[M] | Item[W] | OutDesc[Mo] | pages[]
struct Blob {
  std::vector<int32_t> v;
  size_t rows_off = 0, items_off = 0, outs_off = 0, pages_off = 0;
  int32_t n_items = 0, n_outs = 0;
  bool any_split = false;
};

// Decode/prefill work items for rows with the given total_k values.
// fast_decode: one item per 512-key split of each row (n_q == 1).
// otherwise: one item per (row, query), all keys (no split).
void build_items(Blob& bl, const std::vector<int32_t>& total_k, int32_t n_q,
                 bool fast_decode, std::vector<int32_t>& items,
                 std::vector<int32_t>& outs) {
  items.clear();
  outs.clear();
  bl.any_split = false;
  const int32_t M = static_cast<int32_t>(total_k.size());
  int32_t n_items = 0;
  for (int32_t r = 0; r < M; ++r) {
    for (int32_t i = 0; i < n_q; ++i) {
      const int32_t nsp = fast_decode ? ceil_div(total_k[r], pkv::kDecodeSplit) : 1;
      outs.push_back(n_items);
      outs.push_back(nsp);
      if (nsp > 1) bl.any_split = true;
      for (int32_t s = 0; s < nsp; ++s) {
        items.push_back(r);
        items.push_back(i);
        items.push_back(s);
        items.push_back(nsp);
        ++n_items;
      }
    }
  }
  bl.n_items = n_items;
  bl.n_outs = M * n_q;
}

void assemble(Blob& bl, const std::vector<int32_t>& rows,
              const std::vector<int32_t>& items, const std::vector<int32_t>& outs,
              const std::vector<int32_t>& pages) {
  bl.v.clear();
  bl.rows_off = 0;
  bl.v.insert(bl.v.end(), rows.begin(), rows.end());
  bl.items_off = bl.v.size();
  bl.v.insert(bl.v.end(), items.begin(), items.end());
  bl.outs_off = bl.v.size();
  bl.v.insert(bl.v.end(), outs.begin(), outs.end());
  bl.pages_off = bl.v.size();
  bl.v.insert(bl.v.end(), pages.begin(), pages.end());
  if (bl.v.empty()) bl.v.push_back(0);
}

size_t workspace_bytes_for(const Blob& bl, int32_t n_heads, int32_t head_dim) {
  if (!bl.any_split) return 0;
  return static_cast<size_t>(bl.n_items) * n_heads * (head_dim + 2) * sizeof(float);
}

}  // namespace

// ---------------------------------------------------------------------------

struct pkv_pool {
  pkv::PoolMeta meta;
  float* storage = nullptr;
  size_t storage_bytes = 0;
  int64_t block_floats = 0;
  DeviceCtx dev;
  // scratch reused across calls
  std::vector<int32_t> rows, items, outs, pages, tk;
  Blob blob;

  pkv_pool(int32_t nb, int32_t bs, int32_t nl, int32_t g, int32_t d, int32_t ms)
      : meta(nb, bs, nl, g, d, ms) {}
};


namespace {

PagedMap make_paged_map(const pkv_pool* p, int32_t layer, const int32_t* pages_dev) {
  const auto& m = p->meta;
  const int64_t G = m.n_kv_heads(), B = m.block_size(), D = m.head_dim();
  PagedMap pm;
  pm.base = p->storage;
  pm.pages = pages_dev;
  pm.block_stride = p->block_floats;
  pm.layer_off = static_cast<int64_t>(layer) * 2 * G * B * D;
  pm.head_stride = B * D;
  pm.v_off = G * B * D;
  pm.block_size = m.block_size();
  return pm;
}

bool contig_valid(const pkv_contig* c) {
  return c && c->base_dev && c->n_slots > 0 && c->n_layers > 0 &&
         c->n_kv_heads > 0 && c->max_seq > 0 && c->head_dim > 0 &&
         c->block_size > 0;
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

// Common attention launch (decode: n_q == 1 and decode == true).
template <class Map>
int32_t run_attention(DeviceCtx& dev, const Map& map, const Blob& bl,
                      const int32_t* blob_dev, const float* Q, float* out,
                      void* ws, int32_t n_heads, int32_t n_kv_heads,
                      int32_t head_dim, int32_t n_q, int32_t causal,
                      float scale, int32_t M, int32_t block_size, bool decode,
                      hipStream_t st) {
  const int32_t group = n_heads / n_kv_heads;
  AttnArgs a;
  a.rows = reinterpret_cast<const RowDesc*>(blob_dev + bl.rows_off);
  a.items = reinterpret_cast<const Item*>(blob_dev + bl.items_off);
  a.outs = reinterpret_cast<const OutDesc*>(blob_dev + bl.outs_off);
  a.Q = Q;
  a.out = out;
  a.part_o = static_cast<float*>(ws);
  a.part_ml = ws ? static_cast<float*>(ws) +
                       static_cast<size_t>(bl.n_items) * n_heads * head_dim
                 : nullptr;
  a.n_heads = n_heads;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.n_q = n_q;
  a.causal = causal;
  a.qscale = static_cast<float>(static_cast<double>(scale) * kLog2e);
  a.n_items = bl.n_items;
  a.n_outs = bl.n_outs;
  a.split = kNoSplit;
  hipError_t e;
  if (decode && pkv::fast_decode_ok(head_dim, group, block_size)) {
    {
      DeviceCtx::ProfScope ps(&dev, PKV_K_DECODE, st);
      e = pkv::launch_decode_fast(map, a, group, st);
    }
    if (e != hipSuccess) return PKV_ERR_DEVICE;
    if (bl.any_split) {
      DeviceCtx::ProfScope ps(&dev, PKV_K_COMBINE, st);
      e = pkv::launch_combine(a, st);
      if (e != hipSuccess) return PKV_ERR_DEVICE;
    }
    return PKV_OK;
  }
  if (!decode && pkv::fast_prefill_ok(head_dim, group, block_size)) {
    DeviceCtx::ProfScope ps(&dev, PKV_K_PREFILL, st);
    e = pkv::launch_prefill_mfma(map, a, M, st);
    return dev_status(e);
  }
  if (group > 16) return PKV_ERR_UNSUPPORTED;
  if (static_cast<int64_t>(group) * head_dim * 2 + group * 64 > 16384)
    return PKV_ERR_UNSUPPORTED;  // generic kernel keeps q and o in LDS
  DeviceCtx::ProfScope ps(&dev, decode ? PKV_K_DECODE : PKV_K_PREFILL, st);
  e = pkv::launch_generic(map, a, group, st);
  return dev_status(e);
}

// Common front checks of the attention calls, in the pages' order.
int32_t attn_front_checks(int32_t M, int32_t n_q, int32_t n_heads,
                          int32_t n_kv_heads, int32_t head_dim) {
  if (M <= 0 || n_q <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0)
    return PKV_ERR_BAD_DIM;
  if (n_heads % n_kv_heads != 0) return PKV_ERR_BAD_GQA;
  return PKV_OK;
}

// Build the attention blob for pool rows (total_k = seq_len + n_q).
void pool_attn_blob(pkv_pool* p, const int32_t* seqs, int32_t M, int32_t n_q,
                    bool fast_decode) {
  const int32_t B = p->meta.block_size();
  p->rows.clear();
  p->pages.clear();
  p->tk.clear();
  for (int32_t r = 0; r < M; ++r) {
    const pkv::SeqMeta* q = p->meta.seq(seqs[r]);
    const int32_t total_k = q->seq_len + n_q;
    const int32_t np = ceil_div(total_k, B);
    p->rows.push_back(total_k);
    p->rows.push_back(static_cast<int32_t>(p->pages.size()));
    p->rows.push_back(np);
    p->rows.push_back(0);
    p->pages.insert(p->pages.end(), q->pages.begin(), q->pages.begin() + np);
    p->tk.push_back(total_k);
  }
  build_items(p->blob, p->tk, n_q, fast_decode, p->items, p->outs);
  assemble(p->blob, p->rows, p->items, p->outs, p->pages);
}

std::vector<int64_t> blob_key(uint64_t version, int32_t kind_arg, int32_t n,
                              const int32_t* seqs, int32_t M) {
  std::vector<int64_t> k;
  k.reserve(M + 3);
  k.push_back(static_cast<int64_t>(version));
  k.push_back(kind_arg);
  k.push_back(n);
  for (int32_t r = 0; r < M; ++r) k.push_back(seqs[r]);
  return k;
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
  if (storage_dev) {
    if (storage_bytes < need) return nullptr;
    if (reinterpret_cast<uintptr_t>(storage_dev) % 16 != 0) return nullptr;
  }
  pkv_pool* p = new (std::nothrow) pkv_pool(n_blocks, block_size, n_layers,
                                            n_kv_heads, head_dim, max_seqs);
  if (!p) return nullptr;
  p->storage = static_cast<float*>(storage_dev);
  p->storage_bytes = storage_bytes;
  p->block_floats = static_cast<int64_t>(n_layers) * 2 * n_kv_heads *
                    block_size * head_dim;
  return p;
}

void pkv_pool_free(pkv_pool* pool) { delete pool; }

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
  if (rc != PKV_OK || cows.empty() || !pool->storage) return rc;
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
  std::vector<int64_t> nokey{-1};  // never matches a later COW upload
  pool->dev.buf[kCow].valid = false;
  if (pool->dev.upload(kCow, pairs, nokey, st, &dev) != hipSuccess) return PKV_ERR_DEVICE;
  pool->dev.buf[kCow].valid = false;
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
  if (!pool->storage) return PKV_OK;  // metadata-only pool: checks only
  if (!K_new_dev || !V_new_dev) return PKV_ERR_BAD_ARG;
  const hipStream_t st = as_stream(stream);
  if (pool->dev.use_stream(st) != hipSuccess) return PKV_ERR_DEVICE;

  // rows: start position and the pages the new rows land in
  const int32_t B = pool->meta.block_size();
  pool->rows.clear();
  pool->pages.clear();
  for (int32_t r = 0; r < M; ++r) {
    const pkv::SeqMeta* q = pool->meta.seq(seqs[r]);
    const int32_t np = ceil_div(static_cast<int64_t>(q->seq_len) + n_new, B);
    pool->rows.push_back(q->seq_len);
    pool->rows.push_back(static_cast<int32_t>(pool->pages.size()));
    pool->rows.push_back(np);
    pool->rows.push_back(0);
    pool->pages.insert(pool->pages.end(), q->pages.begin(), q->pages.begin() + np);
  }
  pool->items.clear();
  pool->outs.clear();
  assemble(pool->blob, pool->rows, pool->items, pool->outs, pool->pages);
  int32_t* dev = nullptr;
  if (pool->dev.upload(kAppend, pool->blob.v,
                       blob_key(pool->meta.version(), 0, n_new, seqs, M), st,
                       &dev) != hipSuccess)
    return PKV_ERR_DEVICE;
  const PagedMap pm = make_paged_map(pool, layer, dev + pool->blob.pages_off);
  DeviceCtx::ProfScope ps(&pool->dev, PKV_K_APPEND, st);
  return dev_status(pkv::launch_append(
      pm, reinterpret_cast<const RowDesc*>(dev + pool->blob.rows_off), K_new_dev,
      V_new_dev, M, n_new, pool->meta.n_kv_heads() * pool->meta.head_dim(),
      pool->meta.head_dim(), st));
}

int32_t pkv_advance(pkv_pool* pool, const int32_t* seqs, int32_t M, int32_t n) {
  if (!pool) return PKV_ERR_BAD_ARG;
  return pool->meta.advance(seqs, M, n);
}

size_t pkv_decode_workspace_bytes(pkv_pool* pool, const int32_t* seqs,
                                  int32_t M, int32_t n_heads) {
  if (!pool || M <= 0 || n_heads <= 0) return static_cast<size_t>(-1);
  const auto& m = pool->meta;
  if (n_heads % m.n_kv_heads() != 0) return static_cast<size_t>(-1);
  if (m.check_batch(seqs, M) != PKV_OK) return static_cast<size_t>(-1);
  const bool fast = pkv::fast_decode_ok(m.head_dim(), n_heads / m.n_kv_heads(),
                                        m.block_size());
  if (!fast) return 0;
  int64_t items = 0;
  bool split = false;
  for (int32_t r = 0; r < M; ++r) {
    const int32_t nsp = ceil_div(m.seq(seqs[r])->seq_len + 1, pkv::kDecodeSplit);
    items += nsp;
    split = split || nsp > 1;
  }
  if (!split) return 0;
  return static_cast<size_t>(items) * n_heads * (m.head_dim() + 2) * sizeof(float);
}

int32_t pkv_attn_paged_decode(pkv_pool* pool, const int32_t* seqs, int32_t M,
                              int32_t layer, int32_t n_heads,
                              int32_t n_kv_heads, int32_t head_dim,
                              const float* Q_dev, float scale, float* out_dev,
                              void* ws_dev, size_t ws_bytes, void* stream) {
  if (!pool) return PKV_ERR_BAD_ARG;
  if (int32_t rc = attn_front_checks(M, 1, n_heads, n_kv_heads, head_dim)) return rc;
  const auto& m = pool->meta;
  if (n_kv_heads != m.n_kv_heads() || head_dim != m.head_dim()) return PKV_ERR_BAD_DIM;
  if (int32_t rc = m.check_batch(seqs, M)) return rc;
  if (layer < 0 || layer >= m.n_layers()) return PKV_ERR_BAD_ARG;
  if (!pool->storage) return PKV_ERR_BAD_ARG;
  if (int32_t rc = m.check_rows(seqs, M, 1)) return rc;
  if (!Q_dev || !out_dev) return PKV_ERR_BAD_ARG;
  const int32_t group = n_heads / n_kv_heads;
  const bool fast = pkv::fast_decode_ok(head_dim, group, m.block_size());
  pool_attn_blob(pool, seqs, M, 1, fast);
  const size_t need = workspace_bytes_for(pool->blob, n_heads, head_dim);
  if (need > 0 && (!ws_dev || ws_bytes < need)) return PKV_ERR_BAD_ARG;
  const hipStream_t st = as_stream(stream);
  if (pool->dev.use_stream(st) != hipSuccess) return PKV_ERR_DEVICE;
  int32_t* dev = nullptr;
  if (pool->dev.upload(kDecode, pool->blob.v,
                       blob_key(m.version(), 1, n_heads, seqs, M), st,
                       &dev) != hipSuccess)
    return PKV_ERR_DEVICE;
  const PagedMap pm = make_paged_map(pool, layer, dev + pool->blob.pages_off);
  return run_attention(pool->dev, pm, pool->blob, dev, Q_dev, out_dev, ws_dev,
                       n_heads, n_kv_heads, head_dim, 1, 1, scale, M,
                       m.block_size(), true, st);
}

int32_t pkv_attn_paged_prefill(pkv_pool* pool, const int32_t* seqs, int32_t M,
                               int32_t n_q, int32_t layer, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim,
                               const float* Q_dev, int32_t causal, float scale,
                               float* out_dev, void* stream) {
  if (!pool) return PKV_ERR_BAD_ARG;
  if (int32_t rc = attn_front_checks(M, n_q, n_heads, n_kv_heads, head_dim)) return rc;
  const auto& m = pool->meta;
  if (n_kv_heads != m.n_kv_heads() || head_dim != m.head_dim()) return PKV_ERR_BAD_DIM;
  if (int32_t rc = m.check_batch(seqs, M)) return rc;
  if (layer < 0 || layer >= m.n_layers()) return PKV_ERR_BAD_ARG;
  if (!pool->storage) return PKV_ERR_BAD_ARG;
  if (int32_t rc = m.check_rows(seqs, M, n_q)) return rc;
  if (!Q_dev || !out_dev) return PKV_ERR_BAD_ARG;
  pool_attn_blob(pool, seqs, M, n_q, false);
  const hipStream_t st = as_stream(stream);
  if (pool->dev.use_stream(st) != hipSuccess) return PKV_ERR_DEVICE;
  int32_t* dev = nullptr;
  if (pool->dev.upload(kPrefill, pool->blob.v,
                       blob_key(m.version(), 2, n_q, seqs, M), st,
                       &dev) != hipSuccess)
    return PKV_ERR_DEVICE;
  const PagedMap pm = make_paged_map(pool, layer, dev + pool->blob.pages_off);
  return run_attention(pool->dev, pm, pool->blob, dev, Q_dev, out_dev, nullptr,
                       n_heads, n_kv_heads, head_dim, n_q, causal ? 1 : 0,
                       scale, M, m.block_size(), false, st);
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

// Rows for contiguous calls: pt_off holds the slot.
int32_t contig_rows(const pkv_contig* c, const int32_t* slots,
                    const int32_t* seq_lens, int32_t M, int32_t n,
                    std::vector<int32_t>& rows, std::vector<int32_t>* tk,
                    bool total) {
  if (!slots || !seq_lens) return PKV_ERR_BAD_ARG;
  rows.clear();
  if (tk) tk->clear();
  for (int32_t r = 0; r < M; ++r) {
    if (slots[r] < 0 || slots[r] >= c->n_slots) return PKV_ERR_SEQ;
    for (int32_t r2 = 0; r2 < r; ++r2)
      if (slots[r2] == slots[r]) return PKV_ERR_SEQ;
    if (seq_lens[r] < 0) return PKV_ERR_BAD_ARG;
    if (static_cast<int64_t>(seq_lens[r]) + n > c->max_seq) return PKV_ERR_SEQ;
    const int32_t tkr = seq_lens[r] + n;
    rows.push_back(total ? tkr : seq_lens[r]);
    rows.push_back(slots[r]);
    rows.push_back(ceil_div(tkr, c->block_size));
    rows.push_back(0);
    if (tk) tk->push_back(tkr);
  }
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
  std::vector<int32_t> rows, none;
  if (int32_t rc = contig_rows(cache, slots, seq_lens, M, n_new, rows, nullptr, false))
    return rc;
  Blob bl;
  assemble(bl, rows, none, none, none);
  DeviceCtx& dev = contig_ctx();
  const hipStream_t st = as_stream(stream);
  if (dev.use_stream(st) != hipSuccess) return PKV_ERR_DEVICE;
  int32_t* d = nullptr;
  dev.buf[kAppend].valid = false;
  if (dev.upload(kAppend, bl.v, {-1}, st, &d) != hipSuccess) return PKV_ERR_DEVICE;
  dev.buf[kAppend].valid = false;
  const ContigMap cm = make_contig_map(cache, layer);
  return dev_status(pkv::launch_append(cm, reinterpret_cast<const RowDesc*>(d),
                                       K_new_dev, V_new_dev, M, n_new,
                                       cache->n_kv_heads * cache->head_dim,
                                       cache->head_dim, st));
}

size_t pkv_contig_decode_workspace_bytes(const int32_t* seq_lens, int32_t M,
                                         int32_t n_heads, int32_t n_kv_heads,
                                         int32_t head_dim) {
  if (!seq_lens || M <= 0 || n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0 ||
      n_heads % n_kv_heads != 0)
    return static_cast<size_t>(-1);
  if (!pkv::fast_decode_ok(head_dim, n_heads / n_kv_heads, 16)) return 0;
  int64_t items = 0;
  bool split = false;
  for (int32_t r = 0; r < M; ++r) {
    const int32_t nsp = ceil_div(static_cast<int64_t>(seq_lens[r]) + 1, pkv::kDecodeSplit);
    items += nsp;
    split = split || nsp > 1;
  }
  if (!split) return 0;
  return static_cast<size_t>(items) * n_heads * (head_dim + 2) * sizeof(float);
}

namespace {

int32_t contig_attention(const pkv_contig* cache, const int32_t* slots,
                         const int32_t* seq_lens, int32_t M, int32_t n_q,
                         int32_t layer, int32_t n_heads, int32_t n_kv_heads,
                         int32_t head_dim, const float* Q_dev, int32_t causal,
                         float scale, float* out_dev, void* ws_dev,
                         size_t ws_bytes, bool decode, void* stream) {
  if (int32_t rc = attn_front_checks(M, n_q, n_heads, n_kv_heads, head_dim)) return rc;
  if (!contig_valid(cache)) return PKV_ERR_BAD_ARG;
  if (n_kv_heads != cache->n_kv_heads || head_dim != cache->head_dim) return PKV_ERR_BAD_DIM;
  if (layer < 0 || layer >= cache->n_layers) return PKV_ERR_BAD_ARG;
  if (!Q_dev || !out_dev) return PKV_ERR_BAD_ARG;
  std::lock_guard<std::mutex> g(contig_mutex());
  std::vector<int32_t> rows, items, outs, none, tk;
  if (int32_t rc = contig_rows(cache, slots, seq_lens, M, n_q, rows, &tk, true)) return rc;
  const int32_t group = n_heads / n_kv_heads;
  const bool fast = decode && pkv::fast_decode_ok(head_dim, group, cache->block_size);
  Blob bl;
  build_items(bl, tk, n_q, fast, items, outs);
  assemble(bl, rows, items, outs, none);
  const size_t need = workspace_bytes_for(bl, n_heads, head_dim);
  if (need > 0 && (!ws_dev || ws_bytes < need)) return PKV_ERR_BAD_ARG;
  DeviceCtx& dev = contig_ctx();
  const hipStream_t st = as_stream(stream);
  if (dev.use_stream(st) != hipSuccess) return PKV_ERR_DEVICE;
  const int kind = decode ? kDecode : kPrefill;
  int32_t* d = nullptr;
  dev.buf[kind].valid = false;
  if (dev.upload(kind, bl.v, {-1}, st, &d) != hipSuccess) return PKV_ERR_DEVICE;
  dev.buf[kind].valid = false;
  const ContigMap cm = make_contig_map(cache, layer);
  return run_attention(dev, cm, bl, d, Q_dev, out_dev, ws_dev, n_heads,
                       n_kv_heads, head_dim, n_q, causal, scale, M,
                       cache->block_size, decode, st);
}

}  // namespace

int32_t pkv_attn_contig_decode(const pkv_contig* cache, const int32_t* slots,
                               const int32_t* seq_lens, int32_t M,
                               int32_t layer, int32_t n_heads,
                               int32_t n_kv_heads, int32_t head_dim,
                               const float* Q_dev, float scale, float* out_dev,
                               void* ws_dev, size_t ws_bytes, void* stream) {
  return contig_attention(cache, slots, seq_lens, M, 1, layer, n_heads,
                          n_kv_heads, head_dim, Q_dev, 1, scale, out_dev,
                          ws_dev, ws_bytes, true, stream);
}

int32_t pkv_attn_contig_prefill(const pkv_contig* cache, const int32_t* slots,
                                const int32_t* seq_lens, int32_t M,
                                int32_t n_q, int32_t layer, int32_t n_heads,
                                int32_t n_kv_heads, int32_t head_dim,
                                const float* Q_dev, int32_t causal,
                                float scale, float* out_dev, void* stream) {
  return contig_attention(cache, slots, seq_lens, M, n_q, layer, n_heads,
                          n_kv_heads, head_dim, Q_dev, causal ? 1 : 0, scale,
                          out_dev, nullptr, 0, false, stream);
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

}  // extern "C"

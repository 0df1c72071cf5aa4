// Host-side metadata of the paged KV pool (see pool_meta.hpp for the rules).
#include "pool_meta.hpp"

#include <algorithm>
#include <climits>
#include <unordered_map>

namespace pkv {

static inline int32_t pages_for(int64_t rows, int32_t block_size) {
  return static_cast<int32_t>((rows + block_size - 1) / block_size);
}

PoolMeta::PoolMeta(int32_t n_blocks, int32_t block_size, int32_t n_layers,
                   int32_t n_kv_heads, int32_t head_dim, int32_t max_seqs)
    : n_blocks_(n_blocks),
      block_size_(block_size),
      n_layers_(n_layers),
      n_kv_heads_(n_kv_heads),
      head_dim_(head_dim),
      max_seqs_(max_seqs),
      refcnt_(n_blocks, 0),
      held_(n_blocks, 0),
      free_(n_blocks),
      seqs_(max_seqs),
      stamp_(max_seqs, 0) {
  // back() is popped first, so store ids descending: pops give 0, 1, 2, ...
  for (int32_t i = 0; i < n_blocks; ++i) free_[i] = n_blocks - 1 - i;
}

int32_t PoolMeta::pop() {
  int32_t id = free_.back();
  free_.pop_back();
  refcnt_[id] = 1;
  return id;
}

void PoolMeta::drop_ref(int32_t b) {
  // never below the page-table holders: unref_block refuses their references
  if (--refcnt_[b] == 0) free_.push_back(b);
}

// Every page-table write goes through here so the device mirror and the
// holder counts can follow.
void PoolMeta::set_page(int32_t s, SeqMeta& q, int32_t p, int32_t block) {
  if (p == static_cast<int32_t>(q.pages.size())) {
    q.pages.push_back(block);
  } else {
    --held_[q.pages[p]];
    q.pages[p] = block;
  }
  ++held_[block];
  if (track_) patches_.push_back({s, p, block});
}

int64_t PoolMeta::alloc_block() {
  if (free_.empty()) return -1;
  ++version_;
  return pop();
}

int32_t PoolMeta::unref_block(int64_t id) {
  if (id < 0 || id >= n_blocks_) return kBadArg;
  // only references taken by alloc_block: the page-table entries naming the
  // block are released by truncate and free
  if (refcnt_[id] - held_[id] <= 0) return kBadArg;
  ++version_;
  drop_ref(static_cast<int32_t>(id));
  return kOk;
}

int32_t PoolMeta::set_free_order(const int64_t* ids, int32_t n) {
  if (n != static_cast<int32_t>(free_.size())) return kBadArg;
  if (n > 0 && ids == nullptr) return kBadArg;
  std::vector<char> seen(n_blocks_, 0);
  for (int32_t i = 0; i < n; ++i) {
    const int64_t b = ids[i];
    if (b < 0 || b >= n_blocks_ || refcnt_[b] != 0 || seen[b]) return kBadArg;
    seen[b] = 1;
  }
  for (int32_t i = 0; i < n; ++i) free_[n - 1 - i] = static_cast<int32_t>(ids[i]);
  ++version_;
  return kOk;
}

SeqMeta* PoolMeta::live(int32_t s) {
  if (s < 0 || s >= max_seqs_ || !seqs_[s].alive) return nullptr;
  return &seqs_[s];
}

const SeqMeta* PoolMeta::seq(int32_t s) const {
  if (s < 0 || s >= max_seqs_ || !seqs_[s].alive) return nullptr;
  return &seqs_[s];
}

int32_t PoolMeta::lowest_free_id() const {
  for (int32_t s = 0; s < max_seqs_; ++s)
    if (!seqs_[s].alive) return s;
  return -1;
}

int32_t PoolMeta::seq_new(int32_t max_tokens) {
  if (max_tokens <= 0) return -kBadArg;
  const int32_t s = lowest_free_id();
  if (s < 0) return -kCapacity;
  // the device mirror addresses entry (seq, page) at seq * stride + page in
  // int32
  const int64_t pages = std::max(max_pages_seen_, pages_for(max_tokens, block_size_));
  if (static_cast<int64_t>(max_seqs_) * mirror_stride(pages) > INT32_MAX) return -kCapacity;
  SeqMeta& q = seqs_[s];
  q.alive = true;
  q.seq_len = 0;
  q.max_tokens = max_tokens;
  q.pages.clear();
  q.pages.reserve(pages_for(max_tokens, block_size_));
  max_pages_seen_ = std::max(max_pages_seen_, pages_for(max_tokens, block_size_));
  ++version_;
  return s;
}

void PoolMeta::release_from(SeqMeta& q, int32_t keep_pages) {
  while (static_cast<int32_t>(q.pages.size()) > keep_pages) {
    --held_[q.pages.back()];
    drop_ref(q.pages.back());
    q.pages.pop_back();
  }
}

int32_t PoolMeta::seq_free(int32_t s) {
  SeqMeta* q = live(s);
  if (!q) return kErrSeq;
  release_from(*q, 0);
  q->seq_len = 0;
  q->alive = false;
  ++version_;
  return kOk;
}

int32_t PoolMeta::seq_fork(int32_t s) {
  const SeqMeta* src = live(s);
  if (!src) return -kErrSeq;
  const int32_t c = lowest_free_id();
  if (c < 0) return -kCapacity;
  SeqMeta& dst = seqs_[c];
  dst.alive = true;
  dst.seq_len = src->seq_len;
  dst.max_tokens = src->max_tokens;
  const int32_t shared = pages_for(src->seq_len, block_size_);
  dst.pages.clear();
  for (int32_t p = 0; p < shared; ++p) {
    const int32_t b = src->pages[p];  // src stays valid: c != s
    set_page(c, dst, p, b);
    ++refcnt_[b];
  }
  ++version_;
  return c;
}

int32_t PoolMeta::seq_truncate(int32_t s, int32_t new_len) {
  SeqMeta* q = live(s);
  if (!q) return kErrSeq;
  if (new_len < 0 || new_len > q->seq_len) return kBadArg;
  release_from(*q, pages_for(new_len, block_size_));
  q->seq_len = new_len;
  ++version_;
  return kOk;
}

int32_t PoolMeta::check_batch(const int32_t* seqs, int32_t M) const {
  if (seqs == nullptr) return kErrSeq;
  if (++stamp_gen_ == 0) {  // wrapped: reset stamps
    std::fill(stamp_.begin(), stamp_.end(), 0);
    stamp_gen_ = 1;
  }
  for (int32_t r = 0; r < M; ++r) {
    const int32_t s = seqs[r];
    if (!seq(s)) return kErrSeq;
    if (stamp_[s] == stamp_gen_) return kErrSeq;  // repeated id
    stamp_[s] = stamp_gen_;
  }
  return kOk;
}

int32_t PoolMeta::ensure_append(const int32_t* seqs, int32_t M, int32_t n,
                                std::vector<CowCopy>* cows) {
  if (M <= 0 || n <= 0) return kBadDim;
  if (int32_t rc = check_batch(seqs, M)) return rc;
  for (int32_t r = 0; r < M; ++r) {
    const SeqMeta* q = seq(seqs[r]);
    if (static_cast<int64_t>(q->seq_len) + n > q->max_tokens) return kCapacity;
  }
  // Count the ids this takes, replaying the copy decisions with the
  // reference drops they cause (a later sequence may then own a block alone).
  std::unordered_map<int32_t, int32_t> dropped;
  int64_t need = 0;
  for (int32_t r = 0; r < M; ++r) {
    const SeqMeta* q = seq(seqs[r]);
    const int32_t first = q->seq_len / block_size_;
    const int32_t want = pages_for(static_cast<int64_t>(q->seq_len) + n, block_size_);
    const int32_t have = static_cast<int32_t>(q->pages.size());
    for (int32_t p = first; p < want && p < have; ++p) {
      const int32_t b = q->pages[p];
      auto it = dropped.find(b);
      const int32_t ref = refcnt_[b] - (it == dropped.end() ? 0 : it->second);
      if (ref > 1) {
        ++dropped[b];
        ++need;
      }
    }
    if (want > have) need += want - have;
  }
  if (need > static_cast<int64_t>(free_.size())) return kOom;

  for (int32_t r = 0; r < M; ++r) {
    SeqMeta& q = seqs_[seqs[r]];
    const int32_t first = q.seq_len / block_size_;
    const int32_t want = pages_for(static_cast<int64_t>(q.seq_len) + n, block_size_);
    const int32_t have = static_cast<int32_t>(q.pages.size());
    for (int32_t p = first; p < want && p < have; ++p) {
      const int32_t old = q.pages[p];
      if (refcnt_[old] > 1) {
        const int32_t fresh = pop();
        --refcnt_[old];  // stays >= 1: it was shared
        set_page(seqs[r], q, p, fresh);
        if (cows) cows->push_back({old, fresh});
      }
    }
    while (static_cast<int32_t>(q.pages.size()) < want)
      set_page(seqs[r], q, static_cast<int32_t>(q.pages.size()), pop());
  }
  ++version_;
  return kOk;
}

int32_t PoolMeta::check_append(const int32_t* seqs, int32_t M, int32_t n) const {
  for (int32_t r = 0; r < M; ++r) {
    const SeqMeta* q = seq(seqs[r]);
    const int64_t end = static_cast<int64_t>(q->seq_len) + n;
    if (end > static_cast<int64_t>(q->pages.size()) * block_size_) return kErrSeq;
    for (int32_t p = q->seq_len / block_size_; p < pages_for(end, block_size_); ++p)
      if (refcnt_[q->pages[p]] != 1) return kErrSeq;
  }
  return kOk;
}

int32_t PoolMeta::check_rows(const int32_t* seqs, int32_t M, int32_t n_q) const {
  for (int32_t r = 0; r < M; ++r) {
    const SeqMeta* q = seq(seqs[r]);
    const int64_t end = static_cast<int64_t>(q->seq_len) + n_q;
    if (end > static_cast<int64_t>(q->pages.size()) * block_size_) return kErrSeq;
  }
  return kOk;
}

int32_t PoolMeta::advance(const int32_t* seqs, int32_t M, int32_t n) {
  if (M <= 0 || n <= 0) return kBadDim;
  if (int32_t rc = check_batch(seqs, M)) return rc;
  for (int32_t r = 0; r < M; ++r) {
    const SeqMeta* q = seq(seqs[r]);
    const int64_t end = static_cast<int64_t>(q->seq_len) + n;
    if (end > q->max_tokens) return kCapacity;
    if (end > static_cast<int64_t>(q->pages.size()) * block_size_) return kErrSeq;
  }
  for (int32_t r = 0; r < M; ++r) seqs_[seqs[r]].seq_len += n;
  ++version_;
  return kOk;
}

}  // namespace pkv

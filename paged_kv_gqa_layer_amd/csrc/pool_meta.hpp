// Host-side metadata of the paged KV pool: reference counts, the free-id
// stack, per-sequence page tables and lengths.  Pure host code: no HIP calls,
// so it runs (and is tested) without a GPU.
//
// Behaviour follows "nx_paged_kv_gate.nx source" (KAT, FORK, REWIND parts:
// ids 0,1,2,-1 then recycle; fork shares blocks with reference count 2;
// copy-on-append makes divergent tails private; truncate releases
// references) and the caller contract of "nx_f32_attn_paged.nx source"
// (ensure once per step before the layers, advance once after them).
// Choices the pages leave open, used identically everywhere in this library:
//   - free ids form a LIFO stack; a fresh pool pops 0, 1, 2, ...;
//   - only shared blocks that the next append will write are copied, in
//     ensure_append, per sequence in batch order, ascending page order,
//     before that sequence's new pages are taken;
//   - ensure_append counts the ids it needs over the whole batch first and
//     changes nothing if too few are free;
//   - truncate and free release pages from the last page backwards;
//   - fork shares ceil(seq_len / block_size) pages;
//   - the lowest unused sequence id is handed out;
//   - unref_block releases only references taken by alloc_block: a block's
//     count minus the page-table entries that name it (those are released by
//     truncate and free);
//   - seq_new refuses a max_tokens whose page table, at the device mirror's
//     stride (pages rounded up to 64), would put a sequence's mirror offset
//     past the int32 range.
#pragma once

#include <algorithm>
#include <cstdint>
#include <utility>
#include <vector>

namespace pkv {

enum Status : int32_t {
  kOk = 0,
  kBadDim = 1,
  kBadGqa = 2,
  kErrSeq = 3,
  kOom = 4,
  kCapacity = 5,
  kBadArg = 6,
  kDevice = 7,
  kUnsupported = 8,
};

struct SeqMeta {
  bool alive = false;
  int32_t seq_len = 0;
  int32_t max_tokens = 0;
  std::vector<int32_t> pages;  // block id of page p
};

// A block that ensure_append copies before the append: src -> dst.
struct CowCopy {
  int32_t src;
  int32_t dst;
};

// One page-table entry that changed since the device mirror was last
// brought up to date: page `page` of sequence `seq` now names `block`.
struct PagePatch {
  int32_t seq;
  int32_t page;
  int32_t block;
};

class PoolMeta {
 public:
  PoolMeta(int32_t n_blocks, int32_t block_size, int32_t n_layers,
           int32_t n_kv_heads, int32_t head_dim, int32_t max_seqs);

  int32_t n_blocks() const { return n_blocks_; }
  int32_t block_size() const { return block_size_; }
  int32_t n_layers() const { return n_layers_; }
  int32_t n_kv_heads() const { return n_kv_heads_; }
  int32_t head_dim() const { return head_dim_; }
  int32_t max_seqs() const { return max_seqs_; }
  // Bumped by every call that changes any page table or length.
  uint64_t version() const { return version_; }

  int64_t alloc_block();
  int32_t unref_block(int64_t id);
  int32_t set_free_order(const int64_t* ids, int32_t n);

  int32_t seq_new(int32_t max_tokens);  // id or -status
  int32_t seq_free(int32_t s);
  int32_t seq_fork(int32_t s);          // id or -status
  int32_t seq_truncate(int32_t s, int32_t new_len);

  // Checks ids are live and pairwise distinct.
  int32_t check_batch(const int32_t* seqs, int32_t M) const;
  // On success appends the block copies to *cows (in the order taken).
  int32_t ensure_append(const int32_t* seqs, int32_t M, int32_t n,
                        std::vector<CowCopy>* cows);
  // Checks that n rows at seq_len.. exist and are private (no state change).
  int32_t check_append(const int32_t* seqs, int32_t M, int32_t n) const;
  // Checks that total_k = seq_len + n_q rows are covered by pages.
  int32_t check_rows(const int32_t* seqs, int32_t M, int32_t n_q) const;
  int32_t advance(const int32_t* seqs, int32_t M, int32_t n);

  const SeqMeta* seq(int32_t s) const;
  const std::vector<int32_t>& refcounts() const { return refcnt_; }
  const std::vector<int32_t>& free_stack() const { return free_; }

  // Page-table entries changed since the last take_patches(), in order.
  // Recording is off until enabled (metadata-only pools never enable it).
  void track_patches(bool on) { track_ = on; patches_.clear(); }
  std::vector<PagePatch>& patches() { return patches_; }
  // Largest page-table length any sequence created so far may reach.
  int32_t max_pages_seen() const { return max_pages_seen_; }
  // Page-table entries (over all live sequences) that name each block.
  const std::vector<int32_t>& holders() const { return held_; }
  // Entries per sequence of the device page-table mirror for a longest page
  // table of `pages` entries (a multiple of 64).
  static int64_t mirror_stride(int64_t pages) {
    return (std::max<int64_t>(pages, 1) + 63) / 64 * 64;
  }

 private:
  SeqMeta* live(int32_t s);
  int32_t lowest_free_id() const;
  void release_from(SeqMeta& q, int32_t keep_pages);
  int32_t pop();
  void drop_ref(int32_t b);
  void set_page(int32_t s, SeqMeta& q, int32_t p, int32_t block);

  int32_t n_blocks_, block_size_, n_layers_, n_kv_heads_, head_dim_, max_seqs_;
  std::vector<int32_t> refcnt_;
  std::vector<int32_t> held_;  // page-table entries naming each block
  std::vector<int32_t> free_;  // stack; back() is taken next
  std::vector<SeqMeta> seqs_;
  mutable std::vector<uint64_t> stamp_;  // duplicate detection in batches
  mutable uint64_t stamp_gen_ = 0;
  uint64_t version_ = 0;
  bool track_ = false;
  std::vector<PagePatch> patches_;
  int32_t max_pages_seen_ = 0;
};

}  // namespace pkv

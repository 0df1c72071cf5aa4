// Descriptors shared by the host launch code and the gfx950 kernels, plus the
// host-side launcher declarations.
//
// Device-resident state of a pool: the K/V storage (caller memory) and a
// mirror of every sequence's page table, int32 [max_seqs][stride], kept up
// to date by small patch lists.  Per call the kernels get one RowDesc per
// batch row (uploaded once per pool version and batch, so all layers of a
// step share it).
//
// Decode work items: each row's keys are cut into splits whose size follows
// from the row's own key count (split_keys).  The item list holds (row,
// split) pairs, longest first, so the end of the grid is filled with the
// shortest work.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv {

struct RowDesc {
  int32_t start;       // rows cached before this call (= seq_len)
  int32_t pt_off;      // paged: offset of the row's page table in the mirror;
                       // contiguous: the cache slot
  int32_t n_splits;    // decode: splits of the row's own keys, last may be partial
  int32_t part_base;   // decode: partial-result slot of own split 0
  int32_t k_off;       // first own key: keys below it form a prefix shared with
                       // other rows of the batch (shared-prefix decode), else 0
  int32_t n_pre;       // partial slots of the shared prefix, part_base - n_pre ..
  int32_t append_block;  // paged: block of page start / block_size (where a
                         // one-row append lands), -1 if not yet reserved
  int32_t split;       // decode: own keys per split (split_keys)
};
constexpr int kRowInts = sizeof(RowDesc) / sizeof(int32_t);

// Address of one page (block_size consecutive positions) of one kv head:
// K rows at the returned pointer, V rows at + v_off; position t of the page
// at + t * head_dim.
struct PagedMap {
  float* base;
  const int32_t* pages;  // the page-table mirror
  int64_t block_stride;  // floats per block (all layers)
  int64_t layer_off;     // floats from block start to this layer
  int64_t head_stride;   // floats between kv heads
  int64_t v_off;         // floats from the K part to the V part
  int32_t block_size;
  __device__ __forceinline__ float* block(int64_t b, int32_t kvh) const {
    return base + b * block_stride + layer_off + kvh * head_stride;
  }
  __device__ __forceinline__ float* page(const RowDesc& rd, int32_t p,
                                         int32_t kvh) const {
    return block(pages[rd.pt_off + p], kvh);
  }
};

struct ContigMap {
  float* base;
  int64_t slot_stride;  // floats per sequence slot (all layers)
  int64_t layer_off;
  int64_t head_stride;  // max_seq * head_dim
  int64_t v_off;        // n_kv_heads * max_seq * head_dim
  int64_t page_stride;  // block_size * head_dim
  int32_t block_size;
  __device__ __forceinline__ float* page(const RowDesc& rd, int32_t p,
                                         int32_t kvh) const {
    return base + rd.pt_off * slot_stride + layer_off + kvh * head_stride +
           p * page_stride;
  }
};

// Key split of the decode kernels for rows of 2048-6143 keys (splits are
// multiples of the 16-row page).
constexpr int32_t kDecodeSplit = 512;
// Own keys per split in a shared-prefix decode plan: a forked row's own keys
// follow its shared prefix, which the prefix workgroups cover beside them,
// so shorter splits keep the own-key waves from outlasting the prefix work.
constexpr int32_t kSharedOwnSplit = 128;
// Own keys per split of one row, from the row's own key count alone (so a
// row's result does not depend on the rest of the batch): 256 below 2048
// keys, 512 below 6144, 1024 below 8192, 2048 above -- longer rows take
// longer splits, which cuts the per-wave start-up, partial writes and merge
// reads, while short rows keep enough waves to fill the GPU in small
// batches.  A wave streams at a latency-bound rate, so in a small batch the
// longest split sets the kernel time: rows of 4-6K keys keep 512-key splits
// (1024 there made a 32-row batch of such rows 35% slower, and the 512 costs
// a large batch well under 1%).  Doubled for more than 4 queries per row
// (each key costs more work); the shared own-key split in a shared-prefix
// plan.
inline int32_t split_keys(int64_t own, int32_t n_q, bool shared = false) {
  if (shared) return kSharedOwnSplit;
  const int32_t s = own >= 8192   ? 4 * kDecodeSplit
                    : own >= 6144 ? 2 * kDecodeSplit
                    : own >= 2048 ? kDecodeSplit
                                  : kDecodeSplit / 2;
  return n_q <= 4 ? s : 2 * s;
}
// Queries per workgroup of the MFMA prefill kernel: 4 waves of 32 MFMA rows,
// each row one (query, head of the group).
constexpr int32_t prefill_q_tile(int32_t group) { return 128 / group; }

// Kernel shapes the specialised paths cover.
inline bool fast_decode_ok(int32_t head_dim, int32_t group, int32_t block) {
  return head_dim == 128 && block == 16 &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}
inline bool fast_prefill_ok(int32_t head_dim, int32_t group, int32_t block) {
  return head_dim == 128 && block == 16 &&
         (group == 1 || group == 2 || group == 4 || group == 8);
}
// Query rows (n_q x group) the split multi-query kernel holds per kv head.
constexpr int32_t kVerifyMaxRows = 32;
inline bool fast_verify_ok(int32_t head_dim, int32_t group, int32_t block,
                           int32_t n_q) {
  return head_dim == 128 && block == 16 && n_q >= 1 &&
         static_cast<int64_t>(n_q) * group <= kVerifyMaxRows;
}

struct AttnArgs {
  const RowDesc* rows;
  const int2* items;         // split work items: (row, split)
  const float* Q;
  float* out;
  float* part_o;      // [slots][n_q][n_heads][head_dim]   (split decode)
  float* part_ml;     // [slots][n_q][n_heads][2]
  int32_t n_rows;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t n_q;
  int32_t causal;
  float qscale;  // scale * log2(e): scores are kept in base-2 units
  int32_t n_items;
  // rotary table [positions][head_dim/2] of (cos, sin), or null: queries are
  // turned at their positions before the scores
  const double2* rope;
  // shared-prefix decode: prefix work items (group, split, row block) and the
  // groups they refer to
  const int32_t* pre_items;  // [n_pre_items][4]
  const int32_t* groups;     // [n_groups][4]: rep row, member offset, members, prefix keys
  const int32_t* members;    // batch rows of each group, consecutive
  int32_t n_pre_items;
};
// Keys per split of the shared-prefix kernel (four 32-key tiles).
constexpr int32_t kPrefixSplit = 128;
// Query rows per workgroup of the shared-prefix kernel (four waves of 32
// MFMA rows).
constexpr int32_t kPrefixRows = 128;

// Launchers (kernels.hip).  Each returns hipSuccess or the launch error.
hipError_t launch_patch(int32_t* mirror, const int32_t* patches, int32_t n,
                        int64_t stride, hipStream_t st);
// rope: rotary table (as AttnArgs::rope) or null; K rows are turned at
// their positions before they are stored.
hipError_t launch_append(const PagedMap& m, const RowDesc* rows,
                         const float* K, const float* V, int32_t M, int32_t n,
                         int32_t kv_dim, int32_t head_dim, const double2* rope,
                         hipStream_t st);
hipError_t launch_append(const ContigMap& m, const RowDesc* rows,
                         const float* K, const float* V, int32_t M, int32_t n,
                         int32_t kv_dim, int32_t head_dim, const double2* rope,
                         hipStream_t st);
// Page-table mirror patches (seq, page, block triples) applied by a launch,
// and the row blob it copies to the device on the way (n_copy ints from
// copy_src, device-readable pinned host memory, to copy_dst; n_copy = 0: no
// copy).
struct PatchArgs {
  int32_t* mirror;
  const int32_t* patches;
  int32_t n;
  int64_t stride;
  const int32_t* copy_src;
  int32_t* copy_dst;
  int32_t n_copy;
};
// One new row per sequence, written to each RowDesc's append_block, with the
// pending mirror patches applied and the row blob copied by the same launch
// (the append does not read the mirror; rows and patches may sit in the
// pinned host copy of the blob).
hipError_t launch_append_one(const PagedMap& m, const RowDesc* rows,
                             const float* K, const float* V, int32_t M,
                             int32_t kv_dim, int32_t head_dim,
                             const double2* rope, const PatchArgs& pa,
                             hipStream_t st);
// The same with the row blob (n_blob <= kIntChunk ints) passed in the kernel
// arguments: the launch reads the rows' descriptors and the patches (n_patch
// triples from int patch_off) from its argument copy, applies the patches
// and stores the blob to blob_dst.
hipError_t launch_append_inline(const PagedMap& m, const float* K, const float* V,
                                int32_t M, int32_t kv_dim, int32_t head_dim,
                                const double2* rope, int32_t* mirror, int64_t stride,
                                int32_t* blob_dst, const int32_t* blob, int32_t n_blob,
                                int32_t patch_off, int32_t n_patch, hipStream_t st);
hipError_t launch_cow(float* base, const int32_t* pairs, int32_t n_pairs,
                      int64_t block_floats, hipStream_t st);
// deep: two pages in flight per wave (one wave per SIMD for group 4 and 8)
// instead of one (two waves per SIMD); the same arithmetic, so the same bits.
// The deep form pays where waves stream long splits: a batch with 2048-key
// splits (rows of 8192 keys and more) -- M=64 rows of 1K-16K keys 0.48 vs
// 0.53 ms, M=256 1.657 vs 1.670 ms; without them the plain form is faster
// (M=32 / 64 / 128 rows of 512-4096 keys: 4-6%).
hipError_t launch_decode_fast(const PagedMap& m, const AttnArgs& a,
                              int32_t group, bool deep, hipStream_t st);
hipError_t launch_decode_fast(const ContigMap& m, const AttnArgs& a,
                              int32_t group, bool deep, hipStream_t st);
// Split multi-query decode (n_q x group <= kVerifyMaxRows), then launch_merge.
hipError_t launch_verify_mfma(const PagedMap& m, const AttnArgs& a,
                              int32_t group, hipStream_t st);
hipError_t launch_verify_mfma(const ContigMap& m, const AttnArgs& a,
                              int32_t group, hipStream_t st);
// Shared-prefix decode in one launch (group 1, 2, 4 or 8; decode_fast
// shapes): every group's prefix keys once per kv head for all its members'
// queries, into the members' prefix partial slots, and the rows' own-key
// splits into theirs.
hipError_t launch_shared_decode(const PagedMap& m, const AttnArgs& a,
                                int32_t group, hipStream_t st);
// Merges the key splits of every row with more than one (after decode_fast
// or verify_mfma).
hipError_t launch_merge(const AttnArgs& a, hipStream_t st);
hipError_t launch_generic(const PagedMap& m, const AttnArgs& a,
                          int32_t group, hipStream_t st);
hipError_t launch_generic(const ContigMap& m, const AttnArgs& a,
                          int32_t group, hipStream_t st);
hipError_t launch_prefill_mfma(const PagedMap& m, const AttnArgs& a,
                               int32_t group, hipStream_t st);
hipError_t launch_prefill_mfma(const ContigMap& m, const AttnArgs& a,
                               int32_t group, hipStream_t st);

// Zero-allocation decode: a file-scope device array (one copy per GPU, held
// until the process ends) with a row-blob region followed by a split-partial
// region.
constexpr size_t kNoAllocBlobBytes = size_t(1) << 20;
constexpr size_t kNoAllocPartBytes = size_t(64) << 20;
// Device address of the current GPU's scratch array (looked up once per
// device, with that device current; later calls return the kept address).
hipError_t noalloc_scratch(void** base);
// Writes n ints from host memory to device memory dst by passing them as
// kernel arguments (ceil(n / kIntChunk) launches, no staging buffer).
constexpr int32_t kIntChunk = 896;
hipError_t launch_write_ints(int32_t* dst, const int32_t* src, size_t n,
                             hipStream_t st);

}  // namespace pkv

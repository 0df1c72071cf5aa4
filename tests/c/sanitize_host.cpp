// Host-only driver for an AddressSanitizer + UndefinedBehaviorSanitizer build
// of the library's host code (pool metadata, argument checks, batch and split
// planning, shared-prefix grouping) and of the CPU oracle.
//
// Seeded random operation sequences run on a metadata-only library pool and
// an oracle pool side by side, with reference counts, free stacks, page
// tables and lengths compared after every operation (the same state the
// Python host tests compare, here under the sanitizers); workspace planning
// runs over random batches of large metadata-only pools with forks; the
// oracle's attention runs on small random inputs.  No device work is done:
// the device launchers are stubs that abort if reached.
//
// Built and run by tests/test_sanitize_host.py.  Exit 0 and a summary line
// on success; the first mismatch prints what differed and exits 1.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "device.hpp"
#include "pkv.h"

extern "C" {
typedef struct OPool OPool;
OPool* pkvo_pool_new(int, int, int, int, int, int, int);
void pkvo_pool_free(OPool*);
int64_t pkvo_alloc_block(OPool*);
int pkvo_unref_block(OPool*, int64_t);
int pkvo_set_free_order(OPool*, const int64_t*, int);
int pkvo_seq_new(OPool*, int);
int pkvo_seq_free(OPool*, int);
int pkvo_seq_fork(OPool*, int);
int pkvo_seq_truncate(OPool*, int, int);
int pkvo_ensure_append(OPool*, const int*, int, int);
int pkvo_append_layer(OPool*, const int*, int, int, int, const float*, const float*);
int pkvo_advance(OPool*, const int*, int, int);
int pkvo_attn_paged(OPool*, const int*, int, int, int, int, int, int, const float*, int,
                    float, float*);
int pkvo_attn_contig(const float*, const float*, const float*, int, int, int, int, int, int,
                     float, float*);
int pkvo_gqa_attention(const float*, const float*, const float*, int, int, int, int, float,
                       float*);
int pkvo_rope(float*, int, int, int, const int*, double);
int pkvo_seq_len(OPool*, int);
int pkvo_seq_pages(OPool*, int, int64_t*, int);
int pkvo_refcounts(OPool*, int32_t*);
int pkvo_free_stack(OPool*, int64_t*, int);
}

// Device launchers: never reached by metadata-only pools.
namespace pkv {
[[noreturn]] static void no_device(const char* f) {
  std::fprintf(stderr, "device launcher %s reached in the host-only build\n", f);
  std::abort();
}
hipError_t launch_patch(int32_t*, const int32_t*, int32_t, int64_t, hipStream_t) {
  no_device("launch_patch");
}
hipError_t launch_append(const PagedMap&, const RowDesc*, const float*, const float*,
                         int32_t, int32_t, int32_t, int32_t, const double2*, hipStream_t) {
  no_device("launch_append");
}
hipError_t launch_append(const ContigMap&, const RowDesc*, const float*, const float*,
                         int32_t, int32_t, int32_t, int32_t, const double2*, hipStream_t) {
  no_device("launch_append");
}
hipError_t launch_append_one(const PagedMap&, const RowDesc*, const float*, const float*,
                             int32_t, int32_t, int32_t, const double2*, const PatchArgs&,
                             hipStream_t) {
  no_device("launch_append_one");
}
hipError_t launch_append_inline(const PagedMap&, const float*, const float*, int32_t, int32_t,
                                int32_t, const double2*, int32_t*, int64_t, int32_t*,
                                const int32_t*, int32_t, int32_t, int32_t, hipStream_t) {
  no_device("launch_append_inline");
}
hipError_t launch_cow(float*, const int32_t*, int32_t, int64_t, hipStream_t) {
  no_device("launch_cow");
}
hipError_t launch_decode_fast(const PagedMap&, const AttnArgs&, int32_t, bool, hipStream_t) {
  no_device("launch_decode_fast");
}
hipError_t launch_decode_fast(const ContigMap&, const AttnArgs&, int32_t, bool, hipStream_t) {
  no_device("launch_decode_fast");
}
hipError_t launch_verify_mfma(const PagedMap&, const AttnArgs&, int32_t, hipStream_t) {
  no_device("launch_verify_mfma");
}
hipError_t launch_verify_mfma(const ContigMap&, const AttnArgs&, int32_t, hipStream_t) {
  no_device("launch_verify_mfma");
}
hipError_t launch_shared_decode(const PagedMap&, const AttnArgs&, int32_t, hipStream_t) {
  no_device("launch_shared_decode");
}
hipError_t launch_merge(const AttnArgs&, hipStream_t) { no_device("launch_merge"); }
hipError_t launch_generic(const PagedMap&, const AttnArgs&, int32_t, hipStream_t) {
  no_device("launch_generic");
}
hipError_t launch_generic(const ContigMap&, const AttnArgs&, int32_t, hipStream_t) {
  no_device("launch_generic");
}
hipError_t launch_prefill_mfma(const PagedMap&, const AttnArgs&, int32_t, hipStream_t) {
  no_device("launch_prefill_mfma");
}
hipError_t launch_prefill_mfma(const ContigMap&, const AttnArgs&, int32_t, hipStream_t) {
  no_device("launch_prefill_mfma");
}
hipError_t noalloc_scratch(void**) { no_device("noalloc_scratch"); }
hipError_t launch_write_ints(int32_t*, const int32_t*, size_t, hipStream_t) {
  no_device("launch_write_ints");
}
}  // namespace pkv

namespace {

using Rng = std::mt19937_64;

int fail(const char* what, long a, long b, int seed, int step) {
  std::printf("MISMATCH %s: library %ld, oracle %ld (seed %d, step %d)\n", what, a, b, seed,
              step);
  return 1;
}

// Reference counts, free stack, lengths and page tables of every sequence id.
int same_state(pkv_pool* p, OPool* o, int n_blocks, int max_seqs, int seed, int step) {
  std::vector<int32_t> r1(n_blocks), r2(n_blocks);
  pkv_pool_refcounts(p, r1.data());
  pkvo_refcounts(o, r2.data());
  for (int b = 0; b < n_blocks; ++b)
    if (r1[b] != r2[b]) return fail("refcount", r1[b], r2[b], seed, step);
  std::vector<int64_t> f1(n_blocks), f2(n_blocks);
  const int n1 = pkv_pool_free_stack(p, f1.data(), n_blocks);
  const int n2 = pkvo_free_stack(o, f2.data(), n_blocks);
  if (n1 != n2) return fail("free count", n1, n2, seed, step);
  for (int i = 0; i < n1; ++i)
    if (f1[i] != f2[i]) return fail("free stack", f1[i], f2[i], seed, step);
  std::vector<int64_t> p1(n_blocks + 1), p2(n_blocks + 1);
  for (int s = -1; s <= max_seqs; ++s) {
    const int l1 = pkv_seq_len(p, s), l2 = pkvo_seq_len(o, s);
    if (l1 != l2) return fail("seq_len", l1, l2, seed, step);
    const int c1 = pkv_seq_pages(p, s, p1.data(), n_blocks + 1);
    const int c2 = pkvo_seq_pages(o, s, p2.data(), n_blocks + 1);
    if (c1 != c2) return fail("page count", c1, c2, seed, step);
    for (int i = 0; i < c1 && i <= n_blocks; ++i)
      if (p1[i] != p2[i]) return fail("page", p1[i], p2[i], seed, step);
  }
  return 0;
}

// Random operations on both pools; returns the number of operations run.
long random_ops(int seed, int* bad) {
  Rng g(1000 + seed);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(g); };
  const int B = std::vector<int>{1, 2, 4, 16}[uni(0, 3)];
  const int n_blocks = uni(4, 96), n_layers = uni(1, 2), G = uni(1, 2), D = uni(1, 4) * 2;
  const int max_seqs = uni(2, 9);
  pkv_pool* p = pkv_pool_new(n_blocks, B, n_layers, G, D, max_seqs, nullptr, 0);
  OPool* o = pkvo_pool_new(n_blocks, B, n_layers, G, D, max_seqs, 1);
  std::vector<int64_t> perm(n_blocks);
  for (int i = 0; i < n_blocks; ++i) perm[i] = i;
  std::shuffle(perm.begin(), perm.end(), g);
  if (pkv_pool_set_free_order(p, perm.data(), n_blocks) !=
      pkvo_set_free_order(o, perm.data(), n_blocks))
    return *bad = fail("set_free_order", 0, 0, seed, -1), 0;
  std::vector<int64_t> raw;
  const int kv_dim = G * D;
  long ops = 0;
  for (int step = 0; step < 400; ++step, ++ops) {
    const int op = uni(0, 10);
    const int s = uni(-1, max_seqs);
    long a = 0, b = 0;
    const char* what = "";
    if (op == 0) {
      const int mt = uni(-1, 90);
      a = pkv_seq_new(p, mt), b = pkvo_seq_new(o, mt), what = "seq_new";
    } else if (op == 1) {
      a = pkv_seq_fork(p, s), b = pkvo_seq_fork(o, s), what = "seq_fork";
    } else if (op == 2) {
      const int nl = uni(-1, 50);
      a = pkv_seq_truncate(p, s, nl), b = pkvo_seq_truncate(o, s, nl), what = "truncate";
    } else if (op == 3) {
      a = pkv_seq_free(p, s), b = pkvo_seq_free(o, s), what = "seq_free";
    } else if (op == 4) {
      a = pkv_alloc_block(p), b = pkvo_alloc_block(o), what = "alloc";
      if (a >= 0) raw.push_back(a);
    } else if (op == 5) {
      int64_t id;
      if (!raw.empty() && uni(0, 9) < 6) {
        id = raw.back();
        raw.pop_back();
      } else {
        id = uni(-1, n_blocks);  // free, held by a page table, or out of range
        for (size_t i = 0; i < raw.size(); ++i)
          if (raw[i] == id) raw.erase(raw.begin() + i--);
      }
      a = pkv_unref_block(p, id), b = pkvo_unref_block(o, id), what = "unref";
    } else {
      const int M = uni(0, 4);
      std::vector<int32_t> batch(std::max(M, 1));
      for (int r = 0; r < M; ++r) batch[r] = uni(-1, max_seqs);
      const int n = uni(0, 9);
      a = pkv_ensure_append(p, batch.data(), M, n, nullptr);
      b = pkvo_ensure_append(o, batch.data(), M, n);
      what = "ensure_append";
      if (a == b && op >= 8) {
        const int layer = uni(-1, n_layers);
        std::vector<float> K(std::max(M * n, 1) * kv_dim), V(K.size());
        for (auto& x : K) x = static_cast<float>(uni(-8, 8));
        for (auto& x : V) x = static_cast<float>(uni(-8, 8));
        a = pkv_append_layer(p, batch.data(), M, n, layer, nullptr, nullptr, nullptr);
        b = pkvo_append_layer(o, batch.data(), M, n, layer, K.data(), V.data());
        what = "append_layer";
        if (a == b && a == 0) {
          // the oracle attends over what it holds; the library's
          // metadata-only pool refuses the attention calls
          const int H = G * uni(1, 3);
          std::vector<float> Q(M * n * H * D), out(Q.size());
          for (auto& x : Q) x = static_cast<float>(uni(-8, 8));
          if (pkvo_attn_paged(o, batch.data(), M, n, layer, H, G, D, Q.data(), uni(0, 1),
                              0.25f, out.data()) != 0)
            return *bad = fail("oracle attn_paged", 0, 1, seed, step), ops;
          if (pkv_attn_paged_prefill(p, batch.data(), M, n, layer, H, G, D, Q.data(), 1,
                                     0.25f, out.data(), nullptr) != PKV_ERR_BAD_ARG)
            return *bad = fail("metadata-only prefill", 0, 1, seed, step), ops;
          if (pkv_decode_workspace_bytes(p, batch.data(), M, H) == static_cast<size_t>(-1) ||
              pkv_verify_workspace_bytes(p, batch.data(), M, n, H) ==
                  static_cast<size_t>(-1) ||
              pkv_decode_shared_workspace_bytes(p, batch.data(), M, H) ==
                  static_cast<size_t>(-1))
            return *bad = fail("workspace sizes", 0, 1, seed, step), ops;
        }
      }
      if (a == b && uni(0, 1)) {
        const int nadv = uni(0, 9) < 8 ? n : uni(0, 9);
        a = pkv_advance(p, batch.data(), M, nadv);
        b = pkvo_advance(o, batch.data(), M, nadv);
        what = "advance";
      }
    }
    if (a != b) return *bad = fail(what, a, b, seed, step), ops;
    if (same_state(p, o, n_blocks, max_seqs, seed, step)) return *bad = 1, ops;
  }
  pkv_pool_free(p);
  pkvo_pool_free(o);
  return ops;
}

// Workspace planning (split plan, shared-prefix grouping) over large
// metadata-only pools: many sequences, long rows, forks sharing prefixes.
long planning(int seed, int* bad) {
  Rng g(5000 + seed);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(g); };
  const int max_seqs = 300, B = 16, G = 8, D = 128;
  const int n_blocks = 200000;
  pkv_pool* p = pkv_pool_new(n_blocks, B, 1, G, D, max_seqs, nullptr, 0);
  std::vector<int32_t> live;
  long plans = 0;
  for (int i = 0; i < 120; ++i) {
    const int s = pkv_seq_new(p, 70000);
    if (s < 0) break;
    const int len = uni(1, 20000);
    if (pkv_ensure_append(p, &s, 1, len, nullptr) != 0 || pkv_advance(p, &s, 1, len) != 0)
      return *bad = fail("fill", 0, 1, seed, i), plans;
    live.push_back(s);
    if (uni(0, 3) == 0) {  // a fork family sharing this prefix
      for (int f = uni(1, 6); f > 0; --f) {
        const int c = pkv_seq_fork(p, s);
        if (c < 0) break;
        const int own = uni(0, 300);
        if (own && (pkv_ensure_append(p, &c, 1, own, nullptr) != 0 ||
                    pkv_advance(p, &c, 1, own) != 0))
          return *bad = fail("fork fill", 0, 1, seed, i), plans;
        live.push_back(c);
      }
    }
  }
  for (int t = 0; t < 300; ++t, ++plans) {
    std::vector<int32_t> batch = live;
    std::shuffle(batch.begin(), batch.end(), g);
    batch.resize(uni(1, static_cast<int>(batch.size())));
    const int M = static_cast<int>(batch.size());
    const int H = G * std::vector<int>{1, 2, 4, 8}[uni(0, 3)];
    if (pkv_ensure_append(p, batch.data(), M, 1, nullptr) != 0)
      return *bad = fail("ensure", 0, 1, seed, t), plans;
    const size_t d = pkv_decode_workspace_bytes(p, batch.data(), M, H);
    const size_t sh = pkv_decode_shared_workspace_bytes(p, batch.data(), M, H);
    const size_t v = pkv_verify_workspace_bytes(p, batch.data(), M, uni(1, 8), H);
    if (d == static_cast<size_t>(-1) || sh == static_cast<size_t>(-1) ||
        v == static_cast<size_t>(-1))
      return *bad = fail("workspace", 0, 1, seed, t), plans;
    std::vector<int32_t> lens(M), slots(M);
    for (int r = 0; r < M; ++r) lens[r] = pkv_seq_len(p, batch[r]);
    if (pkv_contig_decode_workspace_bytes(lens.data(), M, H, G, D) != d)
      return *bad = fail("contig workspace", 0, 1, seed, t), plans;
    if (pkv_advance(p, batch.data(), M, 1) != 0)
      return *bad = fail("advance", 0, 1, seed, t), plans;
  }
  pkv_pool_free(p);
  return plans;
}

// The oracle's attention entry points on small random inputs.
long oracle_attention(int seed, int* bad) {
  Rng g(9000 + seed);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(g); };
  std::normal_distribution<float> nd(0.f, 1.f);
  long calls = 0;
  for (int t = 0; t < 60; ++t, ++calls) {
    const int G = uni(1, 3), H = G * uni(1, 4), D = uni(1, 16) * 2;
    const int total_k = uni(1, 70), n_q = uni(1, total_k);
    std::vector<float> Q(n_q * H * D), K(total_k * G * D), V(K.size()), out(Q.size());
    for (auto& x : Q) x = nd(g);
    for (auto& x : K) x = nd(g);
    for (auto& x : V) x = nd(g);
    if (pkvo_attn_contig(Q.data(), K.data(), V.data(), n_q, total_k, H, G, D, uni(0, 1),
                         0.3f, out.data()) != 0)
      return *bad = fail("attn_contig", 0, 1, seed, t), calls;
    if (pkvo_gqa_attention(Q.data(), K.data(), V.data(), n_q, H, G, D, 0.3f, out.data()) != 0)
      return *bad = fail("gqa_attention", 0, 1, seed, t), calls;
    std::vector<int> pos(n_q);
    for (auto& x : pos) x = uni(0, 5000);
    if (pkvo_rope(Q.data(), n_q, H, D, pos.data(), 9.21) != 0)
      return *bad = fail("rope", 0, 1, seed, t), calls;
  }
  return calls;
}

}  // namespace

int main(int argc, char** argv) {
  const int seeds = argc > 1 ? std::atoi(argv[1]) : 40;
  int bad = 0;
  long ops = 0, plans = 0, calls = 0;
  for (int s = 0; s < seeds && !bad; ++s) ops += random_ops(s, &bad);
  for (int s = 0; s < 3 && !bad; ++s) plans += planning(s, &bad);
  for (int s = 0; s < seeds && !bad; ++s) calls += oracle_attention(s, &bad);
  if (bad) return 1;
  std::printf("sanitize_host: %ld pool operations, %ld batch plans, %ld oracle attention "
              "calls, no mismatch\n",
              ops, plans, calls);
  return 0;
}

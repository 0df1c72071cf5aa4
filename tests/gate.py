"""The pages' paged-KV gate as a runnable program ("nx_paged_kv_gate.nx
source": main), on one of two backends:

  python tests/gate.py            the CPU oracle (oracle/)
  python tests/gate.py --gpu      the HIP library on the GPU (paged pool and
                                  its contiguous twin, both through the C ABI)

Four parts, each printing one OK line, then the four-flag summary line and a
final DONE line; exit status 0.  A failed check ends the program at once with
the status the pages give that check (11-13 pool known answers; 20+r, 30+r,
40+r the three rounds of paged == contiguous; 50+r, 61-63, 70+r, 80+r the
fork with copy-on-append; 90-93 the fresh contiguous replays; 94-96 the
truncate-and-reappend rewind), where r is 1 (ensure failed), 2 (contiguous
attention failed), 3 (paged attention failed) or 4 (outputs differ).

Inputs are the pages' own: the 31-bit LCG with seed 20260709 and its fill
order (synth.TinyGate), 2 layers, 4 query heads on 2 kv heads, head_dim 8,
scale 0.25.  The block size, hidden on the pages, is 4.  At that size the
fork-time page holding the last prefill row is page 1 (5 rows, 4 per page),
so the copy-on-append divergence check is made on that page; page 0 is full
and stays shared with two references.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

G = synth.TinyGate()


class Fail(Exception):
    def __init__(self, code):
        super().__init__(code)
        self.code = code


def _same_bits(a, b):
    a = np.ascontiguousarray(a, np.float32)
    b = np.ascontiguousarray(b, np.float32)
    return a.shape == b.shape and np.array_equal(a.view(np.uint32), b.view(np.uint32))


class OracleBackend:
    """Pool, sequences and attention of the CPU oracle."""

    def __init__(self):
        import oracle
        self.o = oracle

    def pool(self, n_blocks):
        return self.o.Pool(n_blocks, G.block_size, G.n_layers, G.n_kv_heads, G.head_dim,
                           max_seqs=8)

    def cache(self):
        return self.o.Cache(G.n_layers, G.n_kv_heads, G.max_tokens, G.head_dim)

    def new_seq(self, pool):
        return pool.seq_new(G.max_tokens)

    def ensure(self, pool, seq, n):
        return pool.ensure_append([seq], n)

    def advance(self, pool, seq, n):
        return pool.advance([seq], n)

    def attn_paged(self, pool, seq, layer, Q, K, V, n):
        return pool.attn_with_paged(Q, K, V, n, G.n_heads, G.n_kv_heads, G.head_dim, seq,
                                    layer, True, G.scale)

    def attn_contig(self, cache, layer, Q, K, V, n):
        return cache.attn_with_cache(Q, K, V, n, G.n_heads, G.n_kv_heads, G.head_dim,
                                     layer, True, G.scale)

    def advance_cache(self, cache, n):
        cache.advance(n)


class GpuBackend:
    """The HIP library: the paged pool, and the same kernels over a
    contiguous cache (one slot per cache) for the contiguous side."""

    def __init__(self):
        import torch
        import paged_kv_gqa_layer_amd as pkv
        self.torch = torch
        self.pkv = pkv
        if not torch.cuda.is_available():
            raise SystemExit("gate.py --gpu needs a GPU")

    def _dev(self, a):
        return self.torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()

    def pool(self, n_blocks):
        return self.pkv.Pool(n_blocks, G.block_size, G.n_layers, G.n_kv_heads, G.head_dim,
                             max_seqs=8)

    def cache(self):
        c = self.pkv.ContigCache(1, G.n_layers, G.n_kv_heads, G.max_tokens, G.head_dim,
                                 block_size=G.block_size)
        c.seq_len = 0
        return c

    def new_seq(self, pool):
        return pool.seq_new(G.max_tokens)

    def ensure(self, pool, seq, n):
        return pool.ensure_append([seq], n)

    def advance(self, pool, seq, n):
        return pool.advance([seq], n)

    def attn_paged(self, pool, seq, layer, Q, K, V, n):
        rc = pool.append_layer([seq], n, layer, self._dev(K), self._dev(V))
        if rc:
            return rc, None
        out = self.torch.full((n, G.q_dim), float("nan"), device="cuda")
        rc = pool.attn_paged_prefill([seq], n, layer, G.n_heads, G.n_kv_heads, G.head_dim,
                                     self._dev(Q), True, G.scale, out)
        self.torch.cuda.synchronize()
        return rc, out.cpu().numpy()

    def attn_contig(self, cache, layer, Q, K, V, n):
        rc = cache.append([0], [cache.seq_len], n, layer, self._dev(K), self._dev(V),
                          check=False)
        if rc:
            return rc, None
        out = self.torch.full((n, G.q_dim), float("nan"), device="cuda")
        rc = cache.attn_prefill([0], [cache.seq_len], n, layer, G.n_heads, self._dev(Q),
                                True, G.scale, out, check=False)
        self.torch.cuda.synchronize()
        return rc, out.cpu().numpy()

    def advance_cache(self, cache, n):
        cache.seq_len += n


def run(be):
    x = G.inputs()

    # ---- KAT: pool mechanics
    p0 = be.pool(3)
    b = [p0.alloc_block() for _ in range(3)]
    if b != [0, 1, 2]:
        raise Fail(11)
    if p0.alloc_block() != -1:
        raise Fail(12)                      # exhaustion fails fast
    p0.unref_block(b[1])
    if p0.alloc_block() != 1:
        raise Fail(13)                      # a released id is handed out again
    print("PKV KAT pool alloc/exhaust/recycle OK", flush=True)

    def round_both(cc, pool, seq, qkv, n):
        """One append round on both paths, compared bit for bit; 0 = ok."""
        Q, K, V = qkv
        if be.ensure(pool, seq, n) != 0:
            return 1
        for L in range(G.n_layers):
            rc, oc = be.attn_contig(cc, L, Q, K, V, n)
            if rc != 0:
                return 2
            rc, op = be.attn_paged(pool, seq, L, Q, K, V, n)
            if rc != 0:
                return 3
            if not _same_bits(oc, op):
                return 4
        be.advance_cache(cc, n)
        be.advance(pool, seq, n)
        return 0

    def round_paged(pool, seq, qkv, n):
        """Append round on a paged sequence only; (status, outputs per layer)."""
        Q, K, V = qkv
        if be.ensure(pool, seq, n) != 0:
            return 1, None
        outs = []
        for L in range(G.n_layers):
            rc, op = be.attn_paged(pool, seq, L, Q, K, V, n)
            if rc != 0:
                return 2, None
            outs.append(op)
        be.advance(pool, seq, n)
        return 0, outs

    def round_contig(cc, qkv, n):
        Q, K, V = qkv
        outs = []
        for L in range(G.n_layers):
            rc, oc = be.attn_contig(cc, L, Q, K, V, n)
            if rc != 0:
                return 2, None
            outs.append(oc)
        be.advance_cache(cc, n)
        return 0, outs

    # ---- EQUIV: three rounds, paged == contiguous
    cc = be.cache()
    pool = be.pool(G.n_blocks)
    s_a = be.new_seq(pool)
    for base, (key, n) in zip((20, 30, 40), (("1", 5), ("2", 1), ("3", 3))):
        r = round_both(cc, pool, s_a, x[key], n)
        if r:
            raise Fail(base + r)
    print("PKV EQUIV paged==contiguous BIT-EXACT (5+1+3 rows, 2 layers, GQA) OK", flush=True)

    # ---- FORK + copy-on-append divergence
    pool2 = be.pool(G.n_blocks)
    f_a = be.new_seq(pool2)
    cc_a = be.cache()
    r = round_both(cc_a, pool2, f_a, x["1"], 5)
    if r:
        raise Fail(50 + r)
    f_b = pool2.seq_fork(f_a)
    if f_b < 0 or pool2.refcounts()[pool2.seq_pages(f_a)[0]] != 2:
        raise Fail(61)                      # the shared prompt block
    r, op_a = round_paged(pool2, f_a, x["A"], 2)
    if r:
        raise Fail(70 + r)
    r, op_b = round_paged(pool2, f_b, x["B"], 2)
    if r:
        raise Fail(80 + r)
    tail = (5 - 1) // G.block_size          # the page the fork shared partly filled
    pa, pb = pool2.seq_pages(f_a), pool2.seq_pages(f_b)
    ref = pool2.refcounts()
    if pa[tail] == pb[tail]:
        raise Fail(62)                      # the forks must have diverged
    if ref[pa[tail]] != 1 or ref[pb[tail]] != 1 or ref[pa[0]] != 2 or pa[0] != pb[0]:
        raise Fail(63)

    # ground truth: fresh contiguous replays of both histories
    g_a, g_b = be.cache(), be.cache()
    if round_contig(g_a, x["1"], 5)[0] or round_contig(g_b, x["1"], 5)[0]:
        raise Fail(90)
    r1, oc_a = round_contig(g_a, x["A"], 2)
    r2, oc_b = round_contig(g_b, x["B"], 2)
    if r1 or r2:
        raise Fail(91)
    if not all(_same_bits(p, c) for p, c in zip(op_a, oc_a)):
        raise Fail(92)
    if not all(_same_bits(p, c) for p, c in zip(op_b, oc_b)):
        raise Fail(93)
    print("PKV FORK+COW both forks BIT-EXACT vs contiguous replays OK", flush=True)

    # ---- REWIND: truncate A to the fork point, re-append B's rows
    if pool2.seq_truncate(f_a, 5) != 0:
        raise Fail(94)
    r, op_r = round_paged(pool2, f_a, x["B"], 2)
    if r:
        raise Fail(95)
    if not all(_same_bits(p, c) for p, c in zip(op_r, oc_b)):
        raise Fail(96)
    print("PKV REWIND truncate-then-append BIT-EXACT (spec-decode contract) OK", flush=True)

    print("LIAR-KILL pool-mechanics=1 equiv-bitexact=1 fork-cow=1 rewind=1", flush=True)
    print("PAGED_KV_GATE DONE", flush=True)


def main(argv):
    be = GpuBackend() if "--gpu" in argv else OracleBackend()
    try:
        run(be)
    except Fail as f:
        print("PAGED_KV_GATE FAILED %d" % f.code, flush=True)
        return f.code
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1:]))

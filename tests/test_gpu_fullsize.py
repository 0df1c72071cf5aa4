"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: outputs against the oracle (one sequence / query per oracle
call, spread over the host cores), properties on every output, pool state
against the oracle's, and the fork / rewind invariants bit for bit.  Decode
(every row of the M=256 step), verify (4 and 8 drafted rows with rewind),
prefill (every 16th query and the tile edges of all 8 sequences) and the
forked workload (every fork at four steps)."""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_layer_amd as pkv
import synth
from bench import HistoryFiller
from pkv_gpu import assert_close, bits_equal, dev

pytestmark = pytest.mark.gpu


def _workers():
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, n))


def _parallel(fn, jobs):
    """fn over jobs on the host cores (the oracle runs outside the GIL)."""
    with ThreadPoolExecutor(max_workers=_workers()) as ex:
        return list(ex.map(fn, jobs))


def _pool_for(wl, n_layers=1, max_seqs=None):
    pool = pkv.Pool(wl.n_blocks, wl.block_size, n_layers, wl.n_kv_heads,
                    wl.head_dim, max_seqs=max_seqs or wl.M + 8)
    pool.set_free_order(wl.free_order())
    return pool


def test_decode_m256_full_size_every_row():
    """Every row of a decode step of the M=256 workload against the oracle."""
    wl = synth.decode_m256(max_steps=2)
    H, G, D, M = wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.M
    pool = _pool_for(wl)
    seqs = [pool.seq_new(wl.max_tokens) for _ in range(M)]
    f = HistoryFiller(wl, int(wl.ctx.max()))
    f.fill(pool, seqs, wl.ctx)
    f.close()
    q, k, v = wl.step(0)
    seqs_np = np.asarray(seqs, np.int32)
    pool.ensure_append(seqs_np, 1, check=True)
    pool.append_layer(seqs_np, 1, 0, dev(k), dev(v), check=True)
    ws = torch.empty(pool.decode_workspace_bytes(seqs_np, H), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((M, H * D), float("nan"), device="cuda")
    pool.attn_paged_decode(seqs_np, 0, H, G, D, dev(q), wl.scale, out, ws=ws,
                           check=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    # |out| is a convex combination of N(0,1) values: loose sanity bound
    assert np.abs(got).max() < 10

    def check(r):
        kh, vh = wl.history(r)
        rc, ref = oracle.attn_contig(q[r:r + 1], np.concatenate([kh, k[r:r + 1]]),
                                     np.concatenate([vh, v[r:r + 1]]), H, G, D, True,
                                     wl.scale)
        assert rc == 0
        assert_close(got[r:r + 1], ref, "m256 row %d (ctx %d)" % (r, wl.ctx[r]))
        return r
    assert _parallel(check, range(M)) == list(range(M))
    pool.advance(seqs_np, 1, check=True)
    pool.close()


def test_verify_m256_full_size_sampled_rows_with_rewind():
    """The verify legs' launches: every sequence of the M=256 pool appends 4
    drafted rows and attends them offset-causally, keeps a seeded 1..4 of
    them (truncate), then appends and attends 8 more.  Sampled rows against
    the oracle over the history plus the kept rows, at both steps."""
    wl = synth.decode_m256(max_steps=16)
    H, G, D, M = wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.M
    pool = _pool_for(wl)
    seqs = [pool.seq_new(wl.max_tokens) for _ in range(M)]
    f = HistoryFiller(wl, int(wl.ctx.max()))
    f.fill(pool, seqs, wl.ctx)
    f.close()
    seqs_np = np.asarray(seqs, np.int32)
    gen = np.random.default_rng(41)
    kept = [np.zeros((0, G * D), np.float32) for _ in range(M)]
    kept_v = [np.zeros((0, G * D), np.float32) for _ in range(M)]
    rows = sorted({int(np.argmin(wl.ctx)), int(np.argmax(wl.ctx)), 1, 77, 255} |
                  set(range(0, M, 8)))
    for n_q in (4, 8):
        q = gen.standard_normal((M * n_q, H * D), dtype=np.float32)
        k = gen.standard_normal((M * n_q, G * D), dtype=np.float32)
        v = gen.standard_normal((M * n_q, G * D), dtype=np.float32)
        pool.ensure_append(seqs_np, n_q, check=True)
        pool.append_layer(seqs_np, n_q, 0, dev(k), dev(v), check=True)
        nb = pool.verify_workspace_bytes(seqs_np, n_q, H)
        ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
        out = torch.full((M * n_q, H * D), float("nan"), device="cuda")
        pool.attn_paged_verify(seqs_np, n_q, 0, H, G, D, dev(q), wl.scale, out, ws=ws,
                               check=True)
        pool.advance(seqs_np, n_q, check=True)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.all(np.isfinite(got))
        assert np.abs(got).max() < 10

        def check(r):
            kh, vh = wl.history(r)
            sl = slice(r * n_q, (r + 1) * n_q)
            rc, ref = oracle.attn_contig(q[sl], np.concatenate([kh, kept[r], k[sl]]),
                                         np.concatenate([vh, kept_v[r], v[sl]]), H, G, D,
                                         True, wl.scale)
            assert rc == 0
            assert_close(got[sl], ref, "verify n_q %d row %d (ctx %d)" % (n_q, r, wl.ctx[r]))
            return r
        assert _parallel(check, rows) == rows
        # keep a seeded 1..n_q of the drafted rows, rewind the rest
        accept = gen.integers(1, n_q + 1, size=M)
        for r, s in enumerate(seqs):
            new_len = int(wl.ctx[r]) + kept[r].shape[0] + int(accept[r])
            pool.seq_truncate(s, new_len, check=True)
            assert pool.seq_len(s) == new_len
            kept[r] = np.concatenate([kept[r], k[r * n_q:r * n_q + int(accept[r])]])
            kept_v[r] = np.concatenate([kept_v[r], v[r * n_q:r * n_q + int(accept[r])]])
    pool.close()


def test_prefill_full_size_every_16th_query():
    """Every 16th chunk query and the tile-edge queries of all 8 sequences of
    the 8 x (3584 + 512) prefill against the oracle."""
    wl = synth.prefill_8x3584p512()
    H, G, D, M, n_q = wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.M, wl.chunk
    pool = _pool_for(wl)
    seqs = [pool.seq_new(wl.max_tokens) for _ in range(M)]
    f = HistoryFiller(wl, wl.cached)
    f.fill(pool, seqs, [wl.cached] * M)
    f.close()
    chunks = [wl.chunk_inputs(r) for r in range(M)]
    Q = np.concatenate([c[0] for c in chunks])
    K = np.concatenate([c[1] for c in chunks])
    V = np.concatenate([c[2] for c in chunks])
    seqs_np = np.asarray(seqs, np.int32)
    pool.ensure_append(seqs_np, n_q, check=True)
    pool.append_layer(seqs_np, n_q, 0, dev(K), dev(V), check=True)
    out = torch.full((M * n_q, H * D), float("nan"), device="cuda")
    pool.attn_paged_prefill(seqs_np, n_q, 0, H, G, D, dev(Q), True, wl.scale, out,
                            check=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    queries = sorted(set(range(0, n_q, 16)) |
                     {1, 31, 32, 33, 63, 64, 127, 128, 255, 256, 480, 510, 511})

    # one sequence per worker would leave most host cores idle: split the
    # query list of each sequence four ways
    parts = [(r, queries[j::4]) for r in range(M) for j in range(4)]

    def check_part(job):
        r, qs = job
        kh, vh = wl.history(r)
        Kall = np.concatenate([kh, chunks[r][1]])
        Vall = np.concatenate([vh, chunks[r][2]])
        for i in qs:
            nk = wl.cached + i + 1
            rc, ref = oracle.attn_contig(chunks[r][0][i:i + 1], Kall[:nk], Vall[:nk],
                                         H, G, D, True, wl.scale)
            assert rc == 0
            assert_close(got[r * n_q + i:r * n_q + i + 1], ref, "seq %d query %d" % (r, i))
        return len(qs)
    assert sum(_parallel(check_part, parts)) == M * len(queries)
    pool.close()


def _oracle_meta(wl, n_layers=1):
    o = oracle.Pool(wl.n_blocks, wl.block_size, n_layers, wl.n_kv_heads,
                    wl.head_dim, max_seqs=wl.n_forks + 8, with_storage=False)
    o.set_free_order(wl.free_order())
    return o


def _state(p, seqs):
    return (p.refcounts().tolist(), p.free_stack().tolist(),
            [(p.seq_len(s), None if p.seq_pages(s) is None else p.seq_pages(s).tolist())
             for s in seqs])


@pytest.mark.parametrize("prefix,n_forks,steps", [
    (2048, 64, 256),   # the forked-batch workload as specified (block-aligned prefix)
    (2053, 16, 24),    # non-aligned prefix: every fork copies the shared tail block
])
def test_forked_prefix_decode_and_rewind(prefix, n_forks, steps):
    wl = synth.forked_2048x64(steps=steps, prefix=prefix)
    wl.n_forks = n_forks
    H, G, D = wl.n_heads, wl.n_kv_heads, wl.head_dim
    pool = pkv.Pool(wl.n_blocks, wl.block_size, 1, G, D, max_seqs=n_forks + 8)
    pool.set_free_order(wl.free_order())
    o = _oracle_meta(wl)
    parent = pool.seq_new(wl.max_tokens)
    assert o.seq_new(wl.max_tokens) == parent
    pk, pv = wl.prefix_kv()
    pool.ensure_append([parent], prefix, check=True)
    pool.append_layer([parent], prefix, 0, dev(pk), dev(pv), check=True)
    pool.advance([parent], prefix, check=True)
    assert o.ensure_append([parent], prefix) == 0 and o.advance([parent], prefix) == 0
    forks = [pool.seq_fork(parent) for _ in range(n_forks)]
    assert [o.seq_fork(parent) for _ in range(n_forks)] == forks
    assert pool.seq_free(parent) == 0 and o.seq_free(parent) == 0
    ref = pool.refcounts()
    for b in pool.seq_pages(forks[0]):
        assert ref[b] == n_forks
    assert _state(pool, forks) == _state(o, forks)

    # per-step inputs of every fork
    steps_in = [[wl.fork_step(f, t) for f in range(n_forks)] for t in range(steps)]
    seqs_np = np.asarray(forks, np.int32)
    ws = torch.empty(pool.decode_workspace_bytes(seqs_np, H) +
                     n_forks * H * (D + 2) * 4 * 2, dtype=torch.uint8, device="cuda")
    outs = []
    for t in range(steps):
        q = np.stack([x[0] for x in steps_in[t]])
        k = np.stack([x[1] for x in steps_in[t]])
        v = np.stack([x[2] for x in steps_in[t]])
        pool.ensure_append(seqs_np, 1, check=True)
        assert o.ensure_append(forks, 1) == 0
        pool.append_layer(seqs_np, 1, 0, dev(k), dev(v), check=True)
        out = torch.empty((n_forks, H * D), device="cuda")
        pool.attn_paged_decode(seqs_np, 0, H, G, D, dev(q), wl.scale, out, ws=ws,
                               check=True)
        pool.advance(seqs_np, 1, check=True)
        assert o.advance(forks, 1) == 0
        outs.append(out)
        if t == 0:
            assert _state(pool, forks) == _state(o, forks)
    torch.cuda.synchronize()
    assert _state(pool, forks) == _state(o, forks)
    if prefix % wl.block_size:
        # the shared partial tail was copied once per fork
        ref = pool.refcounts()
        tails = {int(pool.seq_pages(f)[prefix // wl.block_size]) for f in forks}
        assert len(tails) == n_forks and all(ref[b] == 1 for b in tails)

    # every fork against the oracle at four steps (first, two inner, last)
    check_steps = sorted({0, steps // 3, (2 * steps) // 3, steps - 1})
    got = {t: outs[t].cpu().numpy() for t in check_steps}

    def check(f):
        for t in check_steps:
            kk = np.concatenate([pk] + [steps_in[s][f][1][None] for s in range(t + 1)])
            vv = np.concatenate([pv] + [steps_in[s][f][2][None] for s in range(t + 1)])
            rc, r_ = oracle.attn_contig(steps_in[t][f][0][None], kk, vv, H, G, D, True,
                                        wl.scale)
            assert rc == 0
            assert_close(got[t][f:f + 1], r_, "fork %d step %d" % (f, t))
        return f
    assert _parallel(check, range(n_forks)) == list(range(n_forks))

    # rewind: even forks go back to the fork point and replay their odd
    # partner's stream; every output must equal the partner's bit for bit
    evens = forks[0::2]
    for s in evens:
        assert pool.seq_truncate(s, prefix) == 0 and o.seq_truncate(s, prefix) == 0
    assert _state(pool, forks) == _state(o, forks)
    ev_np = np.asarray(evens, np.int32)
    for t in range(steps):
        q = np.stack([steps_in[t][f + 1][0] for f in range(0, n_forks, 2)])
        k = np.stack([steps_in[t][f + 1][1] for f in range(0, n_forks, 2)])
        v = np.stack([steps_in[t][f + 1][2] for f in range(0, n_forks, 2)])
        pool.ensure_append(ev_np, 1, check=True)
        assert o.ensure_append(evens, 1) == 0
        pool.append_layer(ev_np, 1, 0, dev(k), dev(v), check=True)
        out = torch.empty((len(evens), H * D), device="cuda")
        pool.attn_paged_decode(ev_np, 0, H, G, D, dev(q), wl.scale, out, ws=ws,
                               check=True)
        pool.advance(ev_np, 1, check=True)
        assert o.advance(evens, 1) == 0
        assert bits_equal(out, outs[t][1::2]), "rewind step %d" % t
    assert _state(pool, forks) == _state(o, forks)
    pool.close()

"""GPU parity of shared-prefix decode (pkv_attn_paged_decode_shared): rows of
a batch that share leading blocks after a fork ("nx_paged_kv_gate.nx
source", fork part: the forks hold the same blocks by reference count) have
that prefix attended once per kv head for all of them.

Bars: outputs within 1e-4 + 1e-4 * |oracle| and within the same tolerance
of pkv_attn_paged_decode; pool state untouched by the call (bit-exact with
the oracle pool through the steps); two rows of one group with identical
inputs give identical bits (the rewind replay of the forked workload).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_layer_amd as pkv
import synth
from pkv_gpu import assert_close, bits_equal, dev, fill_history

pytestmark = pytest.mark.gpu


def _rand(rng, shape):
    return rng.standard_normal(shape).astype(np.float32)


def _state(p, seqs):
    return (p.refcounts().tolist(), p.free_stack().tolist(),
            [(p.seq_len(s), None if p.seq_pages(s) is None else p.seq_pages(s).tolist())
             for s in seqs])


def _decode(pool, seqs, q, H, G, D, scale, shared):
    M = len(seqs)
    nb = (pool.decode_shared_workspace_bytes(seqs, H) if shared
          else pool.decode_workspace_bytes(seqs, H))
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
    out = torch.full((M, H * D), float("nan"), device="cuda")
    if shared:
        pool.attn_paged_decode_shared(seqs, 0, H, G, D, dev(q), scale, out, ws=ws,
                                      check=True)
    else:
        pool.attn_paged_decode(seqs, 0, H, G, D, dev(q), scale, out, ws=ws, check=True)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("H,G", [(32, 8), (64, 8), (16, 8)])
def test_mixed_batch_with_two_fork_groups(H, G):
    """Batch = forks of prefix A (2053 rows, non-aligned), forks of prefix B
    (700 rows), a fork of A taken after A grew (longer common prefix for
    that pair only), and unrelated sequences; decode several steps."""
    D, B = 128, 16
    rng = np.random.default_rng(H)
    pool = pkv.Pool(1200, B, 1, G, D, max_seqs=32)
    opool = oracle.Pool(1200, B, 1, G, D, max_seqs=32, with_storage=False)
    perm = rng.permutation(pool.n_blocks)
    pool.set_free_order(perm)
    opool.set_free_order(perm)
    hist = {}

    def new_seq(n, cap=4096):
        s = pool.seq_new(cap)
        assert opool.seq_new(cap) == s
        kv = (_rand(rng, (n, G * D)), _rand(rng, (n, G * D)))
        fill_history(pool, [s], lambda r: kv)
        assert opool.ensure_append([s], n) == 0 and opool.advance([s], n) == 0
        hist[s] = [list(kv[0]), list(kv[1])]
        return s

    def fork(s):
        f = pool.seq_fork(s)
        assert opool.seq_fork(s) == f
        hist[f] = [list(hist[s][0]), list(hist[s][1])]
        return f

    a = new_seq(2053)
    b = new_seq(700)
    lone = [new_seq(300), new_seq(1500)]
    fa = [fork(a) for _ in range(5)]
    fb = [fork(b) for _ in range(3)]
    # a grows 40 rows, then a later fork shares those too
    kv = (_rand(rng, (40, G * D)), _rand(rng, (40, G * D)))
    pool.ensure_append([a], 40, check=True)
    pool.append_layer([a], 40, 0, dev(kv[0]), dev(kv[1]), check=True)
    pool.advance([a], 40, check=True)
    assert opool.ensure_append([a], 40) == 0 and opool.advance([a], 40) == 0
    hist[a][0].extend(kv[0])
    hist[a][1].extend(kv[1])
    late = fork(a)
    seqs = [fa[0], lone[0], b, fa[1], late, fb[0], a, fa[2], lone[1], fb[1], fa[3],
            fb[2], fa[4]]
    scale = float(np.float32(1 / math.sqrt(D)))
    M = len(seqs)
    for step in range(3):
        q = _rand(rng, (M, H * D))
        k = _rand(rng, (M, G * D))
        v = _rand(rng, (M, G * D))
        pool.ensure_append(seqs, 1, check=True)
        assert opool.ensure_append(seqs, 1) == 0
        pool.append_layer(seqs, 1, 0, dev(k), dev(v), check=True)
        out_s = _decode(pool, seqs, q, H, G, D, scale, True)
        out_p = _decode(pool, seqs, q, H, G, D, scale, False)
        assert_close(out_s.cpu().numpy(), out_p.cpu().numpy(), "shared vs plain")
        got = out_s.cpu().numpy()
        for r, s in enumerate(seqs):
            hist[s][0].append(k[r])
            hist[s][1].append(v[r])
            rc, ref = oracle.attn_contig(q[r:r + 1], np.stack(hist[s][0]),
                                         np.stack(hist[s][1]), H, G, D, True, scale)
            assert rc == 0
            assert_close(got[r:r + 1], ref, "step %d row %d" % (step, r))
        pool.advance(seqs, 1, check=True)
        assert opool.advance(seqs, 1) == 0
        assert _state(pool, seqs) == _state(opool, seqs)


def test_forked_workload_shared_decode_and_rewind():
    """The forked workload at reduced steps: 64 forks of a 2048-row prefix,
    shared-prefix decode vs the oracle on sampled rows and vs plain decode on
    every row; then the even forks rewind to the fork point and replay their
    odd partner's stream, and every replayed output equals the partner's bit
    for bit (both rows sit in the same group with the same inputs)."""
    wl = synth.forked_2048x64(steps=12)
    H, G, D, F = wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.n_forks
    pool = pkv.Pool(wl.n_blocks, wl.block_size, 1, G, D, max_seqs=F + 8)
    pool.set_free_order(wl.free_order())
    parent = pool.seq_new(wl.max_tokens)
    pk, pv = wl.prefix_kv()
    fill_history(pool, [parent], lambda r: (pk, pv))
    forks = [pool.seq_fork(parent) for _ in range(F)]
    pool.seq_free(parent, check=True)
    steps_in = [[wl.fork_step(f, t) for f in range(F)] for t in range(wl.steps)]
    outs = []
    for t in range(wl.steps):
        q = np.stack([x[0] for x in steps_in[t]])
        k = np.stack([x[1] for x in steps_in[t]])
        v = np.stack([x[2] for x in steps_in[t]])
        pool.ensure_append(forks, 1, check=True)
        pool.append_layer(forks, 1, 0, dev(k), dev(v), check=True)
        out = _decode(pool, forks, q, H, G, D, wl.scale, True)
        if t in (0, wl.steps - 1):
            plain = _decode(pool, forks, q, H, G, D, wl.scale, False)
            assert_close(out.cpu().numpy(), plain.cpu().numpy(), "plain step %d" % t)
        pool.advance(forks, 1, check=True)
        outs.append(out)
    for f in (0, 17, F - 1):
        for t in (0, wl.steps - 1):
            kk = np.concatenate([pk] + [steps_in[s][f][1][None] for s in range(t + 1)])
            vv = np.concatenate([pv] + [steps_in[s][f][2][None] for s in range(t + 1)])
            rc, ref = oracle.attn_contig(steps_in[t][f][0][None], kk, vv, H, G, D,
                                         True, wl.scale)
            assert rc == 0
            assert_close(outs[t][f:f + 1].cpu().numpy(), ref, "fork %d step %d" % (f, t))
    evens = forks[0::2]
    for s in evens:
        pool.seq_truncate(s, wl.prefix, check=True)
    odds = forks[1::2]
    for t in range(wl.steps):
        q = np.stack([steps_in[t][f + 1][0] for f in range(0, F, 2)])
        k = np.stack([steps_in[t][f + 1][1] for f in range(0, F, 2)])
        v = np.stack([steps_in[t][f + 1][2] for f in range(0, F, 2)])
        pool.ensure_append(evens, 1, check=True)
        pool.append_layer(evens, 1, 0, dev(k), dev(v), check=True)
        out = _decode(pool, evens, q, H, G, D, wl.scale, True)
        pool.advance(evens, 1, check=True)
        assert bits_equal(out, outs[t][1::2]), "rewind step %d" % t
    assert len(odds) == len(evens)


def test_shared_decode_with_rope_and_no_groups():
    """Rotary embedding applies to the prefix queries as well; a batch with
    no shared prefix needs no prefix work and equals plain decode bit for
    bit."""
    H, G, D, B = 32, 8, 128, 16
    rng = np.random.default_rng(3)
    pool = pkv.Pool(200, B, 1, G, D, max_seqs=8)
    rope = pkv.Rope(D, math.log(10000.0), 2048)
    pool.set_rope(rope)
    base = pool.seq_new(1024)
    pk, pv = _rand(rng, (600, G * D)), _rand(rng, (600, G * D))
    fill_history(pool, [base], lambda r: (pk, pv))
    forks = [pool.seq_fork(base) for _ in range(3)]
    q = _rand(rng, (3, H * D))
    k = _rand(rng, (3, G * D))
    v = _rand(rng, (3, G * D))
    pool.ensure_append(forks, 1, check=True)
    pool.append_layer(forks, 1, 0, dev(k), dev(v), check=True)
    out = _decode(pool, forks, q, H, G, D, 0.08, True)
    Kt = oracle.rope(pk, G, D, np.arange(600), math.log(10000.0))[1]
    for r in range(3):
        kr = oracle.rope(k[r:r + 1], G, D, [600], math.log(10000.0))[1]
        qr = oracle.rope(q[r:r + 1], H, D, [600], math.log(10000.0))[1]
        rc, ref = oracle.attn_contig(qr, np.concatenate([Kt, kr]),
                                     np.concatenate([pv, v[r:r + 1]]), H, G, D, True, 0.08)
        assert_close(out[r:r + 1].cpu().numpy(), ref, "rope fork %d" % r)
    pool.advance(forks, 1, check=True)
    # distinct sequences: the shared entry point takes the plain path
    solo = [pool.seq_new(64), pool.seq_new(64)]
    hs = [(_rand(rng, (n, G * D)), _rand(rng, (n, G * D))) for n in (40, 9)]
    fill_history(pool, solo, lambda r: hs[r])
    batch = solo + forks[:1]
    q = _rand(rng, (3, H * D))
    k = _rand(rng, (3, G * D))
    v = _rand(rng, (3, G * D))
    pool.ensure_append(batch, 1, check=True)
    pool.append_layer(batch, 1, 0, dev(k), dev(v), check=True)
    assert pool.decode_shared_workspace_bytes(batch, H) == \
        pool.decode_workspace_bytes(batch, H)
    o1 = _decode(pool, batch, q, H, G, D, 0.08, True)
    o2 = _decode(pool, batch, q, H, G, D, 0.08, False)
    assert bits_equal(o1, o2)


def test_shared_workspace_check():
    H, G, D = 32, 8, 128
    rng = np.random.default_rng(4)
    pool = pkv.Pool(120, 16, 1, G, D, max_seqs=8)
    base = pool.seq_new(1024)
    pk, pv = _rand(rng, (512, G * D)), _rand(rng, (512, G * D))
    fill_history(pool, [base], lambda r: (pk, pv))
    forks = [pool.seq_fork(base) for _ in range(2)]
    pool.ensure_append(forks, 1, check=True)
    kv = torch.zeros((2, G * D), device="cuda")
    pool.append_layer(forks, 1, 0, kv, kv, check=True)
    need = pool.decode_shared_workspace_bytes(forks, H)
    # 512 prefix keys = 4 prefix splits, one own split each
    assert need == 2 * (4 + 1) * H * (D + 2) * 4
    q = torch.zeros((2, H * D), device="cuda")
    out = torch.empty_like(q)
    small = torch.empty(need - 4, dtype=torch.uint8, device="cuda")
    assert pool.attn_paged_decode_shared(forks, 0, H, G, D, q, 0.1, out, ws=small) \
        == pkv.BAD_ARG
    torch.cuda.synchronize()

"""GPU: the append-then-attend call (pkv_attn_with_paged_decode, the pages'
per-layer wrapper "nx_f32_attn_with_paged" with one new row per sequence)
against the two calls it stands for, pkv_append_layer +
pkv_attn_paged_decode, on twin pools (same placement, same history, same
operations); and the same for the shared-prefix form.  Two layers per step
unless stated.

Bars: outputs bit-identical at every step; every written position of the
pools bit-identical afterwards; reference counts and page tables identical;
one step checked against the oracle at 1e-4 + 1e-4 * |oracle|.  Cases: GQA
groups 1, 2, 4, 8 over page boundaries, rotary table on, two layers per
step, forks (a fork's pending page-table entries and the copy of a shared
tail), rows of the deep decode form, forks sharing a prefix through the
shared-prefix decode, the generic kernel's shapes, and the error path
(nothing launched).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_layer_amd as pkv
from pkv_gpu import assert_close, bits_equal, dev

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / math.sqrt(128)))


def _twins(lens, G, D, B=16, n_layers=1, seed=0, extra=40, rope=None):
    """Two pools with the same placement and the same cached rows."""
    rng = np.random.default_rng(seed)
    n_blocks = sum((l + extra) // B + 2 for l in lens) + 8
    order = rng.permutation(n_blocks)
    hist = [[(rng.standard_normal((l, G * D)).astype(np.float32),
              rng.standard_normal((l, G * D)).astype(np.float32)) for l in lens]
            for _ in range(n_layers)]
    pools = []
    for _ in range(2):
        p = pkv.Pool(n_blocks, B, n_layers, G, D, max_seqs=len(lens) + 8)
        p.set_free_order(order)
        if rope is not None:
            p.set_rope(rope)
        seqs = [p.seq_new(l + extra) for l in lens]
        for layer in range(n_layers):
            # history of every layer, then one advance per sequence
            for r, s in enumerate(seqs):
                k, v = hist[layer][r]
                if k.shape[0] == 0:
                    continue
                if layer == 0:
                    p.ensure_append([s], k.shape[0], check=True)
                p.append_layer([s], k.shape[0], layer, dev(k), dev(v), check=True)
        for r, s in enumerate(seqs):
            if lens[r]:
                p.advance([s], lens[r], check=True)
        pools.append((p, seqs))
    torch.cuda.synchronize()
    return pools, hist, rng


def _step(pool, seqs, q, k, v, H, G, D, one_call, layers=1):
    """One decode step over all layers (q, k, v per layer); outputs."""
    M = len(seqs)
    pool.ensure_append(seqs, 1, check=True)
    nb = pool.decode_workspace_bytes(seqs, H)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
    outs = []
    for layer in range(layers):
        out = torch.full((M, H * D), float("nan"), device="cuda")
        if one_call:
            pool.attn_with_paged_decode(seqs, layer, H, G, D, q[layer], k[layer], v[layer],
                                        SCALE, out, ws=ws, check=True)
        else:
            pool.append_layer(seqs, 1, layer, k[layer], v[layer], check=True)
            pool.attn_paged_decode(seqs, layer, H, G, D, q[layer], SCALE, out, ws=ws,
                                   check=True)
        outs.append(out)
    pool.advance(seqs, 1, check=True)
    torch.cuda.synchronize()
    return outs


def _same_pools(a, sa, b, sb):
    """Same reference counts, page tables and lengths, and the same bits at
    every position below each sequence's length (slots past it are never
    written and hold whatever the storage held)."""
    assert a.refcounts().tolist() == b.refcounts().tolist()
    B = a.block_size
    shape = (a.n_blocks, a.n_layers, 2, a.n_kv_heads, B, a.head_dim)
    va, vb = a.storage.view(torch.float32).view(shape), b.storage.view(torch.float32).view(shape)
    for x, y in zip(sa, sb):
        n = a.seq_len(x)
        assert n == b.seq_len(y)
        pa, pb = a.seq_pages(x), b.seq_pages(y)
        assert pa.tolist() == pb.tolist()
        pos = np.arange(n)
        blk = torch.as_tensor(pa[pos // B].astype(np.int64), device="cuda")
        slot = torch.as_tensor(pos % B, device="cuda")
        ra = va[blk].permute(0, 4, 1, 2, 3, 5)[torch.arange(n, device="cuda"), slot]
        rb = vb[blk].permute(0, 4, 1, 2, 3, 5)[torch.arange(n, device="cuda"), slot]
        assert torch.equal(ra, rb), "sequence %d" % x


def _run(lens, H, G, D=128, steps=20, seed=0, layers=2, rope=None):
    (pa, sa), (pb, sb) = _twins(lens, G, D, n_layers=layers, seed=seed, rope=rope)[0]
    rng = np.random.default_rng(seed + 1)
    M = len(lens)
    for t in range(steps):
        q = [dev(rng.standard_normal((M, H * D))) for _ in range(layers)]
        k = [dev(rng.standard_normal((M, G * D))) for _ in range(layers)]
        v = [dev(rng.standard_normal((M, G * D))) for _ in range(layers)]
        oa = _step(pa, sa, q, k, v, H, G, D, one_call=False, layers=layers)
        ob = _step(pb, sb, q, k, v, H, G, D, one_call=True, layers=layers)
        for x, y in zip(oa, ob):
            assert bits_equal(x, y), "step %d" % t
    _same_pools(pa, sa, pb, sb)
    return pa, sa, pb, sb


@pytest.mark.parametrize("H,G", [(8, 8), (16, 8), (32, 8), (64, 8)])
def test_with_paged_equals_append_then_decode(H, G):
    # lengths around page and split edges; 20 steps cross page boundaries
    pa, sa, pb, sb = _run([1, 15, 16, 255, 513, 2047, 3000, 6150], H, G, steps=20, seed=H)
    form = "decode_fast_kernel<%d, PagedMap, false>" % (H // G)
    assert pa.kernel_name(pkv.K_DECODE) == form and pb.kernel_name(pkv.K_DECODE) == form


def test_with_paged_two_layers_and_rope():
    rope = pkv.Rope(128, math.log(10000.0), 8192)
    _run([5, 700, 4100], 32, 8, steps=18, seed=7, layers=2, rope=rope)


def test_with_paged_matches_oracle():
    lens = [33, 1000, 2500]
    H, G, D = 32, 8, 128
    pools, hist, _ = _twins(lens, G, D, seed=3, n_layers=2)
    (pb, sb) = pools[1]
    rng = np.random.default_rng(11)
    q = [rng.standard_normal((3, H * D)).astype(np.float32) for _ in range(2)]
    k = [rng.standard_normal((3, G * D)).astype(np.float32) for _ in range(2)]
    v = [rng.standard_normal((3, G * D)).astype(np.float32) for _ in range(2)]
    outs = _step(pb, sb, [dev(x) for x in q], [dev(x) for x in k], [dev(x) for x in v],
                 H, G, D, one_call=True, layers=2)
    for layer in range(2):
        o = outs[layer].cpu().numpy()
        h = hist[layer]
        for r in range(3):
            rc, ref = oracle.attn_contig(q[layer][r:r + 1],
                                         np.concatenate([h[r][0], k[layer][r:r + 1]]),
                                         np.concatenate([h[r][1], v[layer][r:r + 1]]),
                                         H, G, D, True, SCALE)
            assert rc == 0
            assert_close(o[r:r + 1], ref, "layer %d row %d" % (layer, r))


def test_with_paged_after_fork_and_copy_on_append():
    """Forks: a fork's page table is a pending mirror patch at the step's
    first layer, and the shared partial tail is copied before the new rows
    land."""
    H, G, D = 32, 8, 128
    (pa, sa), (pb, sb) = _twins([1000, 37], G, D, seed=5, extra=80, n_layers=2)[0]
    rng = np.random.default_rng(6)
    ca, cb = pa.seq_fork(sa[0]), pb.seq_fork(sb[0])
    sa2, sb2 = sa + [ca], sb + [cb]
    for t in range(24):
        q = [dev(rng.standard_normal((3, H * D))) for _ in range(2)]
        k = [dev(rng.standard_normal((3, G * D))) for _ in range(2)]
        v = [dev(rng.standard_normal((3, G * D))) for _ in range(2)]
        oa = _step(pa, sa2, q, k, v, H, G, D, one_call=False, layers=2)
        ob = _step(pb, sb2, q, k, v, H, G, D, one_call=True, layers=2)
        assert bits_equal(oa[0], ob[0]) and bits_equal(oa[1], ob[1]), t
        if t == 10:
            # rewind the fork: its tail page is shared with the parent again,
            # so the next step copies it (a pending entry at the new row's page)
            assert pa.seq_truncate(ca, 990) == 0 and pb.seq_truncate(cb, 990) == 0
    _same_pools(pa, sa2, pb, sb2)


def test_with_paged_generic_shape():
    # head_dim 64: the generic kernel; same contract
    (pa, sa), (pb, sb) = _twins([3, 90, 300], 4, 64, seed=9, n_layers=2)[0]
    rng = np.random.default_rng(10)
    for t in range(6):
        q = [dev(rng.standard_normal((3, 12 * 64))) for _ in range(2)]
        k = [dev(rng.standard_normal((3, 4 * 64))) for _ in range(2)]
        v = [dev(rng.standard_normal((3, 4 * 64))) for _ in range(2)]
        oa = _step(pa, sa, q, k, v, 12, 4, 64, one_call=False, layers=2)
        ob = _step(pb, sb, q, k, v, 12, 4, 64, one_call=True, layers=2)
        assert bits_equal(oa[0], ob[0]) and bits_equal(oa[1], ob[1]), t
    _same_pools(pa, sa, pb, sb)


def test_with_paged_errors_leave_the_pool_unchanged():
    H, G, D = 32, 8, 128
    # full last pages: the next rows need pages not reserved yet
    (p, s), _ = _twins([608, 32], G, D, seed=12)[0]
    q = dev(np.ones((2, H * D)))
    k = dev(np.ones((2, G * D)))
    out = torch.zeros((2, H * D), device="cuda")
    # rows not ensured
    assert p.attn_with_paged_decode(s, 0, H, G, D, q, k, k, SCALE, out) == pkv.ERR_SEQ
    p.ensure_append(s, 1, check=True)
    before = p.storage.clone()
    nb = p.decode_workspace_bytes(s, H)
    assert nb > 0
    small = torch.empty(nb - 4, dtype=torch.uint8, device="cuda")
    assert p.attn_with_paged_decode(s, 0, H, G, D, q, k, k, SCALE, out,
                                    ws=small) == pkv.BAD_ARG
    assert p.attn_with_paged_decode(s, 1, H, G, D, q, k, k, SCALE, out) == pkv.BAD_ARG
    q30 = dev(np.ones((2, 30 * D)))
    out30 = torch.zeros((2, 30 * D), device="cuda")
    assert p.attn_with_paged_decode(s, 0, 30, G, D, q30, k, k, SCALE, out30) == pkv.BAD_GQA
    torch.cuda.synchronize()
    assert torch.equal(before, p.storage)
    assert float(out.abs().sum()) == 0.0


def test_with_paged_deep_form():
    # rows of 8192+ keys: 2048-key splits, the decode kernel's deep form
    pa, sa, pb, sb = _run([9000, 300, 16385], 32, 8, steps=6, seed=21)
    assert pb.kernel_name(pkv.K_DECODE) == "decode_fast_kernel<4, PagedMap, true>"
    assert pa.kernel_name(pkv.K_DECODE) == "decode_fast_kernel<4, PagedMap, true>"


def test_with_paged_shared_prefix_decode():
    """pkv_attn_with_paged_decode_shared against pkv_append_layer +
    pkv_attn_paged_decode_shared on twin pools: forks of a 2100-row prefix,
    two layers per step."""
    H, G, D = 32, 8, 128
    (pa, sa), (pb, sb) = _twins([2100], G, D, seed=31, extra=60, n_layers=2)[0]
    fa = [pa.seq_fork(sa[0]) for _ in range(6)]
    fb = [pb.seq_fork(sb[0]) for _ in range(6)]
    assert fa == fb
    rng = np.random.default_rng(32)
    batch = sa + fa
    M = len(batch)
    ws = torch.empty(16 << 20, dtype=torch.uint8, device="cuda")
    for t in range(20):
        q = [dev(rng.standard_normal((M, H * D))) for _ in range(2)]
        k = [dev(rng.standard_normal((M, G * D))) for _ in range(2)]
        v = [dev(rng.standard_normal((M, G * D))) for _ in range(2)]
        outs = []
        for p, one_call in ((pa, False), (pb, True)):
            p.ensure_append(batch, 1, check=True)
            for layer in range(2):
                out = torch.full((M, H * D), float("nan"), device="cuda")
                if one_call:
                    p.attn_with_paged_decode_shared(batch, layer, H, G, D, q[layer], k[layer],
                                                    v[layer], SCALE, out, ws=ws, check=True)
                else:
                    p.append_layer(batch, 1, layer, k[layer], v[layer], check=True)
                    p.attn_paged_decode_shared(batch, layer, H, G, D, q[layer], SCALE, out,
                                               ws=ws, check=True)
                outs.append(out)
            p.advance(batch, 1, check=True)
        torch.cuda.synchronize()
        assert bits_equal(outs[0], outs[2]) and bits_equal(outs[1], outs[3]), t
    assert pb.kernel_name(pkv.K_PREFIX) == "shared_decode_kernel<4>"
    _same_pools(pa, batch, pb, batch)

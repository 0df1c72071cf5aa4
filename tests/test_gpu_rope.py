"""GPU parity of the fused rotary embedding ("nx_f32_llama_v4b.nx source",
nx_f32_llama_block_forward_v4b, RoPE step): with a rotary table set, the
library turns K inside the append scatter and Q inside the attention kernels;
the oracle turns them with its own rope function first and then attends.

Bars: attention outputs within 1e-4 + 1e-4 * |oracle|; stored K rows within
one float ulp of the oracle's turned rows (both evaluate the same double
expression; only the libm that made the table could differ), stored V rows
bit-exact; paged == contiguous bit-identical with the table on; position 0
turns nothing, so there the output equals the unturned path bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_layer_amd as pkv
from pkv_gpu import assert_close, bits_equal, dev, fill_contig, fill_history

pytestmark = pytest.mark.gpu

LB = math.log(10000.0)


def _turn(x, heads, D, positions, log_base=LB):
    rc, y = oracle.rope(x, heads, D, positions, log_base)
    assert rc == oracle.OK
    return y


def _stored_rows(pool, seq, layer, n):
    """(K, V) [n, G*D] of positions 0..n-1 read back from the pool storage
    ([block][layer][K,V][kv head][slot][dim])."""
    G, D, B = pool.n_kv_heads, pool.head_dim, pool.block_size
    st = pool.storage.view(torch.float32).view(pool.n_blocks, pool.n_layers, 2, G,
                                               B, D).cpu().numpy()
    pages = pool.seq_pages(seq)
    k = np.empty((n, G * D), np.float32)
    v = np.empty((n, G * D), np.float32)
    for p in range(n):
        blk, slot = pages[p // B], p % B
        k[p] = st[blk, layer, 0, :, slot, :].reshape(-1)
        v[p] = st[blk, layer, 1, :, slot, :].reshape(-1)
    return k, v


def _max_ulp(a, b):
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return int(np.abs(ai - bi).max()) if ai.size else 0


def _decode(pool, seqs, q, k, v, H, G, D, scale, layer=0):
    M = len(seqs)
    pool.ensure_append(seqs, 1, check=True)
    pool.append_layer(seqs, 1, layer, dev(k), dev(v), check=True)
    nb = pool.decode_workspace_bytes(seqs, H)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
    out = torch.full((M, H * D), float("nan"), device="cuda")
    pool.attn_paged_decode(seqs, layer, H, G, D, dev(q), scale, out, ws=ws,
                           check=True)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("H,G,D,B,log_base", [
    (32, 8, 128, 16, LB),                 # fast decode, group 4
    (64, 8, 128, 16, math.log(1e6)),      # fast decode, group 8, base 1e6
    (12, 4, 64, 16, LB),                  # generic kernel, vector append
    (6, 2, 42, 5, LB),                    # generic kernel, scalar append
])
def test_rope_decode_vs_oracle_and_contiguous(H, G, D, B, log_base):
    rng = np.random.default_rng(H + D + B)
    lens = [0, 1, 17, 511, 512, 1500]
    M = len(lens)
    rope = pkv.Rope(D, log_base, 4096)
    pool = pkv.Pool(sum(l // B + 3 for l in lens), B, 1, G, D, max_seqs=8)
    pool.set_rope(rope)
    pool.set_free_order(rng.permutation(pool.n_blocks))
    seqs = [pool.seq_new(l + 1) for l in lens]
    hist = [(rng.standard_normal((l, G * D)).astype(np.float32),
             rng.standard_normal((l, G * D)).astype(np.float32)) for l in lens]
    fill_history(pool, seqs, lambda r: hist[r])
    q = rng.standard_normal((M, H * D)).astype(np.float32)
    k = rng.standard_normal((M, G * D)).astype(np.float32)
    v = rng.standard_normal((M, G * D)).astype(np.float32)
    scale = float(np.float32(1 / math.sqrt(D)))
    out = _decode(pool, seqs, q, k, v, H, G, D, scale)
    got = out.cpu().numpy()
    for r, L in enumerate(lens):
        Kall = np.concatenate([hist[r][0], k[r:r + 1]])
        Vall = np.concatenate([hist[r][1], v[r:r + 1]])
        Kt = _turn(Kall, G, D, np.arange(L + 1), log_base)
        qt = _turn(q[r:r + 1], H, D, [L], log_base)
        rc, ref = oracle.attn_contig(qt, Kt, Vall, H, G, D, True, scale)
        assert rc == 0
        assert_close(got[r:r + 1], ref, "rope decode row %d (len %d)" % (r, L))
        ks, vs = _stored_rows(pool, seqs[r], 0, L + 1)
        assert _max_ulp(ks, Kt) <= 1, "stored K row %d" % r
        assert np.array_equal(vs.view(np.uint32), Vall.view(np.uint32))
    # the same kernels over a contiguous cache with the same table
    cc = pkv.ContigCache(M, 1, G, max(lens) + 1, D, block_size=B, rope=rope)
    fill_contig(cc, list(range(M)), lambda r: hist[r])
    cc.append(list(range(M)), lens, 1, 0, dev(k), dev(v))
    ws = torch.empty(max(cc.decode_workspace_bytes(lens, H), 4), dtype=torch.uint8,
                     device="cuda")
    cout = torch.full_like(out, float("nan"))
    cc.attn_decode(list(range(M)), lens, 0, H, dev(q), scale, cout, ws=ws)
    torch.cuda.synchronize()
    assert bits_equal(out, cout)


@pytest.mark.parametrize("H,G,D,B,cached,n_q,causal", [
    (32, 8, 128, 16, 0, 37, True),      # MFMA prefill
    (32, 8, 128, 16, 100, 77, True),
    (32, 8, 128, 16, 300, 5, False),
    (6, 2, 42, 5, 9, 7, True),          # generic kernel
])
def test_rope_prefill_vs_oracle_and_contiguous(H, G, D, B, cached, n_q, causal):
    rng = np.random.default_rng(cached * 7 + n_q)
    lens = [cached, cached + 3]
    M = len(lens)
    rope = pkv.Rope(D, LB, 1024)
    pool = pkv.Pool(sum((l + n_q) // B + 2 for l in lens), B, 1, G, D, max_seqs=4)
    pool.set_rope(rope)
    pool.set_free_order(rng.permutation(pool.n_blocks))
    seqs = [pool.seq_new(l + n_q) for l in lens]
    hist = [(rng.standard_normal((l, G * D)).astype(np.float32) * 0.5,
             rng.standard_normal((l, G * D)).astype(np.float32) * 0.5) for l in lens]
    fill_history(pool, seqs, lambda r: hist[r])
    Q = (rng.standard_normal((M * n_q, H * D)) * 0.5).astype(np.float32)
    K = (rng.standard_normal((M * n_q, G * D)) * 0.5).astype(np.float32)
    V = (rng.standard_normal((M * n_q, G * D)) * 0.5).astype(np.float32)
    scale = float(np.float32(1 / math.sqrt(D)))
    pool.ensure_append(seqs, n_q, check=True)
    pool.append_layer(seqs, n_q, 0, dev(K), dev(V), check=True)
    out = torch.full((M * n_q, H * D), float("nan"), device="cuda")
    pool.attn_paged_prefill(seqs, n_q, 0, H, G, D, dev(Q), causal, scale, out,
                            check=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for r, L in enumerate(lens):
        rows = slice(r * n_q, (r + 1) * n_q)
        Kt = _turn(np.concatenate([hist[r][0], K[rows]]), G, D, np.arange(L + n_q))
        Vc = np.concatenate([hist[r][1], V[rows]])
        Qt = _turn(Q[rows], H, D, L + np.arange(n_q))
        rc, ref = oracle.attn_contig(Qt, Kt, Vc, H, G, D, causal, scale)
        assert rc == 0
        assert_close(got[rows], ref, "rope prefill row %d" % r)
    cc = pkv.ContigCache(M, 1, G, max(lens) + n_q, D, block_size=B, rope=rope)
    fill_contig(cc, [0, 1], lambda r: hist[r])
    cc.append([0, 1], lens, n_q, 0, dev(K), dev(V))
    cout = torch.full_like(out, float("nan"))
    cc.attn_prefill([0, 1], lens, n_q, 0, H, dev(Q), causal, scale, cout)
    torch.cuda.synchronize()
    assert bits_equal(out, cout)


def test_rope_multistep_decode_positions_advance():
    """Three decode steps over two layers: each step's rows sit one position
    further on."""
    H, G, D, B = 32, 8, 128, 16
    rng = np.random.default_rng(11)
    lens = [40, 700]
    M, steps, layers = 2, 3, 2
    rope = pkv.Rope(D, LB, 2048)
    pool = pkv.Pool(sum((l + steps) // B + 2 for l in lens), B, layers, G, D,
                    max_seqs=4)
    pool.set_rope(rope)
    seqs = [pool.seq_new(l + steps) for l in lens]
    hist = {(r, L): (rng.standard_normal((lens[r], G * D)).astype(np.float32),
                     rng.standard_normal((lens[r], G * D)).astype(np.float32))
            for r in range(M) for L in range(layers)}
    for r, s in enumerate(seqs):
        pool.ensure_append([s], lens[r], check=True)
        for L in range(layers):
            pool.append_layer([s], lens[r], L, dev(hist[r, L][0]), dev(hist[r, L][1]),
                              check=True)
        pool.advance([s], lens[r], check=True)
    Ks = {(r, L): list(hist[r, L][0]) for r in range(M) for L in range(layers)}
    Vs = {(r, L): list(hist[r, L][1]) for r in range(M) for L in range(layers)}
    scale = 0.0883883
    for t in range(steps):
        pool.ensure_append(seqs, 1, check=True)
        for L in range(layers):
            q = rng.standard_normal((M, H * D)).astype(np.float32)
            k = rng.standard_normal((M, G * D)).astype(np.float32)
            v = rng.standard_normal((M, G * D)).astype(np.float32)
            pool.append_layer(seqs, 1, L, dev(k), dev(v), check=True)
            ws = torch.empty(max(pool.decode_workspace_bytes(seqs, H), 4),
                             dtype=torch.uint8, device="cuda")
            out = torch.empty((M, H * D), device="cuda")
            pool.attn_paged_decode(seqs, L, H, G, D, dev(q), scale, out, ws=ws,
                                   check=True)
            torch.cuda.synchronize()
            for r in range(M):
                Ks[r, L].append(k[r])
                Vs[r, L].append(v[r])
                n = lens[r] + t + 1
                Kt = _turn(np.stack(Ks[r, L]), G, D, np.arange(n))
                qt = _turn(q[r:r + 1], H, D, [n - 1])
                rc, ref = oracle.attn_contig(qt, Kt, np.stack(Vs[r, L]), H, G, D,
                                             True, scale)
                assert rc == 0
                assert_close(out[r:r + 1].cpu().numpy(), ref,
                             "step %d layer %d row %d" % (t, L, r))
        pool.advance(seqs, 1, check=True)


def test_rope_at_position_zero_turns_nothing():
    """An empty sequence's first row sits at position 0 (angle 0): the output
    equals the unturned pool's bit for bit; at position 1 it does not."""
    H, G, D = 32, 8, 128
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, H * D)).astype(np.float32)
    k = rng.standard_normal((2, G * D)).astype(np.float32)
    v = rng.standard_normal((2, G * D)).astype(np.float32)
    rope = pkv.Rope(D, LB, 16)
    outs = []
    for table in (rope, None):
        pool = pkv.Pool(4, 16, 1, G, D, max_seqs=2)
        pool.set_rope(table)
        s = pool.seq_new(8)
        outs.append(_decode(pool, [s], q, k[:1], v[:1], H, G, D, 0.1))
        pool.advance([s], 1, check=True)
        outs.append(_decode(pool, [s], q, k[1:], v[1:], H, G, D, 0.1))
    assert bits_equal(outs[0], outs[2])
    assert not bits_equal(outs[1], outs[3])


def test_rope_errors_and_switching_off():
    G, D = 8, 128
    rope = pkv.Rope(D, LB, 20)
    pool = pkv.Pool(8, 16, 1, G, D, max_seqs=2)
    assert pool.set_rope(pkv.Rope(64, LB, 20), check=False) == pkv.BAD_DIM
    pool.set_rope(rope)
    s = pool.seq_new(64)
    kv = torch.zeros((19, G * D), device="cuda")
    pool.ensure_append([s], 19, check=True)
    pool.append_layer([s], 19, 0, kv, kv, check=True)
    pool.advance([s], 19, check=True)
    # positions 19 and 20: the second is past the table
    pool.ensure_append([s], 2, check=True)
    kv2 = torch.zeros((2, G * D), device="cuda")
    before = (pool.refcounts().tolist(), pool.seq_pages(s).tolist(), pool.seq_len(s))
    assert pool.append_layer([s], 2, 0, kv2, kv2) == pkv.CAPACITY
    q = torch.zeros((2, 32 * D), device="cuda")
    out = torch.zeros_like(q)
    assert pool.attn_paged_prefill([s], 2, 0, 32, G, D, q, True, 0.1, out) \
        == pkv.CAPACITY
    ws = torch.empty(max(pool.decode_workspace_bytes([s], 32), 4), dtype=torch.uint8,
                     device="cuda")
    # decode: the one new row sits at position 19, inside the table
    assert pool.append_layer([s], 1, 0, kv2[:1], kv2[:1]) == pkv.OK
    assert pool.attn_paged_decode([s], 0, 32, G, D, q[:1], 0.1, out[:1], ws=ws) \
        == pkv.OK
    after = (pool.refcounts().tolist(), pool.seq_pages(s).tolist(), pool.seq_len(s))
    assert before == after
    # with the table off the two-row chunk goes through
    pool.set_rope(None)
    assert pool.append_layer([s], 2, 0, kv2, kv2) == pkv.OK
    assert pool.attn_paged_prefill([s], 2, 0, 32, G, D, q, True, 0.1, out) == pkv.OK
    torch.cuda.synchronize()
    with pytest.raises(ValueError):
        pkv.Rope(D - 1, LB, 20)
    with pytest.raises(ValueError):
        pkv.Rope(D, 0.0, 20)
    with pytest.raises(ValueError):
        pkv.Rope(D, LB, 0)
    # a contiguous descriptor whose table has another head size is rejected
    cc = pkv.ContigCache(1, 1, G, 16, D, rope=pkv.Rope(64, LB, 16))
    assert cc.append([0], [0], 1, 0, kv2[:1], kv2[:1], check=False) == pkv.BAD_ARG

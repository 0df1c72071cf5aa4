"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: pool / page-table / reference-count state bit-exact with the oracle;
float32 attention outputs within 1e-4 + 1e-4 * |oracle|; paged and
contiguous forms of the same kernel bit-identical on the GPU; outputs
independent (bitwise) of batch composition and block placement.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_layer_amd as pkv
import synth
from pkv_gpu import (assert_close, bits_equal, decode_pool, decode_step, dev,
                     fill_contig, fill_history)

pytestmark = pytest.mark.gpu


def _state(p, seqs):
    return (p.refcounts().tolist(), p.free_stack().tolist(),
            [(p.seq_len(s), None if p.seq_pages(s) is None else p.seq_pages(s).tolist())
             for s in seqs])


# --------------------------------------------------------------- tiny gate

def _gate_round(pool, opool, ccache, ocache, seq, qkv, n, gate, slot=0):
    """One append round: GPU paged, GPU contiguous, oracle paged, oracle
    contiguous, per layer.  Returns the GPU paged outputs per layer."""
    Q, K, V = qkv
    assert pool.ensure_append([seq], n) == 0
    assert opool.ensure_append([seq], n) == 0
    outs = []
    for L in range(gate.n_layers):
        c_len = ocache.seq_len if ocache is not None else None
        assert pool.append_layer([seq], n, L, dev(K), dev(V)) == 0
        out = torch.full((n, gate.q_dim), float("nan"), device="cuda")
        assert pool.attn_paged_prefill([seq], n, L, gate.n_heads, gate.n_kv_heads,
                                       gate.head_dim, dev(Q), True, gate.scale,
                                       out) == 0
        rc, ref = opool.attn_with_paged(Q, K, V, n, gate.n_heads, gate.n_kv_heads,
                                        gate.head_dim, seq, L, True, gate.scale)
        assert rc == 0
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, "gate layer %d" % L)
        if ccache is not None:
            ccache.append([slot], [c_len], n, L, dev(K), dev(V))
            cout = torch.full_like(out, float("nan"))
            ccache.attn_prefill([slot], [c_len], n, L, gate.n_heads, dev(Q), True,
                                gate.scale, cout)
            rc, cref = ocache.attn_with_cache(Q, K, V, n, gate.n_heads,
                                              gate.n_kv_heads, gate.head_dim, L,
                                              True, gate.scale)
            assert rc == 0
            torch.cuda.synchronize()
            assert bits_equal(out, cout), "paged != contiguous on the GPU"
            assert np.array_equal(ref.view(np.uint32), cref.view(np.uint32))
        outs.append(out.cpu().numpy())
    if ocache is not None:
        assert ocache.advance(n) == 0
    assert pool.advance([seq], n) == 0
    assert opool.advance([seq], n) == 0
    return np.stack(outs)


def test_tiny_gate_on_gpu():
    gate = synth.TinyGate()
    x = gate.inputs()
    # EQUIV: 3 rounds, paged == contiguous bitwise, both within tol of oracle
    pool = pkv.Pool(gate.n_blocks, gate.block_size, gate.n_layers,
                    gate.n_kv_heads, gate.head_dim, max_seqs=8)
    opool = oracle.Pool(gate.n_blocks, gate.block_size, gate.n_layers,
                        gate.n_kv_heads, gate.head_dim, max_seqs=8)
    cc = pkv.ContigCache(1, gate.n_layers, gate.n_kv_heads, gate.max_tokens,
                         gate.head_dim, block_size=gate.block_size)
    oc = oracle.Cache(gate.n_layers, gate.n_kv_heads, gate.max_tokens, gate.head_dim)
    s = pool.seq_new(gate.max_tokens)
    assert opool.seq_new(gate.max_tokens) == s
    for name, n in (("1", 5), ("2", 1), ("3", 3)):
        _gate_round(pool, opool, cc, oc, s, x[name], n, gate)
        assert _state(pool, [s]) == _state(opool, [s])

    # FORK + COW, then REWIND
    pool2 = pkv.Pool(gate.n_blocks, gate.block_size, gate.n_layers,
                     gate.n_kv_heads, gate.head_dim, max_seqs=8)
    op2 = oracle.Pool(gate.n_blocks, gate.block_size, gate.n_layers,
                      gate.n_kv_heads, gate.head_dim, max_seqs=8)
    a = pool2.seq_new(gate.max_tokens)
    op2.seq_new(gate.max_tokens)
    _gate_round(pool2, op2, None, None, a, x["1"], 5, gate)
    b = pool2.seq_fork(a)
    assert op2.seq_fork(a) == b
    assert pool2.refcounts()[pool2.seq_pages(a)[0]] == 2
    opA = _gate_round(pool2, op2, None, None, a, x["A"], 2, gate)
    opB = _gate_round(pool2, op2, None, None, b, x["B"], 2, gate)
    assert _state(pool2, [a, b]) == _state(op2, [a, b])
    pa, pb = pool2.seq_pages(a), pool2.seq_pages(b)
    ref = pool2.refcounts()
    assert pa[1] != pb[1] and ref[pa[1]] == 1 and ref[pb[1]] == 1
    assert pa[0] == pb[0] and ref[pa[0]] == 2

    # fresh contiguous replays on the GPU: bitwise equal to the forks
    for hist, ops in ((("1", "A"), opA), (("1", "B"), opB)):
        cc2 = pkv.ContigCache(1, gate.n_layers, gate.n_kv_heads, gate.max_tokens,
                              gate.head_dim, block_size=gate.block_size)
        pos = 0
        for name in hist:
            Q, K, V = x[name]
            n = Q.shape[0]
            outs = []
            for L in range(gate.n_layers):
                cc2.append([0], [pos], n, L, dev(K), dev(V))
                o = torch.empty((n, gate.q_dim), device="cuda")
                cc2.attn_prefill([0], [pos], n, L, gate.n_heads, dev(Q), True,
                                 gate.scale, o)
                outs.append(o)
            pos += n
        torch.cuda.synchronize()
        assert bits_equal(torch.stack(outs).cpu(), torch.from_numpy(ops))

    # REWIND: truncate A to the fork point and append B's rows -> B's outputs
    assert pool2.seq_truncate(a, 5) == 0 and op2.seq_truncate(a, 5) == 0
    opR = _gate_round(pool2, op2, None, None, a, x["B"], 2, gate)
    assert np.array_equal(opR.view(np.uint32), opB.view(np.uint32))
    assert _state(pool2, [a, b]) == _state(op2, [a, b])


# ------------------------------------------------------- decode, M = 32

def test_decode_m32_full_vs_oracle_and_contiguous():
    wl = synth.decode_m32()
    H, G, D = wl.n_heads, wl.n_kv_heads, wl.head_dim
    pool, seqs = decode_pool(wl)
    q, k, v = wl.step(0)
    out = decode_step(pool, seqs, q, k, v, H, G, D, wl.scale, advance=False)
    got = out.cpu().numpy()
    # oracle: every row, every head
    for r in range(wl.M):
        kh, vh = wl.history(r)
        K = np.concatenate([kh, k[r:r + 1]])
        V = np.concatenate([vh, v[r:r + 1]])
        rc, ref = oracle.attn_contig(q[r:r + 1], K, V, H, G, D, True, wl.scale)
        assert rc == 0
        assert_close(got[r:r + 1], ref, "decode m32 row %d" % r)
    # the same kernels over a contiguous cache: bit-identical
    cc = pkv.ContigCache(wl.M, 1, G, wl.max_tokens, D)
    fill_contig(cc, list(range(wl.M)), wl.history)
    lens = [int(c) for c in wl.ctx]
    cc.append(list(range(wl.M)), lens, 1, 0, dev(k), dev(v))
    ws = torch.empty(max(cc.decode_workspace_bytes(lens, H), 4), dtype=torch.uint8,
                     device="cuda")
    cout = torch.full_like(out, float("nan"))
    cc.attn_decode(list(range(wl.M)), lens, 0, H, dev(q), wl.scale, cout, ws=ws)
    torch.cuda.synchronize()
    assert bits_equal(out, cout)
    pool.advance(seqs, 1, check=True)


def test_decode_batch_and_placement_invariance():
    """A sequence's output does not depend on which other sequences share the
    batch, on its position in the batch, or on where its blocks sit."""
    wl = synth.decode_m32()
    wl.M = 6
    wl.ctx = wl.ctx[:6].copy()
    wl.ctx[0] = 1023  # total_k = 1024: two full splits
    wl.ctx[1] = 512   # split boundary + 1
    H, G, D = wl.n_heads, wl.n_kv_heads, wl.head_dim
    pool, seqs = decode_pool(wl)
    q, k, v = wl.step(0)
    full = decode_step(pool, seqs, q, k, v, H, G, D, wl.scale, advance=False)
    # each row alone, in reverse order batches
    for r in range(wl.M):
        nb = pool.decode_workspace_bytes([seqs[r]], H)
        ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
        o1 = torch.empty((1, H * D), device="cuda")
        pool.attn_paged_decode([seqs[r]], 0, H, G, D, dev(q[r:r + 1]), wl.scale, o1,
                               ws=ws, check=True)
        torch.cuda.synchronize()
        assert bits_equal(o1[0], full[r])
    rev = seqs[::-1]
    nb = pool.decode_workspace_bytes(rev, H)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
    orev = torch.empty_like(full)
    pool.attn_paged_decode(rev, 0, H, G, D, dev(q[::-1]), wl.scale, orev, ws=ws,
                           check=True)
    torch.cuda.synchronize()
    assert bits_equal(orev.flip(0), full)
    # a second pool with a different placement
    wl2 = synth.decode_m32()
    wl2.M, wl2.ctx, wl2.seed = wl.M, wl.ctx, wl.seed
    pool2 = pkv.Pool(wl.n_blocks, 16, 1, G, D, max_seqs=16)
    pool2.set_free_order(np.random.default_rng(99).permutation(wl.n_blocks))
    seqs2 = [pool2.seq_new(wl.max_tokens) for _ in range(wl.M)]
    fill_history(pool2, seqs2, wl.history)
    out2 = decode_step(pool2, seqs2, q, k, v, H, G, D, wl.scale, advance=False)
    assert not np.array_equal(pool.seq_pages(seqs[0]), pool2.seq_pages(seqs2[0]))
    assert bits_equal(out2, full)


def test_decode_same_bits_in_both_launch_forms():
    """A batch holding a row of 8192 keys or more (2048-key splits) runs the
    decode kernel's deep form (two pages in flight per wave), a batch
    without one the plain form: a short row gives the same bits either way
    (same arithmetic, page by page), and matches the oracle."""
    H, G, D = 32, 8, 128
    rng = np.random.default_rng(2024)
    lens = [int(x) for x in rng.integers(700, 3000, size=40)] + [9000, 12001]
    hist = [(rng.standard_normal((l, G * D)).astype(np.float32),
             rng.standard_normal((l, G * D)).astype(np.float32)) for l in lens]
    n_blocks = sum(l // 16 + 2 for l in lens) + 8
    pool = pkv.Pool(n_blocks, 16, 1, G, D, max_seqs=64)
    pool.set_free_order(rng.permutation(n_blocks))
    seqs = [pool.seq_new(l + 4) for l in lens]
    fill_history(pool, seqs, lambda r: hist[r])
    M = len(lens)
    q = rng.standard_normal((M, H * D)).astype(np.float32)
    k = rng.standard_normal((M, G * D)).astype(np.float32)
    v = rng.standard_normal((M, G * D)).astype(np.float32)
    scale = float(np.float32(1 / math.sqrt(D)))
    full = decode_step(pool, seqs, q, k, v, H, G, D, scale, advance=False)  # deep
    for r in (0, 1, 20, M - 1):
        nb = pool.decode_workspace_bytes([seqs[r]], H)
        ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
        o1 = torch.empty((1, H * D), device="cuda")
        pool.attn_paged_decode([seqs[r]], 0, H, G, D, dev(q[r:r + 1]), scale, o1, ws=ws,
                               check=True)  # plain for the short rows
        torch.cuda.synchronize()
        assert bits_equal(o1[0], full[r]), r
        rc, ref = oracle.attn_contig(q[r:r + 1], np.concatenate([hist[r][0], k[r:r + 1]]),
                                     np.concatenate([hist[r][1], v[r:r + 1]]), H, G, D,
                                     True, scale)
        assert rc == 0
        assert_close(o1.cpu().numpy(), ref, "row %d" % r)


@pytest.mark.parametrize("ctx", [0, 1, 15, 16, 17, 255, 256, 511, 512, 513, 1023, 1535,
                                 2046, 2047, 2048,
                                 4094, 4095, 4096, 6142, 6143, 6144, 8190, 8191, 8192,
                                 16383])
def test_decode_lengths_around_page_and_split_edges(ctx):
    H, G, D = 32, 8, 128
    rng = np.random.default_rng(ctx)
    kh = rng.standard_normal((ctx, G * D)).astype(np.float32)
    vh = rng.standard_normal((ctx, G * D)).astype(np.float32)
    q = rng.standard_normal((1, H * D)).astype(np.float32)
    k = rng.standard_normal((1, G * D)).astype(np.float32)
    v = rng.standard_normal((1, G * D)).astype(np.float32)
    pool = pkv.Pool(ctx // 16 + 4, 16, 1, G, D, max_seqs=4)
    s = pool.seq_new(ctx + 1)
    fill_history(pool, [s], lambda r: (kh, vh))
    scale = float(np.float32(1 / np.sqrt(D)))
    out = decode_step(pool, [s], q, k, v, H, G, D, scale)
    rc, ref = oracle.attn_contig(q, np.concatenate([kh, k]), np.concatenate([vh, v]),
                                 H, G, D, True, scale)
    assert rc == 0
    assert_close(out.cpu().numpy(), ref, "ctx %d" % ctx)


@pytest.mark.parametrize("H,G,D,B", [
    (8, 8, 128, 16),   # group 1 (fast)
    (16, 8, 128, 16),  # group 2 (fast)
    (64, 8, 128, 16),  # group 8 (fast)
    (12, 4, 64, 16),   # head_dim 64 (generic)
    (32, 8, 128, 8),   # page 8 (generic)
    (6, 2, 42, 5),     # odd sizes (generic, scalar append)
])
def test_decode_other_shapes(H, G, D, B):
    rng = np.random.default_rng(H * 7 + D + B)
    lens = [700, 33, 1]
    pool = pkv.Pool(sum(l // B + 3 for l in lens), B, 2, G, D, max_seqs=8)
    pool.set_free_order(rng.permutation(pool.n_blocks))
    seqs = [pool.seq_new(l + 1) for l in lens]
    hist = [(rng.standard_normal((l, G * D)).astype(np.float32),
             rng.standard_normal((l, G * D)).astype(np.float32)) for l in lens]
    fill_history(pool, seqs, lambda r: hist[r], layer=1)
    q = rng.standard_normal((3, H * D)).astype(np.float32)
    k = rng.standard_normal((3, G * D)).astype(np.float32)
    v = rng.standard_normal((3, G * D)).astype(np.float32)
    pool.ensure_append(seqs, 1, check=True)
    pool.append_layer(seqs, 1, 1, dev(k), dev(v), check=True)
    nb = pool.decode_workspace_bytes(seqs, H)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
    out = torch.full((3, H * D), float("nan"), device="cuda")
    scale = 0.125
    pool.attn_paged_decode(seqs, 1, H, G, D, dev(q), scale, out, ws=ws, check=True)
    torch.cuda.synchronize()
    for r in range(3):
        rc, ref = oracle.attn_contig(q[r:r + 1], np.concatenate([hist[r][0], k[r:r + 1]]),
                                     np.concatenate([hist[r][1], v[r:r + 1]]),
                                     H, G, D, True, scale)
        assert rc == 0
        assert_close(out[r:r + 1].cpu().numpy(), ref, "row %d" % r)


# --------------------------------------------------------------- prefill

@pytest.mark.parametrize("cached,n_q,causal", [
    (0, 1, True), (0, 37, True), (100, 77, True), (45, 32, True),
    (31, 33, True), (300, 5, False), (0, 64, False), (16, 96, True)])
def test_prefill_small_vs_oracle_and_contiguous(cached, n_q, causal):
    H, G, D = 32, 8, 128
    rng = np.random.default_rng(cached * 1000 + n_q)
    M = 2
    lens = [cached, cached + 3]
    hist = [(rng.standard_normal((l, G * D)).astype(np.float32) * 0.5,
             rng.standard_normal((l, G * D)).astype(np.float32) * 0.5) for l in lens]
    pool = pkv.Pool(sum((l + n_q) // 16 + 2 for l in lens), 16, 1, G, D, max_seqs=4)
    pool.set_free_order(rng.permutation(pool.n_blocks))
    seqs = [pool.seq_new(l + n_q) for l in lens]
    fill_history(pool, seqs, lambda r: hist[r])
    Q = (rng.standard_normal((M * n_q, H * D)) * 0.5).astype(np.float32)
    K = (rng.standard_normal((M * n_q, G * D)) * 0.5).astype(np.float32)
    V = (rng.standard_normal((M * n_q, G * D)) * 0.5).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(D)))
    pool.ensure_append(seqs, n_q, check=True)
    pool.append_layer(seqs, n_q, 0, dev(K), dev(V), check=True)
    out = torch.full((M * n_q, H * D), float("nan"), device="cuda")
    pool.attn_paged_prefill(seqs, n_q, 0, H, G, D, dev(Q), causal, scale, out,
                            check=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for r in range(M):
        Kc = np.concatenate([hist[r][0], K[r * n_q:(r + 1) * n_q]])
        Vc = np.concatenate([hist[r][1], V[r * n_q:(r + 1) * n_q]])
        rc, ref = oracle.attn_contig(Q[r * n_q:(r + 1) * n_q], Kc, Vc, H, G, D,
                                     causal, scale)
        assert rc == 0
        assert_close(got[r * n_q:(r + 1) * n_q], ref, "prefill row %d" % r)
    cc = pkv.ContigCache(M, 1, G, max(lens) + n_q, D)
    fill_contig(cc, [0, 1], lambda r: hist[r])
    cc.append([0, 1], lens, n_q, 0, dev(K), dev(V))
    cout = torch.full_like(out, float("nan"))
    cc.attn_prefill([0, 1], lens, n_q, 0, H, dev(Q), causal, scale, cout)
    torch.cuda.synchronize()
    assert bits_equal(out, cout)


def test_prefill_generic_shape_vs_oracle():
    H, G, D, B = 6, 2, 24, 4
    rng = np.random.default_rng(5)
    lens, n_q = [9, 0], 7
    pool = pkv.Pool(16, B, 1, G, D, max_seqs=4)
    seqs = [pool.seq_new(32) for _ in lens]
    hist = [(rng.standard_normal((l, G * D)).astype(np.float32),
             rng.standard_normal((l, G * D)).astype(np.float32)) for l in lens]
    fill_history(pool, seqs, lambda r: hist[r])
    Q = rng.standard_normal((2 * n_q, H * D)).astype(np.float32)
    K = rng.standard_normal((2 * n_q, G * D)).astype(np.float32)
    V = rng.standard_normal((2 * n_q, G * D)).astype(np.float32)
    pool.ensure_append(seqs, n_q, check=True)
    pool.append_layer(seqs, n_q, 0, dev(K), dev(V), check=True)
    out = torch.full((2 * n_q, H * D), float("nan"), device="cuda")
    pool.attn_paged_prefill(seqs, n_q, 0, H, G, D, dev(Q), True, 0.3, out, check=True)
    torch.cuda.synchronize()
    for r in range(2):
        Kc = np.concatenate([hist[r][0], K[r * n_q:(r + 1) * n_q]])
        Vc = np.concatenate([hist[r][1], V[r * n_q:(r + 1) * n_q]])
        rc, ref = oracle.attn_contig(Q[r * n_q:(r + 1) * n_q], Kc, Vc, H, G, D, True, 0.3)
        assert_close(out[r * n_q:(r + 1) * n_q].cpu().numpy(), ref, "row %d" % r)


def test_errors_leave_device_path_untouched():
    pool = pkv.Pool(4, 16, 1, 8, 128, max_seqs=2)
    s = pool.seq_new(64)
    q = torch.zeros((1, 4096), device="cuda")
    out = torch.zeros((1, 4096), device="cuda")
    # rows not ensured/appended
    assert pool.attn_paged_decode([s], 0, 32, 8, 128, q, 0.1, out) == pkv.ERR_SEQ
    assert pool.attn_paged_decode([s], 0, 24, 8, 128, q[:, :3072], 0.1,
                                  out[:, :3072]) == pkv.ERR_SEQ
    assert pool.attn_paged_decode([s], 0, 30, 8, 128, q[:, :3840], 0.1,
                                  out[:, :3840]) == pkv.BAD_GQA
    assert pool.ensure_append([s], 65) == pkv.CAPACITY


@pytest.mark.parametrize("prefix,n_forks", [(37, 5), (16, 3), (5, 4)])
def test_forks_copy_on_append_in_first_step(prefix, n_forks):
    """Forks of a prefix whose last page is partial all append in the same
    step: the first n-1 copy the shared tail, the last keeps it.  Every fork
    must see exactly its own history (regression: the page-table patches of
    the fork and of the copy hit the same entry)."""
    H, G, D = 32, 8, 128
    rng = np.random.default_rng(prefix * 10 + n_forks)
    pk = rng.standard_normal((prefix, G * D)).astype(np.float32)
    pv = rng.standard_normal((prefix, G * D)).astype(np.float32)
    pool = pkv.Pool(64, 16, 1, G, D, max_seqs=n_forks + 2)
    pool.set_free_order(rng.permutation(64))
    parent = pool.seq_new(prefix + 8)
    fill_history(pool, [parent], lambda r: (pk, pv))
    forks = [pool.seq_fork(parent) for _ in range(n_forks)]
    assert pool.seq_free(parent) == 0
    q = rng.standard_normal((n_forks, H * D)).astype(np.float32)
    k = rng.standard_normal((n_forks, G * D)).astype(np.float32)
    v = rng.standard_normal((n_forks, G * D)).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(D)))
    out = decode_step(pool, forks, q, k, v, H, G, D, scale)
    got = out.cpu().numpy()
    for f in range(n_forks):
        rc, ref = oracle.attn_contig(q[f:f + 1], np.concatenate([pk, k[f:f + 1]]),
                                     np.concatenate([pv, v[f:f + 1]]), H, G, D, True,
                                     scale)
        assert rc == 0
        assert_close(got[f:f + 1], ref, "fork %d" % f)
    tails = [pool.seq_pages(s)[prefix // 16] for s in forks]
    if prefix % 16:
        assert len(set(tails)) == n_forks


def test_multilayer_decode_steps_vs_oracle():
    """The step protocol over several layers: ensure once, append + attend
    per layer (each layer with its own K/V and Q), advance once; each layer
    attends over its own rows only."""
    H, G, D, L = 32, 8, 128, 3
    rng = np.random.default_rng(77)
    lens = [600, 1500, 3, 1023]
    M = len(lens)
    pool = pkv.Pool(sum(l // 16 + 4 for l in lens), 16, L, G, D, max_seqs=8)
    pool.set_free_order(rng.permutation(pool.n_blocks))
    seqs = [pool.seq_new(l + 8) for l in lens]
    hist = [[(rng.standard_normal((l, G * D)).astype(np.float32),
              rng.standard_normal((l, G * D)).astype(np.float32)) for l in lens]
            for _ in range(L)]
    for layer in range(L):
        for r, s in enumerate(seqs):
            k, v = hist[layer][r]
            if layer == 0:
                pool.ensure_append([s], lens[r], check=True)
            pool.append_layer([s], lens[r], layer, dev(k), dev(v), check=True)
    pool.advance(seqs, 0, check=False)  # rejected (n <= 0), state unchanged
    for r, s in enumerate(seqs):
        pool.advance([s], lens[r], check=True)
    scale = float(np.float32(1 / np.sqrt(D)))
    for step in range(3):
        pool.ensure_append(seqs, 1, check=True)
        ws = torch.empty(max(pool.decode_workspace_bytes(seqs, H), 4),
                         dtype=torch.uint8, device="cuda")
        for layer in range(L):
            q = rng.standard_normal((M, H * D)).astype(np.float32)
            k = rng.standard_normal((M, G * D)).astype(np.float32)
            v = rng.standard_normal((M, G * D)).astype(np.float32)
            pool.append_layer(seqs, 1, layer, dev(k), dev(v), check=True)
            out = torch.full((M, H * D), float("nan"), device="cuda")
            pool.attn_paged_decode(seqs, layer, H, G, D, dev(q), scale, out, ws=ws,
                                   check=True)
            torch.cuda.synchronize()
            got = out.cpu().numpy()
            for r in range(M):
                kh, vh = hist[layer][r]
                kh = np.concatenate([kh, k[r:r + 1]])
                vh = np.concatenate([vh, v[r:r + 1]])
                hist[layer][r] = (kh, vh)
                rc, ref = oracle.attn_contig(q[r:r + 1], kh, vh, H, G, D, True, scale)
                assert rc == 0
                assert_close(got[r:r + 1], ref, "step %d layer %d row %d" % (step, layer, r))
        pool.advance(seqs, 1, check=True)


def test_page_table_mirror_grows_after_first_use():
    """A sequence created after device work has started may need a longer
    page table than any before it; the mirror is rebuilt and every earlier
    sequence keeps reading its own rows."""
    H, G, D = 32, 8, 128
    rng = np.random.default_rng(78)
    pool = pkv.Pool(400, 16, 1, G, D, max_seqs=4)
    pool.set_free_order(rng.permutation(400))
    a = pool.seq_new(40)
    ha = (rng.standard_normal((33, G * D)).astype(np.float32),
          rng.standard_normal((33, G * D)).astype(np.float32))
    fill_history(pool, [a], lambda r: ha)
    b = pool.seq_new(5000)  # far longer page table than a's
    hb = (rng.standard_normal((4100, G * D)).astype(np.float32),
          rng.standard_normal((4100, G * D)).astype(np.float32))
    fill_history(pool, [b], lambda r: hb)
    q = rng.standard_normal((2, H * D)).astype(np.float32)
    k = rng.standard_normal((2, G * D)).astype(np.float32)
    v = rng.standard_normal((2, G * D)).astype(np.float32)
    scale = 0.09
    out = decode_step(pool, [a, b], q, k, v, H, G, D, scale)
    got = out.cpu().numpy()
    for r, h in enumerate((ha, hb)):
        rc, ref = oracle.attn_contig(q[r:r + 1], np.concatenate([h[0], k[r:r + 1]]),
                                     np.concatenate([h[1], v[r:r + 1]]), H, G, D, True,
                                     scale)
        assert_close(got[r:r + 1], ref, "row %d" % r)


@pytest.mark.parametrize("H,cached,n_q,causal", [
    (8, 45, 130, True),     # group 1: 128 queries per workgroup, ragged second tile
    (8, 0, 20, False),
    (16, 300, 70, True),    # group 2: 64 per workgroup
    (64, 17, 37, True),     # group 8: 16 per workgroup, three tiles
    (64, 100, 16, False),
])
def test_prefill_mfma_other_groups_vs_oracle_and_contiguous(H, cached, n_q, causal):
    G, D = 8, 128
    rng = np.random.default_rng(H * 100 + n_q)
    lens = [cached, cached + 5]
    M = 2
    hist = [(rng.standard_normal((l, G * D)).astype(np.float32) * 0.5,
             rng.standard_normal((l, G * D)).astype(np.float32) * 0.5) for l in lens]
    pool = pkv.Pool(sum((l + n_q) // 16 + 2 for l in lens), 16, 1, G, D, max_seqs=4)
    pool.set_free_order(rng.permutation(pool.n_blocks))
    seqs = [pool.seq_new(l + n_q) for l in lens]
    fill_history(pool, seqs, lambda r: hist[r])
    Q = (rng.standard_normal((M * n_q, H * D)) * 0.5).astype(np.float32)
    K = (rng.standard_normal((M * n_q, G * D)) * 0.5).astype(np.float32)
    V = (rng.standard_normal((M * n_q, G * D)) * 0.5).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(D)))
    pool.ensure_append(seqs, n_q, check=True)
    pool.append_layer(seqs, n_q, 0, dev(K), dev(V), check=True)
    out = torch.full((M * n_q, H * D), float("nan"), device="cuda")
    pool.attn_paged_prefill(seqs, n_q, 0, H, G, D, dev(Q), causal, scale, out,
                            check=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for r in range(M):
        Kc = np.concatenate([hist[r][0], K[r * n_q:(r + 1) * n_q]])
        Vc = np.concatenate([hist[r][1], V[r * n_q:(r + 1) * n_q]])
        rc, ref = oracle.attn_contig(Q[r * n_q:(r + 1) * n_q], Kc, Vc, H, G, D,
                                     causal, scale)
        assert rc == 0
        assert_close(got[r * n_q:(r + 1) * n_q], ref, "group %d row %d" % (H // G, r))
    cc = pkv.ContigCache(M, 1, G, max(lens) + n_q, D)
    fill_contig(cc, [0, 1], lambda r: hist[r])
    cc.append([0, 1], lens, n_q, 0, dev(K), dev(V))
    cout = torch.full_like(out, float("nan"))
    cc.attn_prefill([0, 1], lens, n_q, 0, H, dev(Q), causal, scale, cout)
    torch.cuda.synchronize()
    assert bits_equal(out, cout)


def test_kernel_forms_recorded():
    """pkv_profile_kernel_name names the template instance each kernel id
    launched last (the bench's roofline entry reads it)."""
    wl = synth.decode_m32(max_steps=2)
    pool, seqs = decode_pool(wl)
    assert pool.kernel_name(pkv.K_DECODE) == ""
    q, k, v = wl.step(0)
    decode_step(pool, seqs, q, k, v, wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.scale)
    assert pool.kernel_name(pkv.K_DECODE) == "decode_fast_kernel<4, PagedMap, false>"
    assert pool.kernel_name(pkv.K_MERGE) == "merge_kernel"
    # the 32-row blob fits the append kernel's arguments
    assert pool.kernel_name(pkv.K_APPEND) == "append_inline_kernel<4, false>"
    pool.close()


def test_mirror_growth_then_multirow_append():
    """A sequence created after earlier device calls with a longer max_tokens
    makes the next call grow (reallocate) the page-table mirror; the
    multi-row append of that call must address pages through the new mirror.
    Outputs of both sequences against the oracle."""
    H, G, D, B = 32, 8, 128, 16
    rng = np.random.default_rng(91)
    pool = pkv.Pool(400, B, 1, G, D, max_seqs=4)
    scale = float(np.float32(1 / np.sqrt(D)))
    s0 = pool.seq_new(40)
    k0 = rng.standard_normal((20, G * D)).astype(np.float32)
    v0 = rng.standard_normal((20, G * D)).astype(np.float32)
    pool.ensure_append([s0], 20, check=True)
    pool.append_layer([s0], 20, 0, dev(k0), dev(v0), check=True)
    pool.advance([s0], 20, check=True)
    s1 = pool.seq_new(5000)  # 313 pages: the mirror's stride grows
    k1 = rng.standard_normal((700, G * D)).astype(np.float32)
    v1 = rng.standard_normal((700, G * D)).astype(np.float32)
    pool.ensure_append([s1], 700, check=True)
    pool.append_layer([s1], 700, 0, dev(k1), dev(v1), check=True)
    pool.advance([s1], 700, check=True)
    q = rng.standard_normal((2, H * D)).astype(np.float32)
    k = rng.standard_normal((2, G * D)).astype(np.float32)
    v = rng.standard_normal((2, G * D)).astype(np.float32)
    out = decode_step(pool, [s0, s1], q, k, v, H, G, D, scale).cpu().numpy()
    for r, (hk, hv) in enumerate(((k0, v0), (k1, v1))):
        rc, ref = oracle.attn_contig(q[r:r + 1], np.concatenate([hk, k[r:r + 1]]),
                                     np.concatenate([hv, v[r:r + 1]]), H, G, D, True, scale)
        assert rc == 0
        assert_close(out[r:r + 1], ref, "row %d" % r)
    pool.close()


def test_one_row_append_staged_blob_matches_oracle():
    """A batch whose row blob is too large for the append kernel's arguments
    (200 sequences: 1600 ints of row descriptors) takes the staged one-row
    append; two steps of it against the oracle."""
    H, G, D, B = 32, 8, 128, 16
    rng = np.random.default_rng(77)
    lens = rng.integers(1, 40, size=200)
    pool = pkv.Pool(int(sum((l + 2) // B + 2 for l in lens)) + 8, B, 1, G, D, max_seqs=208)
    seqs = [pool.seq_new(64) for _ in lens]
    hist = []
    for s_, l in zip(seqs, lens):
        k = rng.standard_normal((l, G * D)).astype(np.float32)
        v = rng.standard_normal((l, G * D)).astype(np.float32)
        pool.ensure_append([s_], int(l), check=True)
        pool.append_layer([s_], int(l), 0, dev(k), dev(v), check=True)
        pool.advance([s_], int(l), check=True)
        hist.append((k, v))
    scale = float(np.float32(1 / np.sqrt(D)))
    for step in range(2):
        q = rng.standard_normal((len(seqs), H * D)).astype(np.float32)
        k = rng.standard_normal((len(seqs), G * D)).astype(np.float32)
        v = rng.standard_normal((len(seqs), G * D)).astype(np.float32)
        out = decode_step(pool, seqs, q, k, v, H, G, D, scale).cpu().numpy()
        assert pool.kernel_name(pkv.K_APPEND) == "append_kernel<4, PagedMap, false, true>"
        for r in range(0, len(seqs), 7):
            hk = np.concatenate([hist[r][0], k[r:r + 1]])
            hv = np.concatenate([hist[r][1], v[r:r + 1]])
            rc, ref = oracle.attn_contig(q[r:r + 1], hk, hv, H, G, D, True, scale)
            assert rc == 0
            assert_close(out[r:r + 1], ref, "step %d row %d" % (step, r))
            hist[r] = (hk, hv)
        for r in range(len(seqs)):
            if r % 7:
                hist[r] = (np.concatenate([hist[r][0], k[r:r + 1]]),
                           np.concatenate([hist[r][1], v[r:r + 1]]))
    pool.close()

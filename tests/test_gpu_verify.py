"""GPU parity of multi-query decode (pkv_attn_paged_verify): n_q new rows per
sequence, offset-causal, key-split with a fixed merge order -- the
speculative-decode verify step ("nx_paged_kv_gate.nx source": header,
"truncate unref" as the rewind after rejected drafts; the attention is the
prefill's, "nx_f32_attn_paged.nx source" header comment).

Bars: outputs within 1e-4 + 1e-4 * |oracle|; paged == contiguous bit for
bit; n_q == 1 equals pkv_attn_paged_decode bit for bit; a row's output does
not depend on the rest of the batch; pool state after append / verify /
accept / truncate cycles equals the oracle pool's bit for bit.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_layer_amd as pkv
import synth
from pkv_gpu import assert_close, bits_equal, decode_pool, dev, fill_contig, fill_history

pytestmark = pytest.mark.gpu


def _verify(pool, seqs, n_q, Q, K, V, H, G, D, scale, layer=0, append=True):
    M = len(seqs)
    if append:
        pool.ensure_append(seqs, n_q, check=True)
        pool.append_layer(seqs, n_q, layer, dev(K), dev(V), check=True)
    nb = pool.verify_workspace_bytes(seqs, n_q, H)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
    out = torch.full((M * n_q, H * D), float("nan"), device="cuda")
    pool.attn_paged_verify(seqs, n_q, layer, H, G, D, dev(Q), scale, out, ws=ws,
                           check=True)
    torch.cuda.synchronize()
    return out


def _rand(rng, shape, sigma=1.0):
    return (rng.standard_normal(shape) * sigma).astype(np.float32)


@pytest.mark.parametrize("H,G,n_q", [
    (32, 8, 2), (32, 8, 3), (32, 8, 4), (32, 8, 5), (32, 8, 8),  # group 4
    (8, 8, 8),     # group 1: 8 rows
    (16, 8, 8),    # group 2: 16 rows, one MFMA block
    (64, 8, 4),    # group 8: 32 rows, two blocks
    (64, 8, 5),    # 40 rows: runs the prefill kernels
    # groups the decode kernel does not take but the split multi-query kernel
    # does (n_q x group <= 32): group 3 and group 16
    (24, 8, 1), (24, 8, 2), (24, 8, 5), (24, 8, 8), (24, 8, 10),
    (24, 8, 11),   # 33 rows: the generic kernel
    (32, 2, 1), (32, 2, 2),
    (32, 2, 3),    # 48 rows: the generic kernel
])
def test_verify_vs_oracle_and_contiguous(H, G, n_q):
    D = 128
    rng = np.random.default_rng(H * 10 + n_q)
    # around the 512-key split edge: with n_q new rows the early queries of a
    # row may see none of the last split
    lens = [0, 1, 13, 509, 510, 511, 512, 1020, 2000]
    M = len(lens)
    pool = pkv.Pool(sum((l + n_q) // 16 + 2 for l in lens), 16, 1, G, D, max_seqs=16)
    pool.set_free_order(rng.permutation(pool.n_blocks))
    seqs = [pool.seq_new(l + n_q) for l in lens]
    hist = [(_rand(rng, (l, G * D)), _rand(rng, (l, G * D))) for l in lens]
    fill_history(pool, seqs, lambda r: hist[r])
    Q = _rand(rng, (M * n_q, H * D))
    K = _rand(rng, (M * n_q, G * D))
    V = _rand(rng, (M * n_q, G * D))
    scale = float(np.float32(1 / math.sqrt(D)))
    out = _verify(pool, seqs, n_q, Q, K, V, H, G, D, scale)
    got = out.cpu().numpy()
    for r in range(M):
        rows = slice(r * n_q, (r + 1) * n_q)
        rc, ref = oracle.attn_contig(Q[rows], np.concatenate([hist[r][0], K[rows]]),
                                     np.concatenate([hist[r][1], V[rows]]),
                                     H, G, D, True, scale)
        assert rc == 0
        assert_close(got[rows], ref, "verify n_q=%d row %d (len %d)" % (n_q, r, lens[r]))
    cc = pkv.ContigCache(M, 1, G, max(lens) + n_q, D)
    fill_contig(cc, list(range(M)), lambda r: hist[r])
    cc.append(list(range(M)), lens, n_q, 0, dev(K), dev(V))
    ws = torch.empty(max(cc.verify_workspace_bytes(lens, n_q, H), 4),
                     dtype=torch.uint8, device="cuda")
    cout = torch.full_like(out, float("nan"))
    cc.attn_verify(list(range(M)), lens, n_q, 0, H, dev(Q), scale, cout, ws=ws)
    torch.cuda.synchronize()
    assert bits_equal(out, cout)


def test_verify_one_query_is_decode_and_rows_are_batch_independent():
    H, G, D = 32, 8, 128
    rng = np.random.default_rng(7)
    lens = [600, 3, 1536, 40]
    pool = pkv.Pool(sum(l // 16 + 3 for l in lens), 16, 1, G, D, max_seqs=8)
    seqs = [pool.seq_new(l + 8) for l in lens]
    hist = [(_rand(rng, (l, G * D)), _rand(rng, (l, G * D))) for l in lens]
    fill_history(pool, seqs, lambda r: hist[r])
    q = _rand(rng, (4, H * D))
    k = _rand(rng, (4, G * D))
    v = _rand(rng, (4, G * D))
    scale = 0.0883883
    ov = _verify(pool, seqs, 1, q, k, v, H, G, D, scale)
    nb = pool.decode_workspace_bytes(seqs, H)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
    od = torch.empty_like(ov)
    pool.attn_paged_decode(seqs, 0, H, G, D, dev(q), scale, od, ws=ws, check=True)
    torch.cuda.synchronize()
    assert bits_equal(ov, od)
    pool.advance(seqs, 1, check=True)
    # four queries: each row alone equals its row in the batch
    n_q = 4
    Q = _rand(rng, (4 * n_q, H * D))
    K = _rand(rng, (4 * n_q, G * D))
    V = _rand(rng, (4 * n_q, G * D))
    full = _verify(pool, seqs, n_q, Q, K, V, H, G, D, scale)
    for r in range(4):
        rows = slice(r * n_q, (r + 1) * n_q)
        one = _verify(pool, [seqs[r]], n_q, Q[rows], None, None, H, G, D, scale,
                      append=False)
        assert bits_equal(one, full[rows])
    # and the prefill kernels agree within the tolerance
    out = torch.empty_like(full)
    pool.attn_paged_prefill(seqs, n_q, 0, H, G, D, dev(Q), True, scale, out,
                            check=True)
    torch.cuda.synchronize()
    assert_close(full.cpu().numpy(), out.cpu().numpy(), "verify vs prefill")


def _ostate(op, seqs):
    return (op.refcounts().tolist(), op.free_stack().tolist(),
            [(op.seq_len(s), None if op.seq_pages(s) is None else op.seq_pages(s).tolist())
             for s in seqs])


def test_speculative_cycles_with_rewind_match_oracle():
    """Draft n_q tokens per sequence, verify them in one call, accept a seeded
    number, rewind the rest with truncate; repeat.  M=32 sequences with
    512..4096 cached rows and random placement."""
    wl = synth.decode_m32(max_steps=40)
    H, G, D, M = wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.M
    pool, seqs = decode_pool(wl)
    opool = oracle.Pool(wl.n_blocks, wl.block_size, 1, G, D, max_seqs=M + 8,
                        with_storage=False)
    opool.set_free_order(wl.free_order())
    oseqs = [opool.seq_new(wl.max_tokens) for _ in range(M)]
    for r, s in enumerate(oseqs):
        assert opool.ensure_append([s], int(wl.ctx[r])) == 0
        assert opool.advance([s], int(wl.ctx[r])) == 0
    assert seqs == oseqs
    assert _ostate(opool, oseqs) == _ostate(pool, seqs)
    rng = np.random.default_rng(123)
    Ks = [list(wl.history(r)[0]) for r in range(M)]
    Vs = [list(wl.history(r)[1]) for r in range(M)]
    n_q = 4
    for cycle in range(3):
        Q = _rand(rng, (M * n_q, H * D))
        K = _rand(rng, (M * n_q, G * D))
        V = _rand(rng, (M * n_q, G * D))
        out = _verify(pool, seqs, n_q, Q, K, V, H, G, D, wl.scale)
        assert opool.ensure_append(oseqs, n_q) == 0
        assert opool.append_layer(oseqs, n_q, 0, K, V) == 0
        got = out.cpu().numpy()
        for r in range(M):
            rows = slice(r * n_q, (r + 1) * n_q)
            Kc = np.concatenate([np.stack(Ks[r]), K[rows]])
            Vc = np.concatenate([np.stack(Vs[r]), V[rows]])
            rc, ref = oracle.attn_contig(Q[rows], Kc, Vc, H, G, D, True, wl.scale)
            assert rc == 0
            assert_close(got[rows], ref, "cycle %d row %d" % (cycle, r))
        # accept 1..n_q drafts per sequence, rewind the others
        acc = rng.integers(1, n_q + 1, size=M)
        pool.advance(seqs, n_q, check=True)
        assert opool.advance(oseqs, n_q) == 0
        for r in range(M):
            new_len = pool.seq_len(seqs[r]) - n_q + int(acc[r])
            pool.seq_truncate(seqs[r], new_len, check=True)
            assert opool.seq_truncate(oseqs[r], new_len) == 0
            Ks[r].extend(K[r * n_q:r * n_q + int(acc[r])])
            Vs[r].extend(V[r * n_q:r * n_q + int(acc[r])])
        assert _ostate(pool, seqs) == _ostate(opool, oseqs)


def test_verify_on_forks_copies_on_append_and_rewinds():
    """Forks of a 37-row prefix verify 3 drafts each: the shared partial page
    is copied before the append, the truncate releases what the rejected
    drafts took, and state follows the oracle pool bit for bit."""
    H, G, D, B = 32, 8, 128, 16
    rng = np.random.default_rng(9)
    pool = pkv.Pool(64, B, 1, G, D, max_seqs=8)
    opool = oracle.Pool(64, B, 1, G, D, max_seqs=8, with_storage=False)
    base = pool.seq_new(128)
    assert opool.seq_new(128) == base
    pk, pv = _rand(rng, (37, G * D)), _rand(rng, (37, G * D))
    fill_history(pool, [base], lambda r: (pk, pv))
    assert opool.ensure_append([base], 37) == 0 and opool.advance([base], 37) == 0
    forks = [pool.seq_fork(base) for _ in range(3)]
    assert [opool.seq_fork(base) for _ in range(3)] == forks
    Ks = {f: list(pk) for f in forks}
    Vs = {f: list(pv) for f in forks}
    n_q, scale = 3, 0.0883883
    for cycle in range(3):
        Q = _rand(rng, (3 * n_q, H * D))
        K = _rand(rng, (3 * n_q, G * D))
        V = _rand(rng, (3 * n_q, G * D))
        out = _verify(pool, forks, n_q, Q, K, V, H, G, D, scale)
        assert opool.ensure_append(forks, n_q) == 0
        got = out.cpu().numpy()
        for i, f in enumerate(forks):
            rows = slice(i * n_q, (i + 1) * n_q)
            rc, ref = oracle.attn_contig(Q[rows], np.concatenate([np.stack(Ks[f]), K[rows]]),
                                         np.concatenate([np.stack(Vs[f]), V[rows]]),
                                         H, G, D, True, scale)
            assert rc == 0
            assert_close(got[rows], ref, "fork %d cycle %d" % (i, cycle))
        pool.advance(forks, n_q, check=True)
        assert opool.advance(forks, n_q) == 0
        for i, f in enumerate(forks):
            a = 1 + (i + cycle) % n_q
            new_len = pool.seq_len(f) - n_q + a
            pool.seq_truncate(f, new_len, check=True)
            assert opool.seq_truncate(f, new_len) == 0
            Ks[f].extend(K[i * n_q:i * n_q + a])
            Vs[f].extend(V[i * n_q:i * n_q + a])
        assert _ostate(pool, [base] + forks) == _ostate(opool, [base] + forks)


def test_verify_errors():
    H, G, D = 32, 8, 128
    pool = pkv.Pool(48, 16, 1, G, D, max_seqs=2)
    s = pool.seq_new(64)
    q = torch.zeros((4, H * D), device="cuda")
    out = torch.zeros_like(q)
    L = pkv.lib()
    import ctypes as C
    a = np.array([s], np.int32)
    ap = a.ctypes.data_as(C.c_void_p)
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    qp, op = C.c_void_p(q.data_ptr()), C.c_void_p(out.data_ptr())
    assert L.pkv_attn_paged_verify(pool._h, ap, 1, 0, 0, H, G, D, qp, 0.1, op, None,
                                   0, st) == pkv.BAD_DIM
    assert L.pkv_attn_paged_verify(pool._h, ap, 1, 4, 0, 30, G, D, qp, 0.1, op, None,
                                   0, st) == pkv.BAD_GQA
    # rows not ensured
    assert L.pkv_attn_paged_verify(pool._h, ap, 1, 4, 0, H, G, D, qp, 0.1, op, None,
                                   0, st) == pkv.ERR_SEQ
    pool.ensure_append([s], 4, check=True)
    # 4 rows of a 4-key sequence fit one split: no workspace needed
    assert pool.verify_workspace_bytes([s], 4, H) == 0
    assert L.pkv_attn_paged_verify(pool._h, ap, 1, 4, 0, H, G, D, qp, 0.1, op, None,
                                   0, st) == pkv.OK
    kv = torch.zeros((600, G * D), device="cuda")
    pool.append_layer([s], 4, 0, kv[:4], kv[:4], check=True)
    pool.advance([s], 4, check=True)
    s2 = pool.seq_new(700)
    pool.ensure_append([s2], 600, check=True)
    pool.append_layer([s2], 600, 0, kv, kv, check=True)
    pool.advance([s2], 600, check=True)
    pool.ensure_append([s2], 4, check=True)
    need = pool.verify_workspace_bytes([s2], 4, H)
    # 604 own keys in 256-key splits (rows below 2048 keys): 3 partial slots
    assert need == 3 * 4 * H * (D + 2) * 4
    a2 = np.array([s2], np.int32)
    small = torch.empty(need - 4, dtype=torch.uint8, device="cuda")
    assert L.pkv_attn_paged_verify(pool._h, a2.ctypes.data_as(C.c_void_p), 1, 4, 0, H,
                                   G, D, qp, 0.1, op, C.c_void_p(small.data_ptr()),
                                   need - 4, st) == pkv.BAD_ARG
    torch.cuda.synchronize()

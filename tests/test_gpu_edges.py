"""GPU parity at the edges of the size range: one very long sequence (33
splits of 2048 keys) beside a short one in decode, verify and prefill; a
single-sequence batch; a 1024-sequence batch of short contexts.  Outputs are
checked against the oracle (sampled where the oracle would be slow) at
1e-4 + 1e-4 * |oracle|, and against the contiguous twin bit for bit."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_layer_amd as pkv
from pkv_gpu import assert_close, bits_equal, dev, fill_contig, fill_history

pytestmark = pytest.mark.gpu

H, G, D, B = 32, 8, 128, 16
SCALE = float(np.float32(1 / math.sqrt(D)))


def _rand(rng, shape, sigma=1.0):
    a = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def test_very_long_sequence_decode_verify_prefill():
    rng = np.random.default_rng(65536)
    lens = [65536, 7]
    extra = 64
    pool = pkv.Pool(sum((l + 2 * extra) // B + 4 for l in lens), B, 1, G, D, max_seqs=4)
    pool.set_free_order(rng.permutation(pool.n_blocks))
    seqs = [pool.seq_new(l + 2 * extra) for l in lens]
    hist = [(_rand(rng, (l, G * D)), _rand(rng, (l, G * D))) for l in lens]
    fill_history(pool, seqs, lambda r: hist[r])
    Ks = [h[0] for h in hist]
    Vs = [h[1] for h in hist]

    def keys(r, new_k, new_v):
        return np.concatenate([Ks[r], new_k]), np.concatenate([Vs[r], new_v])

    # decode
    q = _rand(rng, (2, H * D))
    k = _rand(rng, (2, G * D))
    v = _rand(rng, (2, G * D))
    pool.ensure_append(seqs, 1, check=True)
    pool.append_layer(seqs, 1, 0, dev(k), dev(v), check=True)
    ws = torch.empty(pool.decode_workspace_bytes(seqs, H), dtype=torch.uint8, device="cuda")
    out = torch.full((2, H * D), float("nan"), device="cuda")
    pool.attn_paged_decode(seqs, 0, H, G, D, dev(q), SCALE, out, ws=ws, check=True)
    torch.cuda.synchronize()
    for r in range(2):
        kk, vv = keys(r, k[r:r + 1], v[r:r + 1])
        rc, ref = oracle.attn_contig(q[r:r + 1], kk, vv, H, G, D, True, SCALE)
        assert rc == 0
        assert_close(out[r:r + 1].cpu().numpy(), ref, "long decode row %d" % r)
    pool.advance(seqs, 1, check=True)
    for r in range(2):
        Ks[r] = np.concatenate([Ks[r], k[r:r + 1]])
        Vs[r] = np.concatenate([Vs[r], v[r:r + 1]])

    # verify, four drafted rows
    n_q = 4
    Q = _rand(rng, (2 * n_q, H * D))
    K = _rand(rng, (2 * n_q, G * D))
    V = _rand(rng, (2 * n_q, G * D))
    pool.ensure_append(seqs, n_q, check=True)
    pool.append_layer(seqs, n_q, 0, dev(K), dev(V), check=True)
    ws = torch.empty(pool.verify_workspace_bytes(seqs, n_q, H), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((2 * n_q, H * D), float("nan"), device="cuda")
    pool.attn_paged_verify(seqs, n_q, 0, H, G, D, dev(Q), SCALE, out, ws=ws, check=True)
    torch.cuda.synchronize()
    for r in range(2):
        rows = slice(r * n_q, (r + 1) * n_q)
        kk, vv = keys(r, K[rows], V[rows])
        rc, ref = oracle.attn_contig(Q[rows], kk, vv, H, G, D, True, SCALE)
        assert rc == 0
        assert_close(out[rows].cpu().numpy(), ref, "long verify row %d" % r)
    # accept the drafts, then reject them all again: rewind to before them
    pool.advance(seqs, n_q, check=True)
    for s in seqs:
        pool.seq_truncate(s, pool.seq_len(s) - n_q, check=True)

    # prefill chunk of 40 rows; sampled queries against truncated key sets
    n_q = 40
    Q = _rand(rng, (2 * n_q, H * D), 0.5)
    K = _rand(rng, (2 * n_q, G * D), 0.5)
    V = _rand(rng, (2 * n_q, G * D), 0.5)
    pool.ensure_append(seqs, n_q, check=True)
    pool.append_layer(seqs, n_q, 0, dev(K), dev(V), check=True)
    out = torch.full((2 * n_q, H * D), float("nan"), device="cuda")
    pool.attn_paged_prefill(seqs, n_q, 0, H, G, D, dev(Q), True, SCALE, out, check=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for r in range(2):
        kk, vv = keys(r, K[r * n_q:(r + 1) * n_q], V[r * n_q:(r + 1) * n_q])
        L = len(Ks[r])
        for i in (0, 17, n_q - 1):
            row = r * n_q + i
            rc, ref = oracle.attn_contig(Q[row:row + 1], kk[:L + i + 1], vv[:L + i + 1],
                                         H, G, D, True, SCALE)
            assert rc == 0
            assert_close(got[row:row + 1], ref, "long prefill row %d query %d" % (r, i))
    pool.close()


def test_single_sequence_batch():
    rng = np.random.default_rng(1)
    L = 3000
    pool = pkv.Pool(L // B + 4, B, 1, G, D, max_seqs=1)
    s = pool.seq_new(L + 1)
    kh, vh = _rand(rng, (L, G * D)), _rand(rng, (L, G * D))
    fill_history(pool, [s], lambda r: (kh, vh))
    q, k, v = _rand(rng, (1, H * D)), _rand(rng, (1, G * D)), _rand(rng, (1, G * D))
    pool.ensure_append([s], 1, check=True)
    pool.append_layer([s], 1, 0, dev(k), dev(v), check=True)
    ws = torch.empty(pool.decode_workspace_bytes([s], H), dtype=torch.uint8, device="cuda")
    out = torch.full((1, H * D), float("nan"), device="cuda")
    pool.attn_paged_decode([s], 0, H, G, D, dev(q), SCALE, out, ws=ws, check=True)
    torch.cuda.synchronize()
    rc, ref = oracle.attn_contig(q, np.concatenate([kh, k]), np.concatenate([vh, v]),
                                 H, G, D, True, SCALE)
    assert_close(out.cpu().numpy(), ref, "single")
    # the one sequence may use the last free sequence id and every block
    assert pool.seq_new(8) == -pkv.CAPACITY


def test_large_batch_of_short_contexts():
    rng = np.random.default_rng(2)
    M = 1024
    lens = rng.integers(0, 64, size=M)
    pool = pkv.Pool(int(sum(l // B + 2 for l in lens)), B, 1, G, D, max_seqs=M)
    pool.set_free_order(rng.permutation(pool.n_blocks))
    seqs = [pool.seq_new(int(l) + 1) for l in lens]
    hist = [(_rand(rng, (int(l), G * D)), _rand(rng, (int(l), G * D))) for l in lens]
    # one batched append per distinct length keeps the fill quick
    for n in sorted(set(int(l) for l in lens) - {0}):
        rows = [r for r in range(M) if lens[r] == n]
        kk = np.concatenate([hist[r][0] for r in rows])
        vv = np.concatenate([hist[r][1] for r in rows])
        sq = [seqs[r] for r in rows]
        pool.ensure_append(sq, n, check=True)
        pool.append_layer(sq, n, 0, dev(kk), dev(vv), check=True)
        pool.advance(sq, n, check=True)
    q, k, v = _rand(rng, (M, H * D)), _rand(rng, (M, G * D)), _rand(rng, (M, G * D))
    pool.ensure_append(seqs, 1, check=True)
    pool.append_layer(seqs, 1, 0, dev(k), dev(v), check=True)
    nb = pool.decode_workspace_bytes(seqs, H)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
    out = torch.full((M, H * D), float("nan"), device="cuda")
    pool.attn_paged_decode(seqs, 0, H, G, D, dev(q), SCALE, out, ws=ws, check=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for r in list(range(0, M, 37)) + [M - 1]:
        rc, ref = oracle.attn_contig(q[r:r + 1], np.concatenate([hist[r][0], k[r:r + 1]]),
                                     np.concatenate([hist[r][1], v[r:r + 1]]), H, G, D,
                                     True, SCALE)
        assert_close(got[r:r + 1], ref, "row %d (len %d)" % (r, lens[r]))
    cc = pkv.ContigCache(M, 1, G, 64 + 1, D)
    fill_contig(cc, list(range(M)), lambda r: hist[r])
    cc.append(list(range(M)), [int(l) for l in lens], 1, 0, dev(k), dev(v))
    cws = torch.empty(max(cc.decode_workspace_bytes([int(l) for l in lens], H), 4),
                      dtype=torch.uint8, device="cuda")
    cout = torch.full_like(out, float("nan"))
    cc.attn_decode(list(range(M)), [int(l) for l in lens], 0, H, dev(q), SCALE, cout,
                   ws=cws)
    torch.cuda.synchronize()
    assert bits_equal(out, cout)


def test_group_16_generic_path_and_unsupported_shapes():
    """Group 16 (beyond the fast kernels' 1/2/4/8) runs the generic kernel for
    decode and prefill and matches the oracle; group 17, or a group whose q
    and o vectors do not fit the generic kernel's LDS, is refused with
    UNSUPPORTED and leaves the output untouched."""
    rng = np.random.default_rng(16)
    Gk, Dk, Bk = 1, 64, 16
    pool = pkv.Pool(64, Bk, 1, Gk, Dk, max_seqs=4)
    pool.set_free_order(rng.permutation(pool.n_blocks))
    seqs = [pool.seq_new(300), pool.seq_new(300)]
    hist = [(_rand(rng, (n, Gk * Dk)), _rand(rng, (n, Gk * Dk))) for n in (131, 40)]
    fill_history(pool, seqs, lambda r: hist[r])
    scale = float(np.float32(1 / math.sqrt(Dk)))
    for n_q, Hk in ((1, 16), (5, 16)):
        Q = _rand(rng, (2 * n_q, Hk * Dk))
        K = _rand(rng, (2 * n_q, Gk * Dk))
        V = _rand(rng, (2 * n_q, Gk * Dk))
        pool.ensure_append(seqs, n_q, check=True)
        pool.append_layer(seqs, n_q, 0, dev(K), dev(V), check=True)
        out = torch.full((2 * n_q, Hk * Dk), float("nan"), device="cuda")
        if n_q == 1:
            pool.attn_paged_decode(seqs, 0, Hk, Gk, Dk, dev(Q), scale, out, check=True)
        else:
            pool.attn_paged_prefill(seqs, n_q, 0, Hk, Gk, Dk, dev(Q), True, scale, out,
                                    check=True)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        for r in range(2):
            rows = slice(r * n_q, (r + 1) * n_q)
            kk = np.concatenate([hist[r][0], K[rows]])
            vv = np.concatenate([hist[r][1], V[rows]])
            rc, ref = oracle.attn_contig(Q[rows], kk, vv, Hk, Gk, Dk, True, scale)
            assert rc == 0
            assert_close(got[rows], ref, "group 16 n_q %d row %d" % (n_q, r))
        pool.advance(seqs, n_q, check=True)
        hist = [(np.concatenate([hist[r][0], K[r * n_q:(r + 1) * n_q]]),
                 np.concatenate([hist[r][1], V[r * n_q:(r + 1) * n_q]])) for r in range(2)]
    # group 17
    pool.ensure_append(seqs, 1, check=True)
    pool.append_layer(seqs, 1, 0, dev(_rand(rng, (2, Dk))), dev(_rand(rng, (2, Dk))),
                      check=True)
    out = torch.full((2, 17 * Dk), 7.0, device="cuda")
    q = dev(_rand(rng, (2, 17 * Dk)))
    assert pool.attn_paged_decode(seqs, 0, 17, Gk, Dk, q, scale, out) == pkv.UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    pool.close()
    # group 16 at head_dim 600: q and o of the group exceed the generic LDS budget
    Dl = 600
    big = pkv.Pool(8, Bk, 1, Gk, Dl, max_seqs=2)
    s = big.seq_new(32)
    big.ensure_append([s], 1, check=True)
    big.append_layer([s], 1, 0, dev(_rand(rng, (1, Dl))), dev(_rand(rng, (1, Dl))),
                     check=True)
    out = torch.full((1, 16 * Dl), 7.0, device="cuda")
    q = dev(_rand(rng, (1, 16 * Dl)))
    assert big.attn_paged_decode([s], 0, 16, Gk, Dl, q, 0.04, out) == pkv.UNSUPPORTED
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    big.close()


def test_profile_kernel_mask():
    """pkv_profile_kernels limits which launches are timed."""
    rng = np.random.default_rng(5)
    pool = pkv.Pool(64, B, 1, G, D, max_seqs=2)
    s = pool.seq_new(600)
    kv = (_rand(rng, (300, G * D)), _rand(rng, (300, G * D)))
    fill_history(pool, [s], lambda r: kv)
    q, k, v = _rand(rng, (1, H * D)), _rand(rng, (1, G * D)), _rand(rng, (1, G * D))
    ws = torch.empty(max(pool.decode_workspace_bytes([s], H), 4), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((1, H * D), device="cuda")
    for kernels, timed in (([pkv.K_DECODE], {pkv.K_DECODE}),
                           (None, {pkv.K_DECODE, pkv.K_APPEND})):
        pool.profile_kernels(kernels)
        pool.profile_enable(True)
        pool.ensure_append([s], 1, check=True)
        pool.append_layer([s], 1, 0, dev(k), dev(v), check=True)
        pool.attn_paged_decode([s], 0, H, G, D, dev(q), SCALE, out, ws=ws, check=True)
        pool.advance([s], 1, check=True)
        for kid in (pkv.K_APPEND, pkv.K_DECODE):
            ms, n = pool.profile_read(kid)
            assert (n == 1) == (kid in timed), (kernels, kid, n)
            assert (ms > 0) == (kid in timed)
        pool.profile_enable(False)
    pool.profile_kernels(None)
    pool.close()

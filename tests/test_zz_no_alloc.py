"""The zero-allocation decode entry point (pkv_attn_paged_decode_noalloc)
against pkv_attn_paged_decode on the same rows: bit for bit, and within the
float tolerance of the oracle, on two calls in a row, the second with a
smaller batch of shorter rows (the fixed scratch array keeps the first
call's contents).  Also the refusal when the page-table mirror would have
to grow, and no change in free device memory across a call."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_layer_amd as pkv
from pkv_gpu import assert_close, bits_equal, dev

pytestmark = pytest.mark.gpu

H, G, D, B = 32, 8, 128, 16


def _decode_both(pool, seqs, hist, rng, scale):
    """Append one row per sequence, then decode with both entry points."""
    M = len(seqs)
    q = rng.standard_normal((M, H * D), dtype=np.float32)
    k = rng.standard_normal((M, G * D), dtype=np.float32)
    v = rng.standard_normal((M, G * D), dtype=np.float32)
    pool.ensure_append(seqs, 1, check=True)
    pool.append_layer(seqs, 1, 0, dev(k), dev(v), check=True)
    nb = pool.decode_workspace_bytes(seqs, H)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
    ref = torch.full((M, H * D), float("nan"), device="cuda")
    got = torch.full((M, H * D), float("nan"), device="cuda")
    qd = dev(q)
    pool.attn_paged_decode(seqs, 0, H, G, D, qd, scale, ref, ws=ws, check=True)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    pool.attn_paged_decode_noalloc(seqs, 0, H, G, D, qd, scale, got, check=True)
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    pool.advance(seqs, 1, check=True)
    for r, s in enumerate(seqs):
        hk, hv = hist[s]
        hist[s] = (np.concatenate([hk, k[r:r + 1]]), np.concatenate([hv, v[r:r + 1]]))
    return q, ref, got, free0 - free1


def _oracle_check(q, got, seqs, hist, scale, what):
    g = got.cpu().numpy()
    for r, s in enumerate(seqs):
        rc, o = oracle.attn_contig(q[r:r + 1], hist[s][0], hist[s][1], H, G, D, True, scale)
        assert rc == 0
        assert_close(g[r:r + 1], o, "%s row %d (%d keys)" % (what, r, hist[s][0].shape[0]))


def test_noalloc_decode_equals_decode_twice_second_smaller():
    rng = np.random.default_rng(808)
    lens1 = [int(x) for x in rng.integers(1, 9000, size=24)] + [2047, 2048, 8192, 15]
    n_blocks = sum(l // B + 4 for l in lens1) + 16
    pool = pkv.Pool(n_blocks, B, 1, G, D, max_seqs=64)
    pool.set_free_order(rng.permutation(n_blocks))
    seqs = [pool.seq_new(l + 8) for l in lens1]
    hist = {}
    for s, l in zip(seqs, lens1):
        k = rng.standard_normal((l, G * D), dtype=np.float32)
        v = rng.standard_normal((l, G * D), dtype=np.float32)
        hist[s] = (k, v)
        pool.ensure_append([s], l, check=True)
        pool.append_layer([s], l, 0, dev(k), dev(v), check=True)
        pool.advance([s], l, check=True)
    scale = float(np.float32(1 / np.sqrt(D)))

    # first call: the whole batch (rows with 1 to 5 key splits)
    q, ref, got, dmem = _decode_both(pool, seqs, hist, rng, scale)
    assert bits_equal(got, ref), "first call: noalloc != decode"
    _oracle_check(q, got, seqs, hist, scale, "first call")
    assert dmem == 0, "free device memory changed by %d bytes" % dmem

    # second call: fewer, shorter rows (the scratch holds the first call's data)
    small = [s for s, l in zip(seqs, lens1) if l < 1500][:6]
    assert len(small) >= 3
    q, ref, got, dmem = _decode_both(pool, small, hist, rng, scale)
    assert bits_equal(got, ref), "second call: noalloc != decode"
    _oracle_check(q, got, small, hist, scale, "second call")
    assert dmem == 0, "free device memory changed by %d bytes" % dmem
    pool.close()


def test_noalloc_decode_refuses_to_grow_the_mirror():
    """A sequence whose page table is longer than any before needs a larger
    device mirror: the call refuses (UNSUPPORTED, nothing launched) until a
    call that may allocate (the step's append) has grown it."""
    rng = np.random.default_rng(9)
    pool = pkv.Pool(600, B, 1, G, D, max_seqs=8)
    a = pool.seq_new(64)
    k = rng.standard_normal((40, G * D), dtype=np.float32)
    v = rng.standard_normal((40, G * D), dtype=np.float32)
    pool.ensure_append([a], 40, check=True)
    pool.append_layer([a], 40, 0, dev(k), dev(v), check=True)
    pool.advance([a], 40, check=True)
    b = pool.seq_new(64 * 16 * 8)          # 512 pages: past the 64-entry stride
    pool.ensure_append([a, b], 1, check=True)
    q = dev(rng.standard_normal((2, H * D), dtype=np.float32))
    out = torch.zeros((2, H * D), device="cuda")
    scale = 0.0883883
    assert pool.attn_paged_decode_noalloc([a, b], 0, H, G, D, q, scale, out) == pkv.UNSUPPORTED
    torch.cuda.synchronize()
    assert float(out.abs().max()) == 0.0
    kn = dev(rng.standard_normal((2, G * D), dtype=np.float32))
    pool.append_layer([a, b], 1, 0, kn, kn, check=True)
    assert pool.attn_paged_decode_noalloc([a, b], 0, H, G, D, q, scale, out) == pkv.OK
    torch.cuda.synchronize()
    assert np.all(np.isfinite(out.cpu().numpy()))
    pool.close()

"""GPU-side helpers for the parity tests: build pools and contiguous caches
from the synthetic workloads through the library's own entry points, and
compare results with the oracle's at the stated tolerance."""
import numpy as np
import torch

import paged_kv_gqa_layer_amd as pkv

ATOL = 1e-4
RTOL = 1e-4


def assert_close(gpu, ref, what=""):
    """|gpu - ref| <= 1e-4 + 1e-4 * |ref| elementwise (float32 outputs)."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), what
    err = np.abs(gpu - ref)
    lim = ATOL + RTOL * np.abs(ref)
    bad = err > lim
    if bad.any():
        i = np.unravel_index(np.argmax(err - lim), err.shape)
        raise AssertionError("%s: %d/%d outside tol; worst at %s gpu=%r ref=%r"
                             % (what, bad.sum(), bad.size, i, gpu[i], ref[i]))


def bits_equal(a, b):
    a = a.detach().cpu().contiguous() if isinstance(a, torch.Tensor) else a
    b = b.detach().cpu().contiguous() if isinstance(b, torch.Tensor) else b
    return np.array_equal(np.asarray(a).view(np.uint32), np.asarray(b).view(np.uint32))


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def fill_history(pool, seqs, hist_fn, layer=0, chunk=8192):
    """Append each sequence's cached rows (hist_fn(r) -> (K, V)) and advance."""
    for r, s in enumerate(seqs):
        k, v = hist_fn(r)
        n = k.shape[0]
        if n == 0:
            continue
        pool.ensure_append([s], n, check=True)
        kd, vd = dev(k), dev(v)
        pool.append_layer([s], n, layer, kd, vd, check=True)
        pool.advance([s], n, check=True)
        del kd, vd


def fill_contig(cache, slots, hist_fn, layer=0):
    for r, slot in enumerate(slots):
        k, v = hist_fn(r)
        n = k.shape[0]
        if n == 0:
            continue
        cache.append([slot], [0], n, layer, dev(k), dev(v))


def decode_pool(wl, device="cuda", max_seqs=None):
    """Pool for a DecodeWorkload with its random placement and every
    sequence's cached rows appended (one layer)."""
    pool = pkv.Pool(wl.n_blocks, wl.block_size, 1, wl.n_kv_heads, wl.head_dim,
                    max_seqs=max_seqs or wl.M + 8, device=device)
    pool.set_free_order(wl.free_order())
    seqs = [pool.seq_new(wl.max_tokens) for _ in range(wl.M)]
    assert min(seqs) >= 0
    fill_history(pool, seqs, wl.history)
    return pool, seqs


def decode_step(pool, seqs, q, k, v, n_heads, n_kv_heads, head_dim, scale,
                advance=True):
    """ensure + append + decode (+ advance) for one token per sequence."""
    M = len(seqs)
    pool.ensure_append(seqs, 1, check=True)
    pool.append_layer(seqs, 1, 0, dev(k), dev(v), check=True)
    nb = pool.decode_workspace_bytes(seqs, n_heads)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
    out = torch.full((M, n_heads * head_dim), float("nan"), device="cuda")
    pool.attn_paged_decode(seqs, 0, n_heads, n_kv_heads, head_dim, dev(q),
                           scale, out, ws=ws, check=True)
    if advance:
        pool.advance(seqs, 1, check=True)
    torch.cuda.synchronize()
    return out

"""GPU: attention with widely spread scores against the oracle.

The keys carry a ramp on the first dimension of every kv head and the
queries weight that dimension (the score in base-2 units is about the ramp
value), so a row's running maximum keeps rising along the keys:

- steep: +10 every 32 keys over the first 320 keys, then flat at ~100 --
  the softmax reference moves in every tile of the MFMA bodies (prefill,
  the prefix part of the shared-prefix decode) and every page of the
  decode kernel there;
- moderate: each row rises by 100 over its whole length -- the reference
  moves every few tiles, in between the weights are taken against a stale
  reference (up to 2^8), and a row's split partials differ widely in their
  maxima;
- spike: random keys plus one key ~60 above the rest late in the sequence.

The rise is capped near 100 so that fp32 scores keep ~1e-5 absolute
accuracy (larger scores would test fp32, not the kernels).

Prefill (a 64-row chunk), decode, verify (n_q = 4) and the shared-prefix
decode of three forks, each compared with the oracle at 1e-4 + 1e-4 * |ref|.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_layer_amd as pkv
from pkv_gpu import assert_close, dev, fill_history

pytestmark = pytest.mark.gpu

H, G, D, B = 32, 8, 128, 16
SCALE = float(np.float32(1 / np.sqrt(D)))
SPIKE_AT = 1100


def _kv(profile, first, n, total, rng):
    """K and V rows for positions first .. first + n - 1 of a row of `total`
    keys."""
    K = (rng.standard_normal((n, G * D)) * 0.1).astype(np.float32)
    V = rng.standard_normal((n, G * D)).astype(np.float32)
    pos = np.arange(first, first + n, dtype=np.float64)
    if profile == "steep":
        ramp = np.minimum(pos, 320.0) * (10.0 / 32.0)
    elif profile == "moderate":
        ramp = 100.0 * pos / total
    else:
        ramp = np.where(pos == SPIKE_AT, 60.0, 0.0)
    ramp = ramp.astype(np.float32)
    for g in range(G):
        K[:, g * D] += ramp
    return K, V


def _q(n, rng):
    Q = (rng.standard_normal((n, H * D)) * 0.1).astype(np.float32)
    Q[:, ::D] = 8.0  # dimension 0 of every query head
    return Q


def _pool(lens, extra, rng, profile):
    pool = pkv.Pool(sum((l + extra) // B + 3 for l in lens) * 4, B, 1, G, D, max_seqs=16)
    pool.set_free_order(rng.permutation(pool.n_blocks))
    seqs = [pool.seq_new(l + extra) for l in lens]
    hist = [_kv(profile, 0, l, l + extra, rng) for l in lens]
    fill_history(pool, seqs, lambda r: hist[r])
    return pool, seqs, hist


def _check(got, Q, K, V, causal=True, what=""):
    rc, ref = oracle.attn_contig(Q, K, V, H, G, D, causal, SCALE)
    assert rc == 0
    assert np.isfinite(got).all(), what
    assert_close(got, ref, what)


@pytest.mark.parametrize("profile", ["steep", "moderate", "spike"])
def test_prefill_chunk(profile):
    rng = np.random.default_rng(len(profile))
    lens, n_q = [1436, 636], 64
    pool, seqs, hist = _pool(lens, n_q, rng, profile)
    new = [_kv(profile, l, n_q, l + n_q, rng) for l in lens]
    Q = _q(len(lens) * n_q, rng)
    pool.ensure_append(seqs, n_q, check=True)
    pool.append_layer(seqs, n_q, 0, dev(np.concatenate([k for k, _ in new])),
                      dev(np.concatenate([v for _, v in new])), check=True)
    out = torch.full((len(lens) * n_q, H * D), float("nan"), device="cuda")
    pool.attn_paged_prefill(seqs, n_q, 0, H, G, D, dev(Q), True, SCALE, out, check=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for r in range(len(lens)):
        _check(got[r * n_q:(r + 1) * n_q], Q[r * n_q:(r + 1) * n_q],
               np.concatenate([hist[r][0], new[r][0]]),
               np.concatenate([hist[r][1], new[r][1]]), what="%s seq %d" % (profile, r))
    pool.close()


@pytest.mark.parametrize("profile", ["steep", "moderate", "spike"])
@pytest.mark.parametrize("n_q", [1, 4])
def test_decode_and_verify(profile, n_q):
    rng = np.random.default_rng(10 * n_q + len(profile))
    lens = [1500, 700, 9000]  # the last: 2048-key splits, the decode kernel's deep form
    pool, seqs, hist = _pool(lens, n_q, rng, profile)
    new = [_kv(profile, l, n_q, l + n_q, rng) for l in lens]
    Q = _q(len(lens) * n_q, rng)
    pool.ensure_append(seqs, n_q, check=True)
    pool.append_layer(seqs, n_q, 0, dev(np.concatenate([k for k, _ in new])),
                      dev(np.concatenate([v for _, v in new])), check=True)
    out = torch.full((len(lens) * n_q, H * D), float("nan"), device="cuda")
    if n_q == 1:
        nb = pool.decode_workspace_bytes(seqs, H)
        ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
        pool.attn_paged_decode(seqs, 0, H, G, D, dev(Q), SCALE, out, ws=ws, check=True)
    else:
        nb = pool.verify_workspace_bytes(seqs, n_q, H)
        ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
        pool.attn_paged_verify(seqs, n_q, 0, H, G, D, dev(Q), SCALE, out, ws=ws, check=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for r in range(len(lens)):
        _check(got[r * n_q:(r + 1) * n_q], Q[r * n_q:(r + 1) * n_q],
               np.concatenate([hist[r][0], new[r][0]]),
               np.concatenate([hist[r][1], new[r][1]]),
               what="%s n_q=%d seq %d" % (profile, n_q, r))
    pool.close()


@pytest.mark.parametrize("profile", ["steep", "moderate", "spike"])
def test_shared_prefix_decode(profile):
    rng = np.random.default_rng(100 + len(profile))
    pool, seqs, hist = _pool([2050], 1, rng, profile)
    forks = [pool.seq_fork(seqs[0]) for _ in range(3)]
    batch = seqs + forks
    new = [_kv(profile, 2050, 1, 2051, rng) for _ in batch]
    Q = _q(len(batch), rng)
    pool.ensure_append(batch, 1, check=True)
    pool.append_layer(batch, 1, 0, dev(np.concatenate([k for k, _ in new])),
                      dev(np.concatenate([v for _, v in new])), check=True)
    nb = pool.decode_shared_workspace_bytes(batch, H)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
    out = torch.full((len(batch), H * D), float("nan"), device="cuda")
    pool.attn_paged_decode_shared(batch, 0, H, G, D, dev(Q), SCALE, out, ws=ws, check=True)
    torch.cuda.synchronize()
    assert pool.kernel_name(pkv.K_PREFIX).startswith("shared_decode_kernel")
    got = out.cpu().numpy()
    for r in range(len(batch)):
        _check(got[r:r + 1], Q[r:r + 1], np.concatenate([hist[0][0], new[r][0]]),
               np.concatenate([hist[0][1], new[r][1]]), what="%s row %d" % (profile, r))
    pool.close()

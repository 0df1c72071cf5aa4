"""Pins for the oracle's attention arithmetic (CPU only).

Each test checks the oracle against something other than itself: the worked
example printed on the pages, closed forms, invariants that follow from the
definition, or a float64 library attention routine.  Together they catch a
dropped term, a wrong sign, a wrong kv-head mapping, a transposed operand or
a wrong causal offset.
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden


def _nums(s, dtype=np.float32):
    return np.array([float(x) for x in s.split()], dtype=dtype)


# ---------------------------------------------------------------- the pages

def test_worked_example_q0_from_pages():
    g = read_golden("gqa_q0_worked_example.txt")
    n, H, G, D = (int(g[k]) for k in ("n_tokens", "n_q_heads", "n_kv_heads", "head_dim"))
    Q = _nums(g["Q"]).reshape(n, H * D)
    K = _nums(g["K"]).reshape(n, G * D)
    V = _nums(g["V"]).reshape(n, G * D)
    rc, out = oracle.gqa_attention(Q, K, V, n, H, G, D, float(g["scale"]))
    assert rc == 0
    want = _nums(g["expected_per_token_head"])
    tol = float(g["tolerance"])
    for t in range(n):
        for h in range(H):
            got = out[t, h * D:(h + 1) * D]
            assert np.all(np.abs(got - want) < tol)
            # the mean of two small integers is exact in float
            assert np.array_equal(got, want)


def test_bad_grouping_rejected_by_every_form():
    g = read_golden("gqa_q0_worked_example.txt")
    H, G = int(g["bad_grouping_q_heads"]), int(g["bad_grouping_kv_heads"])
    D, n = 2, 2
    Q = np.zeros((n, H * D), np.float32)
    K = np.ones((n, G * D), np.float32)
    V = np.ones((n, G * D), np.float32)
    rc, _ = oracle.gqa_attention(Q, K, V, n, H, G, D, 1.0)
    assert rc == 1
    rc, _ = oracle.attn_contig(Q, K, V, H, G, D, True, 1.0)
    assert rc == oracle.BAD_GQA
    c = oracle.Cache(1, G, 8, D)
    rc, _ = c.attn_with_cache(Q, K, V, n, H, G, D, 0, True, 1.0)
    assert rc == oracle.BAD_GQA
    p = oracle.Pool(4, 4, 1, G, D)
    s = p.seq_new(8)
    assert p.ensure_append([s], n) == 0
    rc, _ = p.attn_with_paged(Q, K, V, n, H, G, D, s, 0, True, 1.0)
    assert rc == oracle.BAD_GQA


@pytest.mark.parametrize("bad", [
    dict(n_q=0), dict(H=0), dict(G=0), dict(D=0)])
def test_bad_dims_rejected(bad):
    a = dict(n_q=2, H=4, G=2, D=4)
    a.update(bad)
    Q = np.zeros((max(a["n_q"], 1), max(a["H"], 1) * max(a["D"], 1)), np.float32)
    K = np.zeros((4, 8), np.float32)
    rc = oracle.lib().pkvo_attn_contig(
        oracle._ptr(Q), oracle._ptr(K), oracle._ptr(K), a["n_q"], 4, a["H"],
        a["G"], a["D"], 1, 1.0, oracle._ptr(np.zeros(64, np.float32)))
    assert rc == oracle.BAD_DIM


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("H,G", [(4, 2), (8, 2), (6, 3), (4, 4), (4, 1)])
@pytest.mark.parametrize("causal", [False, True])
def test_q_zero_gives_mean_of_shared_kv_head(H, G, causal):
    rng = np.random.default_rng(11)
    D, n_q, total_k = 5, 3, 7
    Q = np.zeros((n_q, H * D), np.float32)
    K = rng.standard_normal((total_k, G * D)).astype(np.float32)
    # distinct values per kv head so a wrong head mapping shows
    V = (rng.standard_normal((total_k, G * D)) +
         np.repeat(np.arange(G) * 10.0, D)[None, :]).astype(np.float32)
    rc, out = oracle.attn_contig(Q, K, V, H, G, D, causal, 0.37)
    assert rc == 0
    g = H // G
    for i in range(n_q):
        q_pos = total_k - n_q + i
        vis = q_pos + 1 if causal else total_k
        for h in range(H):
            c = h // g
            want = V[:vis, c * D:(c + 1) * D].astype(np.float64).mean(axis=0)
            np.testing.assert_allclose(out[i, h * D:(h + 1) * D], want,
                                       rtol=1e-6, atol=1e-6)


def test_single_visible_key_returns_that_value_row():
    rng = np.random.default_rng(12)
    H, G, D, n = 4, 2, 6, 5
    Q = rng.standard_normal((n, H * D)).astype(np.float32)
    K = rng.standard_normal((n, G * D)).astype(np.float32)
    V = rng.standard_normal((n, G * D)).astype(np.float32)
    # n_q == total_k and causal: query 0 sits at position 0 and sees key 0 only
    rc, out = oracle.attn_contig(Q, K, V, H, G, D, True, 0.5)
    assert rc == 0
    for h in range(H):
        c = h // (H // G)
        assert np.array_equal(out[0, h * D:(h + 1) * D], V[0, c * D:(c + 1) * D])


def test_identical_keys_give_mean_of_values():
    rng = np.random.default_rng(13)
    H, G, D, n_q, total_k = 4, 2, 8, 2, 9
    Q = rng.standard_normal((n_q, H * D)).astype(np.float32)
    K = np.tile(rng.standard_normal((1, G * D)).astype(np.float32), (total_k, 1))
    V = rng.standard_normal((total_k, G * D)).astype(np.float32)
    rc, out = oracle.attn_contig(Q, K, V, H, G, D, False, 0.3)
    assert rc == 0
    for h in range(H):
        c = h // (H // G)
        want = V[:, c * D:(c + 1) * D].astype(np.float64).mean(axis=0)
        for i in range(n_q):
            np.testing.assert_allclose(out[i, h * D:(h + 1) * D], want,
                                       rtol=1e-6, atol=1e-6)


def test_hard_attention_limit_picks_argmax_key():
    rng = np.random.default_rng(14)
    H, G, D, total_k = 2, 1, 4, 6
    K = rng.integers(-3, 4, size=(total_k, G * D)).astype(np.float32)
    V = rng.standard_normal((total_k, G * D)).astype(np.float32)
    Q = rng.integers(-3, 4, size=(1, H * D)).astype(np.float32)
    rc, out = oracle.attn_contig(Q, K, V, H, G, D, False, 1000.0)
    assert rc == 0
    for h in range(H):
        s = K @ Q[0, h * D:(h + 1) * D]
        top = np.sort(s)[::-1]
        if top[0] - top[1] < 0.5:
            continue  # tie: no unique hard choice
        j = int(np.argmax(s))
        np.testing.assert_allclose(out[0, h * D:(h + 1) * D], V[j], atol=1e-30)


def test_key_shift_invariance():
    """Adding one vector c to every key adds q.c to every score of a query,
    which the softmax cancels."""
    rng = np.random.default_rng(15)
    H, G, D, n_q, total_k = 4, 2, 8, 3, 10
    Q = rng.standard_normal((n_q, H * D)).astype(np.float32)
    K = rng.integers(-4, 5, size=(total_k, G * D)).astype(np.float32)
    V = rng.standard_normal((total_k, G * D)).astype(np.float32)
    c = rng.integers(-4, 5, size=(1, G * D)).astype(np.float32)
    rc1, o1 = oracle.attn_contig(Q, K, V, H, G, D, True, 0.25)
    rc2, o2 = oracle.attn_contig(Q, K + c, V, H, G, D, True, 0.25)
    assert rc1 == rc2 == 0
    np.testing.assert_allclose(o1, o2, rtol=2e-6, atol=2e-6)


# ---------------------------------------------- float64 library attention

def _sdpa_reference(Q, K, V, H, G, D, causal, scale):
    """torch SDPA in float64 on the CPU: kv heads expanded to their groups
    (head h reads kv head h // (H/G)) and an explicit offset-causal mask."""
    n_q, total_k = Q.shape[0], K.shape[0]
    q = torch.from_numpy(Q.astype(np.float64)).view(n_q, H, D).transpose(0, 1)
    k = torch.from_numpy(K.astype(np.float64)).view(total_k, G, D).transpose(0, 1)
    v = torch.from_numpy(V.astype(np.float64)).view(total_k, G, D).transpose(0, 1)
    k = k.repeat_interleave(H // G, dim=0).contiguous()
    v = v.repeat_interleave(H // G, dim=0).contiguous()
    mask = None
    if causal:
        q_pos = torch.arange(n_q) + (total_k - n_q)
        mask = torch.arange(total_k)[None, :] <= q_pos[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(
        q[None], k[None], v[None], attn_mask=mask, scale=float(scale))[0]
    return o.transpose(0, 1).reshape(n_q, H * D).numpy()


@pytest.mark.parametrize("H,G,D,n_q,total_k,causal", [
    (4, 2, 8, 1, 1, True),          # first decode step
    (4, 2, 8, 1, 13, True),         # decode: one query sees all keys
    (8, 2, 16, 5, 5, True),         # prefill from empty
    (8, 2, 16, 5, 23, True),        # chunked prefill with offset
    (6, 3, 12, 7, 19, False),       # unmasked
    (32, 8, 128, 3, 40, True),      # the Qwen3-4B head shape
    (4, 4, 8, 2, 9, True),          # multi-head (group 1)
    (8, 1, 8, 3, 9, True),          # multi-query (one kv head)
])
def test_matches_float64_sdpa(H, G, D, n_q, total_k, causal):
    rng = np.random.default_rng(H * 1000 + n_q * 10 + total_k)
    Q = rng.standard_normal((n_q, H * D)).astype(np.float32)
    K = rng.standard_normal((total_k, G * D)).astype(np.float32)
    V = rng.standard_normal((total_k, G * D)).astype(np.float32)
    scale = float(np.float32(1 / np.sqrt(D)))
    rc, out = oracle.attn_contig(Q, K, V, H, G, D, causal, scale)
    assert rc == 0
    ref = _sdpa_reference(Q, K, V, H, G, D, causal, scale)
    # the oracle rounds once from double to float: within half an ulp
    np.testing.assert_allclose(out, ref, rtol=1.2e-7, atol=1e-30)

"""Pins of the oracle's rotary embedding ("nx_f32_llama_v4b.nx source",
nx_f32_llama_block_forward_v4b, the RoPE step: neox form, position = the
row's sequence length, applied to every q head and kv head before the
append).

The reading pinned here: pair (x_i, x_{i+D/2}) turns by pos * exp(-(2i/D) *
log_base) radians, counter-clockwise.  Each test checks the oracle against
something other than its own formula: a complex-number form evaluated by
numpy, the rotation group law, the relative-position property the method
exists for, closed forms at D = 2, and exact special cases.
"""
import math

import numpy as np
import pytest

import oracle

LOG_BASE = math.log(10000.0)


def _rand(rng, shape):
    return rng.standard_normal(shape).astype(np.float32)


def test_position_zero_is_identity():
    rng = np.random.default_rng(1)
    x = _rand(rng, (3, 4 * 16))
    rc, y = oracle.rope(x, 4, 16, [0, 0, 0], LOG_BASE)
    assert rc == oracle.OK
    assert np.array_equal(x, y)


def test_head_dim_two_is_plain_rotation_by_pos_radians():
    # D = 2: one pair, frequency exp(0) = 1, angle = pos.
    for pos in (1, 2, 7, 1000):
        rc, y = oracle.rope(np.array([[1.0, 0.0], [0.0, 1.0]], np.float32), 1, 2,
                            [pos, pos], LOG_BASE)
        assert rc == oracle.OK
        c, s = math.cos(pos), math.sin(pos)
        # e1 -> (cos, sin), e2 -> (-sin, cos): counter-clockwise
        assert y[0, 0] == np.float32(c) and y[0, 1] == np.float32(s)
        assert y[1, 0] == np.float32(-s) and y[1, 1] == np.float32(c)


def test_matches_complex_multiplication_form():
    # neox pairing as complex numbers z_i = x_i + j x_{i+half}, turned by
    # exp(j * pos * base^(-2i/D)), evaluated independently with numpy.
    rng = np.random.default_rng(2)
    H, D = 3, 64
    pos = np.array([0, 1, 5, 77, 4095, 16383], np.int32)
    x = _rand(rng, (pos.size, H * D))
    rc, y = oracle.rope(x, H, D, pos, LOG_BASE)
    assert rc == oracle.OK
    half = D // 2
    base = math.exp(LOG_BASE)
    freq = base ** (-(2.0 * np.arange(half)) / D)
    xr = x.astype(np.float64).reshape(pos.size, H, D)
    z = xr[..., :half] + 1j * xr[..., half:]
    rot = np.exp(1j * pos[:, None, None].astype(np.float64) * freq[None, None, :])
    w = z * rot
    ref = np.concatenate([w.real, w.imag], axis=-1).reshape(pos.size, H * D)
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-6 * (1 + np.abs(ref)).max())


def test_pair_norms_preserved():
    rng = np.random.default_rng(3)
    H, D = 2, 128
    x = _rand(rng, (5, H * D))
    rc, y = oracle.rope(x, H, D, [3, 100, 999, 5000, 65535], LOG_BASE)
    assert rc == oracle.OK
    half = D // 2
    xr = x.astype(np.float64).reshape(5, H, D)
    yr = y.astype(np.float64).reshape(5, H, D)
    nx = xr[..., :half] ** 2 + xr[..., half:] ** 2
    ny = yr[..., :half] ** 2 + yr[..., half:] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-6, atol=1e-7)


def test_group_law_composition():
    # R(a) R(b) = R(a + b): rotating at 37 then at 91 equals rotating at 128.
    rng = np.random.default_rng(4)
    H, D = 2, 32
    x = _rand(rng, (1, H * D))
    _, y1 = oracle.rope(x, H, D, [37], LOG_BASE)
    _, y2 = oracle.rope(y1, H, D, [91], LOG_BASE)
    _, y3 = oracle.rope(x, H, D, [128], LOG_BASE)
    np.testing.assert_allclose(y2, y3, rtol=0, atol=2e-6)


def test_scores_depend_only_on_relative_position():
    # <R(q, m), R(k, n)> is a function of m - n.
    rng = np.random.default_rng(5)
    D = 128
    q = _rand(rng, (1, D))
    k = _rand(rng, (1, D))
    dots = []
    for shift in (0, 1, 500, 9000):
        _, qr = oracle.rope(q, 1, D, [40 + shift], LOG_BASE)
        _, kr = oracle.rope(k, 1, D, [13 + shift], LOG_BASE)
        dots.append(float(qr[0].astype(np.float64) @ kr[0].astype(np.float64)))
    np.testing.assert_allclose(dots, dots[0], rtol=0, atol=2e-4)
    # and it does change with the offset (a dropped rotation would not)
    _, qr = oracle.rope(q, 1, D, [41], LOG_BASE)
    _, kr = oracle.rope(k, 1, D, [13], LOG_BASE)
    assert abs(float(qr[0].astype(np.float64) @ kr[0].astype(np.float64)) - dots[0]) > 1e-3


def test_first_pair_has_unit_frequency_and_last_the_lowest():
    # i = 0 turns by exactly pos radians whatever the base; the highest pair
    # turns by pos * base^(-(D-2)/D).
    D = 8
    x = np.zeros((1, D), np.float32)
    x[0, 0] = 1.0
    x[0, 3] = 1.0
    pos = 3
    _, y = oracle.rope(x, 1, D, [pos], math.log(500000.0))
    assert y[0, 0] == np.float32(math.cos(pos)) and y[0, 4] == np.float32(math.sin(pos))
    ang = pos * 500000.0 ** (-(D - 2) / D)
    assert abs(y[0, 3] - math.cos(ang)) < 1e-7 and abs(y[0, 7] - math.sin(ang)) < 1e-7


def test_pairs_split_halves_not_neighbours():
    # Only dims i and i + D/2 mix (neox); dims 0 and 1 stay apart.
    D = 8
    x = np.zeros((1, D), np.float32)
    x[0, 1] = 1.0
    _, y = oracle.rope(x, 1, D, [5], LOG_BASE)
    nz = set(np.nonzero(y[0])[0].tolist())
    assert nz == {1, 5}


def test_heads_rotate_independently_at_the_rows_position():
    rng = np.random.default_rng(6)
    H, D = 4, 16
    x = _rand(rng, (2, H * D))
    _, y = oracle.rope(x, H, D, [9, 21], LOG_BASE)
    for r, p in enumerate((9, 21)):
        for h in range(H):
            _, yh = oracle.rope(x[r:r + 1, h * D:(h + 1) * D], 1, D, [p], LOG_BASE)
            assert np.array_equal(yh[0], y[r, h * D:(h + 1) * D])


def test_errors():
    x = np.zeros((1, 6), np.float32)
    assert oracle.rope(x, 1, 6, [0], 0.0)[0] == oracle.BAD_ARG
    assert oracle.rope(x, 1, 6, [-1], LOG_BASE)[0] == oracle.BAD_ARG
    assert oracle.rope(np.zeros((1, 5), np.float32), 1, 5, [0], LOG_BASE)[0] == oracle.BAD_DIM
    with pytest.raises(ValueError):
        oracle.rope(x, 1, 6, [0, 1], LOG_BASE)


def test_rotated_attention_is_shift_invariant():
    # Rotating queries and keys at their positions makes the attention output
    # a function of relative positions only: a chunk whose positions are all
    # shifted by s gives the same output (the reading's purpose).
    rng = np.random.default_rng(7)
    H, G, D, n = 4, 2, 32, 9
    Q = _rand(rng, (n, H * D))
    K = _rand(rng, (n, G * D))
    V = _rand(rng, (n, G * D))
    outs = []
    for s in (0, 1000):
        pos = np.arange(n, dtype=np.int32) + s
        _, Qr = oracle.rope(Q, H, D, pos, LOG_BASE)
        _, Kr = oracle.rope(K, G, D, pos, LOG_BASE)
        rc, o = oracle.attn_contig(Qr, Kr, V, H, G, D, True, 1.0 / math.sqrt(D))
        assert rc == oracle.OK
        outs.append(o)
    np.testing.assert_allclose(outs[0], outs[1], rtol=0, atol=5e-5)

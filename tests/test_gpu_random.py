"""Seeded randomised GPU parity: shapes (fast and generic paths), batch
sizes, history lengths (now and then a row of 8192+ keys, which takes the
decode kernel's deep form), query counts, entry points (decode, the
append-then-attend call, shared-prefix decode, verify, prefill causal /
non-causal), rotary embedding on / off and block placement are drawn per
case; every output row is compared with the
oracle at 1e-4 + 1e-4 * |oracle|, and the contiguous twin must agree bit for
bit where it applies."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_layer_amd as pkv
from pkv_gpu import assert_close, bits_equal, dev, fill_contig, fill_history

pytestmark = pytest.mark.gpu

SHAPES = [  # (H, G, D, B)
    (32, 8, 128, 16), (8, 8, 128, 16), (16, 8, 128, 16), (64, 8, 128, 16),
    (12, 4, 64, 16), (6, 2, 42, 5), (32, 8, 128, 8), (4, 1, 32, 4),
]
KINDS = ["decode", "with", "shared", "verify", "prefill", "prefill_nc"]
LB = math.log(10000.0)


def _case(seed):
    rng = np.random.default_rng(seed)
    H, G, D, B = SHAPES[rng.integers(len(SHAPES))]
    kind = KINDS[rng.integers(len(KINDS))]
    M = int(rng.integers(1, 6))
    n_q = {"decode": 1, "with": 1, "shared": 1, "verify": int(rng.integers(1, 9)),
           "prefill": int(rng.integers(1, 70)), "prefill_nc": int(rng.integers(1, 70))}[kind]
    rope = bool(rng.integers(2)) and D % 2 == 0
    lens = [int(x) for x in rng.integers(0, 1300, size=M)]
    if kind in ("decode", "with", "verify") and rng.random() < 0.2:
        lens[int(rng.integers(M))] = int(rng.integers(8192, 9200))
    return rng, H, G, D, B, kind, M, n_q, rope, lens


def _turn(x, heads, D, pos, rope):
    if not rope:
        return x
    rc, y = oracle.rope(x, heads, D, pos, LB)
    assert rc == 0
    return y


def _seeds():
    """range(180), or PKV_RANDOM_SEEDS="lo:hi" for a wider campaign."""
    import os
    lo, _, hi = os.environ.get("PKV_RANDOM_SEEDS", "0:180").partition(":")
    return range(int(lo), int(hi))


@pytest.mark.parametrize("seed", _seeds())
def test_random_case(seed):
    rng, H, G, D, B, kind, M, n_q, rope, lens = _case(1000 + seed)
    scale = float(np.float32(1 / math.sqrt(D)))
    max_len = max(lens) + n_q + 1
    pool = pkv.Pool(sum((l + n_q) // B + 3 for l in lens) + 4 * (600 // B + 2), B, 1, G, D,
                    max_seqs=M + 8)
    pool.set_free_order(rng.permutation(pool.n_blocks))
    table = pkv.Rope(D, LB, max_len + 600) if rope else None
    pool.set_rope(table)
    if kind == "shared":
        # forks of one prefix (>= 16 full pages) beside unrelated sequences
        pre = int(rng.integers(16 * B, 16 * B + 300))
        base = pool.seq_new(pre + max_len)
        pk = rng.standard_normal((pre, G * D), dtype=np.float32)
        pv = rng.standard_normal((pre, G * D), dtype=np.float32)
        fill_history(pool, [base], lambda r: (pk, pv))
        n_fork = max(2, M - 1)
        seqs = [pool.seq_fork(base) for _ in range(n_fork)]
        hist = [(pk, pv)] * n_fork
        extra = pool.seq_new(max_len)
        ek = rng.standard_normal((lens[0], G * D), dtype=np.float32)
        ev = rng.standard_normal((lens[0], G * D), dtype=np.float32)
        fill_history(pool, [extra], lambda r: (ek, ev))
        seqs.append(extra)
        hist.append((ek, ev))
        lens = [pre] * n_fork + [lens[0]]
        M = len(seqs)
    else:
        seqs = [pool.seq_new(l + n_q) for l in lens]
        hist = [(rng.standard_normal((l, G * D), dtype=np.float32),
                 rng.standard_normal((l, G * D), dtype=np.float32)) for l in lens]
        fill_history(pool, seqs, lambda r: hist[r])
    Q = rng.standard_normal((M * n_q, H * D), dtype=np.float32)
    K = rng.standard_normal((M * n_q, G * D), dtype=np.float32)
    V = rng.standard_normal((M * n_q, G * D), dtype=np.float32)
    pool.ensure_append(seqs, n_q, check=True)
    if kind != "with":
        pool.append_layer(seqs, n_q, 0, dev(K), dev(V), check=True)
    out = torch.full((M * n_q, H * D), float("nan"), device="cuda")
    causal = kind != "prefill_nc"
    if kind == "with":
        nb = pool.decode_workspace_bytes(seqs, H)
        ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
        pool.attn_with_paged_decode(seqs, 0, H, G, D, dev(Q), dev(K), dev(V), scale, out,
                                    ws=ws, check=True)
    elif kind == "decode":
        nb = pool.decode_workspace_bytes(seqs, H)
        ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
        pool.attn_paged_decode(seqs, 0, H, G, D, dev(Q), scale, out, ws=ws, check=True)
    elif kind == "shared":
        nb = pool.decode_shared_workspace_bytes(seqs, H)
        ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
        pool.attn_paged_decode_shared(seqs, 0, H, G, D, dev(Q), scale, out, ws=ws,
                                      check=True)
    elif kind == "verify":
        nb = pool.verify_workspace_bytes(seqs, n_q, H)
        ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
        pool.attn_paged_verify(seqs, n_q, 0, H, G, D, dev(Q), scale, out, ws=ws,
                               check=True)
    else:
        pool.attn_paged_prefill(seqs, n_q, 0, H, G, D, dev(Q), causal, scale, out,
                                check=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    what = "seed %d: %s H=%d G=%d D=%d B=%d M=%d n_q=%d rope=%d" % (
        seed, kind, H, G, D, B, M, n_q, rope)
    for r in range(M):
        rows = slice(r * n_q, (r + 1) * n_q)
        L = lens[r]
        Kc = _turn(np.concatenate([hist[r][0], K[rows]]), G, D, np.arange(L + n_q), rope)
        Vc = np.concatenate([hist[r][1], V[rows]])
        Qr = _turn(Q[rows], H, D, L + np.arange(n_q), rope)
        rc, ref = oracle.attn_contig(Qr, Kc, Vc, H, G, D, causal, scale)
        assert rc == 0
        assert_close(got[rows], ref, "%s row %d (len %d)" % (what, r, L))
    if kind in ("decode", "with", "prefill", "prefill_nc"):
        cc = pkv.ContigCache(M, 1, G, max(lens) + n_q, D, block_size=B, rope=table)
        fill_contig(cc, list(range(M)), lambda r: hist[r])
        cc.append(list(range(M)), lens, n_q, 0, dev(K), dev(V))
        cout = torch.full_like(out, float("nan"))
        if kind in ("decode", "with"):
            cws = torch.empty(max(cc.decode_workspace_bytes(lens, H), 4), dtype=torch.uint8,
                              device="cuda")
            cc.attn_decode(list(range(M)), lens, 0, H, dev(Q), scale, cout, ws=cws)
        else:
            cc.attn_prefill(list(range(M)), lens, n_q, 0, H, dev(Q), causal, scale, cout)
        torch.cuda.synchronize()
        assert bits_equal(out, cout), what
    pool.close()

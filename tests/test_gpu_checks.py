"""Debug state checks (pkv_pool_set_checks level 2: host state, row
descriptors and the device page-table mirror read back before every launch)
on a pool driven through decode, fork with copy-on-append, verify with
truncate, prefill, shared-prefix decode and the zero-allocation decode: no
check fires, and every output is bit-identical to a twin pool without checks
fed the same calls."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_layer_amd as pkv
from pkv_gpu import bits_equal, dev

pytestmark = pytest.mark.gpu

H, G, D, B = 32, 8, 128, 16


def test_checked_pool_matches_unchecked_twin():
    rng = np.random.default_rng(515)
    n_blocks = 1200
    order = rng.permutation(n_blocks)
    pools = []
    for checks in (2, 0):
        p = pkv.Pool(n_blocks, B, 2, G, D, max_seqs=32)
        p.set_free_order(order)
        p.set_checks(checks)
        pools.append(p)
    scale = float(np.float32(1 / np.sqrt(D)))
    lens = [2053, 700, 33, 4100]

    def both(fn):
        outs = [fn(p) for p in pools]
        return outs

    seqs = both(lambda p: [p.seq_new(9000) for _ in lens])
    assert seqs[0] == seqs[1]
    seqs = seqs[0]
    for s, l in zip(seqs, lens):
        k = dev(rng.standard_normal((l, G * D), dtype=np.float32))
        v = dev(rng.standard_normal((l, G * D), dtype=np.float32))
        for p in pools:
            p.ensure_append([s], l, check=True)
            for L in range(2):
                p.append_layer([s], l, L, k, v, check=True)
            p.advance([s], l, check=True)
    # forks of the non-aligned first sequence: copy-on-append at the next append
    forks = both(lambda p: [p.seq_fork(seqs[0]) for _ in range(3)])
    assert forks[0] == forks[1]
    batch = seqs + forks[0]
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")

    def decode_step(kind):
        M = len(batch)
        q = dev(rng.standard_normal((M, H * D), dtype=np.float32))
        k = dev(rng.standard_normal((M, G * D), dtype=np.float32))
        v = dev(rng.standard_normal((M, G * D), dtype=np.float32))
        outs = []
        for p in pools:
            p.ensure_append(batch, 1, check=True)
            o = []
            for L in range(2):
                p.append_layer(batch, 1, L, k, v, check=True)
                out = torch.full((M, H * D), float("nan"), device="cuda")
                if kind == "plain":
                    p.attn_paged_decode(batch, L, H, G, D, q, scale, out, ws=ws, check=True)
                elif kind == "shared":
                    p.attn_paged_decode_shared(batch, L, H, G, D, q, scale, out, ws=ws,
                                               check=True)
                else:
                    p.attn_paged_decode_noalloc(batch, L, H, G, D, q, scale, out, check=True)
                o.append(out)
            p.advance(batch, 1, check=True)
            outs.append(o)
        torch.cuda.synchronize()
        for a, b in zip(*outs):
            assert bits_equal(a, b), kind

    for kind in ("plain", "plain", "shared", "noalloc", "plain"):
        decode_step(kind)

    # verify 4 drafted rows, keep 2, then a prefill chunk of 40 rows
    for n_q, keep in ((4, 2), (40, 40)):
        M = len(batch)
        q = dev(rng.standard_normal((M * n_q, H * D), dtype=np.float32))
        k = dev(rng.standard_normal((M * n_q, G * D), dtype=np.float32))
        v = dev(rng.standard_normal((M * n_q, G * D), dtype=np.float32))
        outs = []
        for p in pools:
            lens_now = [p.seq_len(s) for s in batch]
            p.ensure_append(batch, n_q, check=True)
            p.append_layer(batch, n_q, 0, k, v, check=True)
            out = torch.full((M * n_q, H * D), float("nan"), device="cuda")
            if n_q == 4:
                p.attn_paged_verify(batch, n_q, 0, H, G, D, q, scale, out, ws=ws, check=True)
            else:
                p.attn_paged_prefill(batch, n_q, 0, H, G, D, q, True, scale, out, check=True)
            p.advance(batch, n_q, check=True)
            for s, l in zip(batch, lens_now):
                p.seq_truncate(s, l + keep, check=True)
            outs.append(out)
        torch.cuda.synchronize()
        assert bits_equal(outs[0], outs[1]), n_q
    assert [p.refcounts().tolist() for p in pools][0] == pools[1].refcounts().tolist()
    for p in pools:
        p.close()

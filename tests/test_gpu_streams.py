"""GPU: the library on caller streams.  All of a pool's device work goes to
the stream each call names; a call naming a different stream than the
pool's previous one first waits for that stream to drain.  Decode steps run
on one side stream, and alternating between two side streams, give the same
bits as on the default stream; so does prefill on a side stream."""
import math

import numpy as np
import pytest
import torch

import paged_kv_gqa_layer_amd as pkv
from pkv_gpu import bits_equal, dev, fill_history

pytestmark = pytest.mark.gpu

H, G, D, B = 32, 8, 128, 16
SCALE = float(np.float32(1 / math.sqrt(D)))


def _pool(lens, seed):
    rng = np.random.default_rng(seed)
    n_blocks = sum((l + 64) // B + 2 for l in lens) + 8
    pool = pkv.Pool(n_blocks, B, 1, G, D, max_seqs=len(lens) + 4)
    pool.set_free_order(np.random.default_rng(seed + 1).permutation(n_blocks))
    seqs = [pool.seq_new(l + 64) for l in lens]
    hist = [(rng.standard_normal((l, G * D)).astype(np.float32),
             rng.standard_normal((l, G * D)).astype(np.float32)) for l in lens]
    fill_history(pool, seqs, lambda r: hist[r])
    torch.cuda.synchronize()
    return pool, seqs


def _steps(pool, seqs, inputs, streams):
    """Decode steps, step t on streams[t % len(streams)] (None: default)."""
    outs = []
    M = len(seqs)
    for t, (q, k, v) in enumerate(inputs):
        st = streams[t % len(streams)]
        ctx = torch.cuda.stream(st) if st is not None else torch.cuda.stream(
            torch.cuda.current_stream())
        with ctx:
            cur = torch.cuda.current_stream()
            out = torch.full((M, H * D), float("nan"), device="cuda")
            nb = pool.decode_workspace_bytes(seqs, H)
            ws = torch.empty(max(nb, 4), dtype=torch.uint8, device="cuda")
            pool.ensure_append(seqs, 1, stream=cur, check=True)
            pool.append_layer(seqs, 1, 0, q_k_v(k), q_k_v(v), stream=cur, check=True)
            pool.attn_paged_decode(seqs, 0, H, G, D, q_k_v(q), SCALE, out, ws=ws,
                                   stream=cur, check=True)
            pool.advance(seqs, 1, check=True)
            outs.append(out)
    torch.cuda.synchronize()
    return outs


def q_k_v(x):
    # inputs were made on the default stream and synchronised; a copy made on
    # the current stream keeps the tensor's use on that stream
    return x.clone()


@pytest.mark.parametrize("mode", ["one_side_stream", "alternating"])
def test_decode_on_caller_streams(mode):
    lens = [1, 300, 2047, 5000, 9000]
    rng = np.random.default_rng(7)
    M = len(lens)
    inputs = [tuple(dev(rng.standard_normal(s, dtype=np.float32))
                    for s in ((M, H * D), (M, G * D), (M, G * D))) for _ in range(12)]
    torch.cuda.synchronize()
    pa, sa = _pool(lens, 3)
    ref = _steps(pa, sa, inputs, [None])
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    pb, sb = _pool(lens, 3)
    got = _steps(pb, sb, inputs, [s1] if mode == "one_side_stream" else [s1, None, s2])
    for t, (x, y) in enumerate(zip(ref, got)):
        assert bits_equal(x, y), t
    pa.close()
    pb.close()


def test_prefill_on_a_side_stream():
    lens = [700, 40]
    rng = np.random.default_rng(8)
    n_q = 37
    Q = dev(rng.standard_normal((2 * n_q, H * D), dtype=np.float32))
    K = dev(rng.standard_normal((2 * n_q, G * D), dtype=np.float32))
    V = dev(rng.standard_normal((2 * n_q, G * D), dtype=np.float32))
    torch.cuda.synchronize()
    outs = []
    for st in (None, torch.cuda.Stream()):
        pool, seqs = _pool(lens, 4)
        ctx = torch.cuda.stream(st) if st is not None else torch.cuda.stream(
            torch.cuda.current_stream())
        with ctx:
            cur = torch.cuda.current_stream()
            out = torch.full((2 * n_q, H * D), float("nan"), device="cuda")
            pool.ensure_append(seqs, n_q, stream=cur, check=True)
            pool.append_layer(seqs, n_q, 0, K.clone(), V.clone(), stream=cur, check=True)
            pool.attn_paged_prefill(seqs, n_q, 0, H, G, D, Q.clone(), True, SCALE, out,
                                    stream=cur, check=True)
        torch.cuda.synchronize()
        outs.append(out)
        pool.close()
    assert bits_equal(outs[0], outs[1])

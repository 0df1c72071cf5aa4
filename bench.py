"""Benchmark: batched paged-GQA decode on one MI355X.

One step = the whole decode hot path for M=256 sequences, one new token
each: ensure_append (capacity + copy-on-append), append_layer (scatter of
the new K/V rows), attn_paged_decode (split decode kernel + split merge,
page tables uploaded once per step), advance.  Workload: Qwen3-4B-shaped
attention (32 query heads, 8 kv heads, head_dim 128), float32, 16-row pages
placed by a seeded random permutation, context lengths log-uniform on
[1024, 16384].  All inputs are synthetic (seeded numpy) and resident in HBM
before the timed region.

Prints one JSON line.  ``value`` is the whole-step KV throughput in GB/s
(algorithmic K+V bytes the step must read, 8192 B per visible key, divided
by wall time of the timed steps); ``roofline`` is the decode kernel's
achieved bandwidth from HIP events around each launch against 8 TB/s;
``cpu_baseline`` is the CPU oracle on a bounded sample of the same workload.
A secondary object measures chunked prefill (8 x (3584 cached + 512 new))
against the FP32 MFMA peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
VERIFY_NQ = (4, 8)       # drafted tokens verified per sequence and step
VERIFY_ROWS_MAX = 8
COLD_STEPS = 10  # decode steps each preceded by a cache-evicting 1 GiB write
FP32_MFMA_PEAK_TFLOPS = 157.3
METRIC = ("paged GQA decode: achieved KV HBM GB/s (% peak) + "
          "seq-tokens/s at M=256")
ROOT = os.path.dirname(os.path.abspath(__file__))


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def pct(x):
    """p10 / median / p90 of a list of durations."""
    a = np.asarray(x, np.float64)
    return {"p10": float(np.percentile(a, 10)), "p50": float(np.median(a)),
            "p90": float(np.percentile(a, 90))}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_m256",
                    choices=["decode_m256", "decode_m32"])
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-forked", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-keys", type=int, default=700000,
                    help="keys in the oracle sample (first sequences of the workload)")
    ap.add_argument("--prefill-steps", type=int, default=10)
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates the "
                         "HBM byte counters) and exit")
    return ap.parse_args()


def copy_probe():
    """A plain device-to-device copy of known size, for scaling the
    FETCH_SIZE / WRITE_SIZE counters: 1 GiB read + 1 GiB written per launch."""
    import torch
    n = (1 << 30) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                      "launches": 3}), flush=True)


class HistoryFiller:
    """Generates each sequence's seeded history into reusable pinned buffers
    on worker threads and appends it through the library."""

    def __init__(self, wl, max_rows, workers=8):
        import torch
        from concurrent.futures import ThreadPoolExecutor
        self.torch = torch
        self.wl = wl
        self.workers = workers
        pin = torch.cuda.is_available()
        self.bufs = []
        for _ in range(workers):
            k = torch.empty((max_rows, wl.kv_dim), dtype=torch.float32, pin_memory=pin)
            v = torch.empty((max_rows, wl.kv_dim), dtype=torch.float32, pin_memory=pin)
            self.bufs.append((k, v))
        self.ex = ThreadPoolExecutor(max_workers=workers)

    def fill(self, pool, seqs, n_rows, layer=0):
        torch = self.torch
        W = self.workers
        kd = torch.empty((max(n_rows), self.wl.kv_dim), device="cuda")
        vd = torch.empty_like(kd)
        for base in range(0, len(seqs), W):
            idx = list(range(base, min(base + W, len(seqs))))
            futs = [self.ex.submit(self.wl.history, r,
                                   (self.bufs[i][0].numpy(), self.bufs[i][1].numpy()))
                    for i, r in enumerate(idx)]
            for i, (r, f) in enumerate(zip(idx, futs)):
                f.result()
                n = int(n_rows[r])
                kd[:n].copy_(self.bufs[i][0][:n], non_blocking=True)
                vd[:n].copy_(self.bufs[i][1][:n], non_blocking=True)
                pool.ensure_append([seqs[r]], n, check=True)
                pool.append_layer([seqs[r]], n, layer, kd[:n], vd[:n], check=True)
                pool.advance([seqs[r]], n, check=True)
                torch.cuda.synchronize()  # pinned buffer i is reused next round
            if base % (8 * W) == 0:
                log("history %d/%d" % (idx[-1] + 1, len(seqs)))
        del kd, vd

    def close(self):
        self.ex.shutdown()


def kernel_code_digest(*paths):
    """SHA-256 of source files with their comments and blank space removed, so
    that the digest changes with the code and not with its comments."""
    import re
    parts = []
    for path in paths:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        parts.append(" ".join(text.split()))
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()


# The device work of a launch: the kernels, and the host code that plans and
# launches them (split sizes, item order, grids).
DEVICE_CODE = ("kernels.hip", "device.hpp", "api.cpp")


def device_code_digest(csrc=None):
    csrc = csrc or os.path.join(ROOT, "paged_kv_gqa_layer_amd", "csrc")
    return kernel_code_digest(*[os.path.join(csrc, f) for f in DEVICE_CODE])


def traffic_for(kernel_name, algorithmic_bytes_per_launch):
    """HBM bytes per launch implied by the committed rocprofv3 counter summary
    (its calibrated FETCH_SIZE + WRITE_SIZE over the algorithmic bytes of the
    profiled launches, times this run's algorithmic bytes per launch), if it
    was taken on the current device code (comments aside); else None."""
    path = os.path.join(ROOT, "profiles", "%s_traffic.json" % kernel_name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("device_code_sha256") != device_code_digest():
        return None
    return t["traffic_over_algorithmic"] * algorithmic_bytes_per_launch


def bench_decode(args, synth, pkv):
    import torch
    mk = synth.decode_m256 if args.workload == "decode_m256" else synth.decode_m32
    n_steps = args.warmup + args.steps
    # head-room for the plain run, the rotary run and the verify runs
    wl = mk(max_steps=3 * n_steps + COLD_STEPS + 1 +
            VERIFY_ROWS_MAX * (n_steps + 2) * len(VERIFY_NQ))
    H, G, D = wl.n_heads, wl.n_kv_heads, wl.head_dim
    M = wl.M
    log("workload %s: M=%d, cached rows %d..%d (sum %d), pool %d blocks (%.2f GB)"
        % (wl.name, M, wl.ctx.min(), wl.ctx.max(), wl.ctx.sum(), wl.n_blocks,
           pkv.pool_storage_bytes(wl.n_blocks, 16, 1, G, D) / 1e9))
    pool = pkv.Pool(wl.n_blocks, wl.block_size, 1, G, D, max_seqs=M + 8)
    pool.set_free_order(wl.free_order())
    seqs = [pool.seq_new(wl.max_tokens) for _ in range(M)]
    t0 = time.time()
    filler = HistoryFiller(wl, int(wl.ctx.max()))
    filler.fill(pool, seqs, wl.ctx)
    filler.close()
    log("history appended in %.1fs" % (time.time() - t0))

    # step inputs, resident in HBM before timing
    steps = []
    for t in range(n_steps):
        q, k, v = wl.step(t)
        steps.append(tuple(torch.from_numpy(x).cuda() for x in (q, k, v)))
    out = torch.empty((M, H * D), device="cuda")
    seqs_np = np.asarray(seqs, np.int32)
    # workspace for the longest step (contexts grow by one row per step); an
    # upper bound for any split of at least 128 keys
    wsb = int(sum(math.ceil((int(c) + 3 * n_steps + COLD_STEPS + 1) / 128)
                  for c in wl.ctx)) * H * (D + 2) * 4
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    scale = wl.scale

    def step(t):
        q, k, v = steps[t % n_steps]
        pool.ensure_append(seqs_np, 1, check=True)
        pool.append_layer(seqs_np, 1, 0, k, v, check=True)
        pool.attn_paged_decode(seqs_np, 0, H, G, D, q, scale, out, ws=ws, check=True)
        pool.advance(seqs_np, 1, check=True)

    def run(t_first, kernels=None):
        """warmup + timed steps from step index t_first (rows cached before
        step t: ctx + t); the library times the launches of `kernels` (ids,
        None: all) with HIP events on its stream."""
        # warm-up steps carry the timing events too: the first timed launches
        # of a process have stalled the host once for ~35 ms (HIP runtime
        # set-up), which must not land in the timed steps
        pool.profile_kernels(kernels)
        pool.profile_enable(True)
        for t in range(t_first, t_first + args.warmup):
            step(t)
        torch.cuda.synchronize()
        pool.profile_enable(True)  # clears the warm-up's totals
        # per-step GPU time: events on the stream the library is given
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record()
        for i, t in enumerate(range(t_first + args.warmup, t_first + n_steps)):
            step(t)
            ev[i + 1].record()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
        kv_bytes = 0
        for t in range(t_first + args.warmup, t_first + n_steps):
            kv_bytes += int((wl.ctx.astype(np.int64) + t + 1).sum()) * 2 * wl.kv_dim * 4
        kern = {}
        for name, kid in (("append", pkv.K_APPEND), ("decode", pkv.K_DECODE),
                          ("merge", pkv.K_MERGE), ("cow", pkv.K_COW)):
            ms, n = pool.profile_read(kid)
            kern[name] = {"launches": n, "avg_us": (1e3 * ms / n) if n else 0.0}
        dec_us = 1e3 * pool.profile_samples(pkv.K_DECODE)
        pool.profile_enable(False)
        pool.profile_kernels(None)
        dec_s = kern["decode"]["avg_us"] * 1e-6 * kern["decode"]["launches"]
        return {"elapsed": elapsed, "kv_bytes": kv_bytes, "kern": kern,
                "gbs": kv_bytes / elapsed / 1e9, "achieved": kv_bytes / dec_s / 1e9,
                "step_ms_pct": pct(step_ms), "decode_us_pct": pct(dec_us)}

    # Headline: only the decode kernel carries timing events (each timed
    # launch adds two event records to the stream, ~5-10 us per step).
    r = run(0, kernels=[pkv.K_DECODE])
    res = dict(r, wl=wl, pool=pool, seqs=seqs,
               seq_tok_s=M * args.steps / r["elapsed"],
               kernel_name=pool.kernel_name(pkv.K_DECODE))
    log("decode: %.3f ms/step, %.0f GB/s step, kernel %.1f us avg -> %.0f GB/s (%.1f%% of peak)"
        % (1e3 * r["elapsed"] / args.steps, r["gbs"], r["kern"]["decode"]["avg_us"],
           r["achieved"], 100 * r["achieved"] / HBM_PEAK_GBS))

    # The same steps with every kernel timed: the per-kernel breakdown.
    rb = run(n_steps)
    res["breakdown"] = {
        "ms_per_step": 1e3 * rb["elapsed"] / args.steps,
        "kernels_us": {k: v["avg_us"] for k, v in rb["kern"].items()},
        "step": "as the headline step, every kernel launch timed",
    }
    log("decode, all kernels timed: %.3f ms/step, append %.1f us, decode %.1f us, merge %.1f us"
        % (res["breakdown"]["ms_per_step"], rb["kern"]["append"]["avg_us"],
           rb["kern"]["decode"]["avg_us"], rb["kern"]["merge"]["avg_us"]))

    # The same steps with rotary embedding fused in (K turned in the append
    # scatter, Q at load in the decode kernel), base 10000.
    rope = pkv.Rope(D, math.log(10000.0), wl.max_tokens)
    pool.set_rope(rope)
    rr = run(2 * n_steps)
    pool.set_rope(None)
    res["rope"] = {
        "ms_per_step": 1e3 * rr["elapsed"] / args.steps,
        "gbs": rr["gbs"], "kernel_gbs": rr["achieved"],
        "kernels_us": {k: v["avg_us"] for k, v in rr["kern"].items()},
        "step_cost_vs_plain": (rb["gbs"] / rr["gbs"]) - 1.0,
        "step": "as the headline step with a rotary table set (neox, base 1e4), "
                "every kernel timed (compare with kernel_breakdown)",
    }
    log("decode + rope: %.3f ms/step, %.0f GB/s step, append %.1f us, decode %.1f us"
        % (1e3 * rr["elapsed"] / args.steps, rr["gbs"], rr["kern"]["append"]["avg_us"],
           rr["kern"]["decode"]["avg_us"]))

    # Cache-cold steps: before each, a 1 GiB read evicts the L2s and the
    # 256 MB Infinity Cache (clean lines, so the step pays no write-back of
    # the eviction), and no step reads K/V left there by the previous one;
    # only the step itself is inside the events.
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    flush.sum()
    t_first = 3 * n_steps
    pool.profile_kernels([pkv.K_DECODE])
    pool.profile_enable(True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(COLD_STEPS)]
    cold_bytes = []
    for i in range(COLD_STEPS):
        flush.sum()
        ev[i][0].record()
        step(t_first + i)
        ev[i][1].record()
        cold_bytes.append(int((wl.ctx.astype(np.int64) + t_first + i + 1).sum())
                          * 2 * wl.kv_dim * 4)
    torch.cuda.synchronize()
    cold_ms = [a.elapsed_time(b) for a, b in ev]
    cold_dec = 1e3 * pool.profile_samples(pkv.K_DECODE)
    pool.profile_enable(False)
    pool.profile_kernels(None)
    del flush
    res["cold"] = {
        "steps": COLD_STEPS,
        "step_ms_percentiles": pct(cold_ms),
        "decode_kernel_us_percentiles": pct(cold_dec),
        "kernel_gbs_median": float(np.median(np.asarray(cold_bytes) /
                                             (np.asarray(cold_dec) * 1e-6) / 1e9)),
        "note": "each step preceded by a 1 GiB device read (outside the events)",
    }
    log("decode, cache-cold: step p50 %.3f ms, kernel p50 %.1f us -> %.0f GB/s"
        % (res["cold"]["step_ms_percentiles"]["p50"],
           res["cold"]["decode_kernel_us_percentiles"]["p50"], res["cold"]["kernel_gbs_median"]))
    if not args.no_verify:
        res["verify"] = [bench_verify(args, wl, pool, seqs, n_q, pkv, torch)
                         for n_q in VERIFY_NQ]
    return res


def bench_verify(args, wl, pool, seqs, n_q, pkv, torch):
    """Speculative-decode verify steps on the same pool: every sequence
    appends n_q drafted rows and attends them in one call (offset-causal),
    then keeps a seeded 1..n_q of them and rewinds the rest (truncate)."""
    H, G, D, M = wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.M
    n_steps = args.warmup + args.steps
    rng = np.random.default_rng(1000 + n_q)
    gen = np.random.default_rng(2000 + n_q)
    Q = torch.from_numpy(gen.standard_normal((M * n_q, H * D), dtype=np.float32)).cuda()
    K = torch.from_numpy(gen.standard_normal((M * n_q, G * D), dtype=np.float32)).cuda()
    V = torch.from_numpy(gen.standard_normal((M * n_q, G * D), dtype=np.float32)).cuda()
    out = torch.empty_like(Q)
    seqs_np = np.asarray(seqs, np.int32)
    max_len = max(pool.seq_len(s) for s in seqs) + n_q * (n_steps + 1)
    ws = torch.empty(M * math.ceil(max_len / 128) * n_q * H * (D + 2) * 4,
                     dtype=torch.uint8, device="cuda")
    accept = rng.integers(1, n_q + 1, size=(n_steps, M))

    def step(t):
        pool.ensure_append(seqs_np, n_q, check=True)
        pool.append_layer(seqs_np, n_q, 0, K, V, check=True)
        pool.attn_paged_verify(seqs_np, n_q, 0, H, G, D, Q, wl.scale, out, ws=ws,
                               check=True)
        pool.advance(seqs_np, n_q, check=True)
        for r, s in enumerate(seqs):
            pool.seq_truncate(s, lens[r] + int(accept[t, r]), check=True)
            lens[r] += int(accept[t, r])

    lens = [pool.seq_len(s) for s in seqs]
    pool.profile_enable(True)  # warm-up with the timing events on (see run())
    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    kv_bytes = 0
    for t in range(args.warmup, n_steps):
        kv_bytes += (sum(lens) + int(accept[args.warmup:t].sum()) + M * n_q) * 2 * wl.kv_dim * 4
    pool.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.warmup, n_steps):
        step(t)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern = {}
    for name, kid in (("append", pkv.K_APPEND), ("verify", pkv.K_VERIFY),
                      ("merge", pkv.K_MERGE), ("cow", pkv.K_COW)):
        ms, n = pool.profile_read(kid)
        kern[name] = (1e3 * ms / n) if n else 0.0
    pool.profile_enable(False)
    ver_s = kern["verify"] * 1e-6 * args.steps
    res = {
        "n_q": n_q, "ms_per_step": 1e3 * elapsed / args.steps,
        "gbs": kv_bytes / elapsed / 1e9, "kernel_gbs": kv_bytes / ver_s / 1e9,
        "kernels_us": kern,
        "accepted_tokens_per_s": float(accept[args.warmup:].sum()) / elapsed,
        "step": "ensure_append(n_q) + append_layer + attn_paged_verify + advance "
                "+ truncate to 1..n_q accepted",
    }
    log("verify n_q=%d: %.3f ms/step, %.0f GB/s step, kernel %.1f us -> %.0f GB/s, merge %.1f us"
        % (n_q, res["ms_per_step"], res["gbs"], kern["verify"], res["kernel_gbs"],
           kern["merge"]))
    return res


def bench_forked(args, synth, pkv, shared):
    """The forked batch: one 2048-row prefix forked into 64 sequences (the
    parent then freed, so every prefix block has 64 references), each
    decoding its own token stream with pkv_attn_paged_decode or (shared)
    pkv_attn_paged_decode_shared; then the rewind half: the even forks
    truncate back to the fork point and replay their odd partner's stream,
    every replayed output compared bit for bit with the partner's.

    Both halves time their steps after `warmup` with no timing event in
    them (at ~0.05 ms per step, the two event records of a timed launch are
    a tenth of the step); a second run of the decode half with every launch
    timed by HIP events gives the per-kernel breakdown and the attention
    kernel's durations.
    Reports logical KV bytes (every sequence's visible keys) and unique
    bytes (the prefix once + each sequence's own rows) per second."""
    import torch
    wl = synth.forked_2048x64()
    H, G, D, F = wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.n_forks
    kv_row = 2 * wl.kv_dim * 4

    def step_inputs(t):
        xs = [wl.fork_step(f, t) for f in range(F)]
        return tuple(np.stack([x[i] for x in xs]) for i in range(3))
    inputs = [tuple(torch.from_numpy(a).cuda() for a in x)
              for x in synth.parallel_map(step_inputs, range(wl.steps))]
    # the odd forks' inputs, replayed by the even forks in the rewind half
    odd_inputs = [tuple(a[1::2].contiguous() for a in x) for x in inputs]
    attn_id = pkv.K_PREFIX if shared else pkv.K_DECODE

    def run(kernels, rewind):
        pool = pkv.Pool(wl.n_blocks, wl.block_size, 1, G, D, max_seqs=F + 8)
        pool.set_free_order(wl.free_order())
        parent = pool.seq_new(wl.max_tokens)
        pk, pv = wl.prefix_kv()
        pool.ensure_append([parent], wl.prefix, check=True)
        pool.append_layer([parent], wl.prefix, 0, torch.from_numpy(pk).cuda(),
                          torch.from_numpy(pv).cuda(), check=True)
        pool.advance([parent], wl.prefix, check=True)
        forks = [pool.seq_fork(parent) for _ in range(F)]
        pool.seq_free(parent, check=True)
        seqs_np = np.asarray(forks, np.int32)
        evens_np = seqs_np[0::2].copy()
        outs = torch.empty((wl.steps, F, H * D), device="cuda")
        # workspace: the library's own count for this batch, doubled for the
        # rows the forks add over the steps (a few more splits at most)
        ws_bytes = max(pool.decode_workspace_bytes(seqs_np, H),
                       pool.decode_shared_workspace_bytes(seqs_np, H))
        ws = torch.empty(2 * ws_bytes + 4, dtype=torch.uint8, device="cuda")
        attn = pool.attn_paged_decode_shared if shared else pool.attn_paged_decode

        def step(batch, inp, out):
            q, k, v = inp
            pool.ensure_append(batch, 1, check=True)
            pool.append_layer(batch, 1, 0, k, v, check=True)
            attn(batch, 0, H, G, D, q, wl.scale, out, ws=ws, check=True)
            pool.advance(batch, 1, check=True)

        def timed(batch, inps, outs_):
            w = min(args.warmup, wl.steps - 1)
            pool.profile_kernels(kernels)
            pool.profile_enable(True)  # warm-up with the timing events on
            for t in range(w):
                step(batch, inps[t], outs_[t])
            torch.cuda.synchronize()
            pool.profile_enable(True)
            t0 = time.perf_counter()
            for t in range(w, wl.steps):
                step(batch, inps[t], outs_[t])
            torch.cuda.synchronize()
            elapsed = time.perf_counter() - t0
            kern = {}
            for name, kid in (("append", pkv.K_APPEND), ("shared_decode", pkv.K_PREFIX),
                              ("decode", pkv.K_DECODE), ("merge", pkv.K_MERGE),
                              ("cow", pkv.K_COW)):
                ms, n = pool.profile_read(kid)
                if n:
                    kern[name] = 1e3 * ms / n
            att_us = 1e3 * pool.profile_samples(attn_id) if kernels != [] else None
            pool.profile_enable(False)
            pool.profile_kernels(None)
            return w, elapsed, kern, att_us

        w, el, kern, att_us = timed(seqs_np, inputs, outs)
        n = wl.steps - w
        logical = sum(F * (wl.prefix + t + 1) for t in range(w, wl.steps)) * kv_row
        unique = sum(wl.prefix + F * (t + 1) for t in range(w, wl.steps)) * kv_row
        res = {
            "ms_per_step": 1e3 * el / n, "steps": n,
            "logical_gbs": logical / el / 1e9, "unique_gbs": unique / el / 1e9,
            "seq_tokens_per_s": F * n / el, "kernels_us": kern,
            "attention_kernel": pool.kernel_name(attn_id),
        }
        if att_us is not None:
            res["attention_kernel_us_percentiles"] = pct(att_us)
        if not rewind:
            pool.close()
            return res
        # rewind half: even forks go back to the fork point and replay the
        # odd forks' streams
        for s in evens_np:
            pool.seq_truncate(int(s), wl.prefix, check=True)
        routs = torch.empty((wl.steps, F // 2, H * D), device="cuda")
        w, el, kern, att_us = timed(evens_np, odd_inputs, routs)
        torch.cuda.synchronize()
        same = [bool(torch.equal(routs[t].view(torch.int32),
                                 outs[t, 1::2].contiguous().view(torch.int32)))
                for t in range(wl.steps)]
        n = wl.steps - w
        R = F // 2
        res["rewind"] = {
            "ms_per_step": 1e3 * el / n, "steps": n, "sequences": R,
            "logical_gbs": sum(R * (wl.prefix + t + 1) for t in range(w, wl.steps))
            * kv_row / el / 1e9,
            "unique_gbs": sum(wl.prefix + R * (t + 1) for t in range(w, wl.steps))
            * kv_row / el / 1e9,
            "bitwise_equal_steps": int(sum(same)), "checked_steps": wl.steps,
            "step": "even forks truncated to the fork point, then ensure_append + "
                    "append_layer + attention + advance on the odd partner's inputs",
        }
        pool.close()
        return res

    res = run([], rewind=True)
    del res["kernels_us"]
    res.update({"workload": wl.name, "forks": F, "prefix": wl.prefix,
                "step": "ensure_append + append_layer + %s + advance"
                        % ("attn_paged_decode_shared" if shared else "attn_paged_decode")})
    bd = run(None, rewind=False)
    res["attention_kernel_us_percentiles"] = bd["attention_kernel_us_percentiles"]
    res["breakdown"] = {"ms_per_step": bd["ms_per_step"], "kernels_us": bd["kernels_us"],
                        "step": "as the decode half, every kernel launch timed"}
    log("forked%s: %.4f ms/step, logical %.0f GB/s, unique %.0f GB/s, %s p50 %.1f us; "
        "rewind %.4f ms/step, bitwise %d/%d; all timed %.4f ms/step %s"
        % (" shared" if shared else "", res["ms_per_step"], res["logical_gbs"],
           res["unique_gbs"], res["attention_kernel"],
           res["attention_kernel_us_percentiles"]["p50"], res["rewind"]["ms_per_step"],
           res["rewind"]["bitwise_equal_steps"], res["rewind"]["checked_steps"],
           bd["ms_per_step"], json.dumps(bd["kernels_us"])))
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(args, wl, oracle):
    """Time the oracle on a sample of the same workload (decode step 0 of the
    first sequences: every cached row plus the new one): once on one thread,
    then the same sample split over every host core available to this process
    (one oracle call per sequence per thread; the C oracle runs without the
    interpreter lock).  The sample is the first sequences up to ~700K keys."""
    from concurrent.futures import ThreadPoolExecutor
    q_all, k_all, v_all = wl.step(0)
    H, G, D = wl.n_heads, wl.n_kv_heads, wl.head_dim
    sample, keys = [], 0
    for r in range(wl.M):
        kh, vh = wl.history(r)
        sample.append((r, np.concatenate([kh, k_all[r:r + 1]]),
                       np.concatenate([vh, v_all[r:r + 1]])))
        keys += sample[-1][1].shape[0]
        if keys >= args.cpu_keys:
            break
    kvb = keys * wl.kv_dim * 2 * 4

    def one(item):
        r, K, V = item
        rc, _ = oracle.attn_contig(q_all[r:r + 1], K, V, H, G, D, True, wl.scale)
        assert rc == 0

    t0 = time.perf_counter()
    for item in sample:
        one(item)
    t1 = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=cores) as ex:
        list(ex.map(one, sample))
    tn = time.perf_counter() - t0
    log("cpu oracle: %d sequences (%d keys): %.2fs on one thread, %.2fs on %d threads"
        % (len(sample), keys, t1, tn, cores))
    return {
        "value": kvb / tn / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": "decode step of sequences 0..%d of %d (%d keys), one oracle call per "
                  "sequence per thread" % (len(sample) - 1, wl.M, keys),
        "seq_tokens_per_s": len(sample) / tn,
        "one_thread": {"value": kvb / t1 / 1e9, "unit": "GB/s", "cores": 1,
                       "seq_tokens_per_s": len(sample) / t1},
        "cpu_model": cpu_model(),
    }


def cpu_baseline_prefill(synth, oracle, n_last=64):
    """The oracle on a sample of the prefill workload: the last n_last chunk
    queries of every sequence (each sees ~4K keys), cut into (sequence,
    query head) units -- one oracle call per unit over that head's queries
    and its kv head's K/V columns -- run once on one thread, then over every
    host core available to this process.  Reported in TFLOP/s of the same
    algorithmic flops as the kernel (4 * D per visible key and head)."""
    from concurrent.futures import ThreadPoolExecutor
    wl = synth.prefill_8x3584p512()
    H, G, D = wl.n_heads, wl.n_kv_heads, wl.head_dim
    group = H // G
    units = []
    for r in range(wl.M):
        kh, vh = wl.history(r)
        q, k, v = wl.chunk_inputs(r)
        K = np.concatenate([kh, k])
        V = np.concatenate([vh, v])
        for h in range(H):
            c = h // group
            units.append((np.ascontiguousarray(q[-n_last:, h * D:(h + 1) * D]),
                          np.ascontiguousarray(K[:, c * D:(c + 1) * D]),
                          np.ascontiguousarray(V[:, c * D:(c + 1) * D])))
    total_k = wl.cached + wl.chunk
    flops = wl.M * sum(4 * D * H * (total_k - n_last + i + 1) for i in range(n_last))

    def one(item):
        q, K, V = item
        rc, _ = oracle.attn_contig(q, K, V, 1, 1, D, True, wl.scale)
        assert rc == 0

    t0 = time.perf_counter()
    for item in units:
        one(item)
    t1 = time.perf_counter() - t0
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=cores) as ex:
        list(ex.map(one, units))
    tn = time.perf_counter() - t0
    log("cpu oracle, prefill: %d (sequence, head) units: %.2fs on one thread, %.2fs on %d threads"
        % (len(units), t1, tn, cores))
    return {
        "value": flops / tn / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": "last %d chunk queries of each of the %d sequences (%.2e flop), as %d "
                  "(sequence, query head) oracle calls over the host cores"
                  % (n_last, wl.M, flops, len(units)),
        "one_thread": {"value": flops / t1 / 1e12, "unit": "TFLOP/s", "cores": 1},
    }


def bench_decode_small(args, synth, pkv):
    """The M=32 decode workload (contexts 512-4096): the headline step at a
    small batch.  The step time comes from steps that carry no timing event
    (at this size two event records per step are several percent of it);
    the decode kernel's time from the steps that follow, its launches timed
    by HIP events."""
    import torch
    n_steps = args.warmup + args.steps
    wl = synth.decode_m32(max_steps=2 * n_steps + 1)
    H, G, D, M = wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.M
    pool = pkv.Pool(wl.n_blocks, wl.block_size, 1, G, D, max_seqs=M + 8)
    pool.set_free_order(wl.free_order())
    seqs = [pool.seq_new(wl.max_tokens) for _ in range(M)]
    filler = HistoryFiller(wl, int(wl.ctx.max()))
    filler.fill(pool, seqs, wl.ctx)
    filler.close()
    steps = [tuple(torch.from_numpy(x).cuda() for x in wl.step(t)) for t in range(n_steps)]
    out = torch.empty((M, H * D), device="cuda")
    seqs_np = np.asarray(seqs, np.int32)
    wsb = int(sum(math.ceil((int(c) + 2 * n_steps + 1) / 128) for c in wl.ctx)) * H * (D + 2) * 4
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")

    def step(t):
        q, k, v = steps[t % n_steps]
        pool.ensure_append(seqs_np, 1, check=True)
        pool.append_layer(seqs_np, 1, 0, k, v, check=True)
        pool.attn_paged_decode(seqs_np, 0, H, G, D, q, wl.scale, out, ws=ws, check=True)
        pool.advance(seqs_np, 1, check=True)

    def timed(t_first, kernels):
        pool.profile_kernels(kernels)
        pool.profile_enable(True)  # warm-up with the timing events on (see run())
        for t in range(t_first, t_first + args.warmup):
            step(t)
        torch.cuda.synchronize()
        pool.profile_enable(True)
        t0 = time.perf_counter()
        for t in range(t_first + args.warmup, t_first + n_steps):
            step(t)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    elapsed = timed(0, [])
    kernel_elapsed = timed(n_steps, [pkv.K_DECODE])
    ms, n = pool.profile_read(pkv.K_DECODE)
    dec_us = 1e3 * pool.profile_samples(pkv.K_DECODE)
    kname = pool.kernel_name(pkv.K_DECODE)
    pool.profile_enable(False)
    pool.close()
    def kv(t0, t1):
        return sum(int((wl.ctx.astype(np.int64) + t + 1).sum()) * 2 * wl.kv_dim * 4
                   for t in range(t0, t1))
    kv_bytes = kv(args.warmup, n_steps)
    kv_kernel = kv(n_steps + args.warmup, 2 * n_steps)
    res = {
        "workload": wl.name, "M": M, "ms_per_step": 1e3 * elapsed / args.steps,
        "gbs": kv_bytes / elapsed / 1e9, "pct_hbm_peak": 100 * kv_bytes / elapsed / 1e9
        / HBM_PEAK_GBS, "seq_tokens_per_s": M * args.steps / elapsed,
        "kernel_timed_ms_per_step": 1e3 * kernel_elapsed / args.steps,
        "kernel_us": 1e3 * ms / n, "kernel_gbs": kv_kernel / (ms * 1e-3) / 1e9,
        "kernel": kname, "decode_kernel_us_percentiles": pct(dec_us),
        "step": "ensure_append + append_layer + attn_paged_decode + advance; "
                "ms_per_step from steps without timing events, kernel_* from the "
                "next steps with the decode launches timed (kernel_timed_ms_per_step)",
    }
    log("decode M=32: %.4f ms/step, %.0f GB/s step; decode-timed steps %.4f ms, kernel "
        "%.1f us -> %.0f GB/s" % (res["ms_per_step"], res["gbs"],
                                  res["kernel_timed_ms_per_step"], res["kernel_us"],
                                  res["kernel_gbs"]))
    return res


def bench_prefill(args, synth, pkv):
    import torch
    wl = synth.prefill_8x3584p512()
    H, G, D, M = wl.n_heads, wl.n_kv_heads, wl.head_dim, wl.M
    pool = pkv.Pool(wl.n_blocks, wl.block_size, 1, G, D, max_seqs=M + 4)
    pool.set_free_order(wl.free_order())
    seqs = [pool.seq_new(wl.max_tokens) for _ in range(M)]
    filler = HistoryFiller(wl, wl.cached)
    filler.fill(pool, seqs, [wl.cached] * M)
    filler.close()
    Q = torch.empty((M * wl.chunk, H * D), device="cuda")
    K = torch.empty((M * wl.chunk, G * D), device="cuda")
    V = torch.empty_like(K)
    for r in range(M):
        q, k, v = wl.chunk_inputs(r)
        Q[r * wl.chunk:(r + 1) * wl.chunk].copy_(torch.from_numpy(q))
        K[r * wl.chunk:(r + 1) * wl.chunk].copy_(torch.from_numpy(k))
        V[r * wl.chunk:(r + 1) * wl.chunk].copy_(torch.from_numpy(v))
    out = torch.empty_like(Q)
    seqs_np = np.asarray(seqs, np.int32)

    def step():
        pool.ensure_append(seqs_np, wl.chunk, check=True)
        pool.append_layer(seqs_np, wl.chunk, 0, K, V, check=True)
        pool.attn_paged_prefill(seqs_np, wl.chunk, 0, H, G, D, Q, True, wl.scale,
                                out, check=True)
        for s in seqs:  # rewind so the next step appends the same chunk
            pool.seq_truncate(s, wl.cached, check=True)

    pool.profile_enable(True)  # warm-up with the timing events on (see run())
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    pool.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.prefill_steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms, n = pool.profile_read(pkv.K_PREFILL)
    kern_ms = pool.profile_samples(pkv.K_PREFILL)
    kname = pool.kernel_name(pkv.K_PREFILL)
    pool.profile_enable(False)
    visible = M * sum(wl.cached + i + 1 for i in range(wl.chunk))
    flops = 4 * D * H * visible
    # bytes the launch must move: Q read and out written, K/V of every row read
    unique_bytes = (2 * M * wl.chunk * H * D + M * (wl.cached + wl.chunk) * 2 * G * D) * 4
    kern_s = ms * 1e-3 / n
    tf = flops / kern_s / 1e12
    log("prefill: step %.3f ms, kernel %.3f ms -> %.1f TFLOP/s (%.1f%% of FP32 MFMA peak)"
        % (1e3 * elapsed / args.prefill_steps, 1e3 * kern_s, tf,
           100 * tf / FP32_MFMA_PEAK_TFLOPS))
    pool.close()
    return {
        "workload": wl.name, "ms_per_step": 1e3 * elapsed / args.prefill_steps,
        "steps": args.prefill_steps,
        "step": "ensure_append(512) + append_layer + attn_paged_prefill + truncate",
        "kernel_ms": 1e3 * kern_s, "flops_per_step": flops,
        "kernel_ms_percentiles": pct(kern_ms),
        "roofline": {"bound": "mfma", "achieved": tf, "peak": FP32_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tf / FP32_MFMA_PEAK_TFLOPS,
                     "traffic": traffic_for("prefill_mfma_kernel", unique_bytes),
                     "kernel": kname, "unique_bytes_per_launch": unique_bytes},
    }


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE %d)" % (args.gpus, world),
              file=sys.stderr, flush=True)
        sys.exit(2)
    sys.path.insert(0, ROOT)
    import torch
    import paged_kv_gqa_layer_amd as pkv
    import synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    pkv.lib()  # fail loudly if the HIP library is not built

    d = bench_decode(args, synth, pkv)
    wl = d["wl"]
    traffic = traffic_for("decode_fast_kernel", d["kv_bytes"] / args.steps)
    line = {
        "metric": METRIC,
        "value": d["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": 1e3 * d["elapsed"] / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "M": wl.M, "n_heads": wl.n_heads,
            "n_kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim,
            "block_size": wl.block_size, "layers": 1,
            "context_rows": [int(wl.ctx.min()), int(wl.ctx.max())],
            "mean_total_k": float(wl.ctx.mean() + 1 + args.warmup + (args.steps - 1) / 2),
            "split_keys": "256 / 512 / 1024 / 2048 for rows below 2048 / 6144 / 8192 / above",
            "placement": "random permutation",
            "step": "ensure_append + append_layer + attn_paged_decode + advance",
        },
        "seq_tokens_per_s": d["seq_tok_s"],
        "pct_hbm_peak": 100.0 * d["gbs"] / HBM_PEAK_GBS,
        "kv_bytes_per_step": d["kv_bytes"] / args.steps,
        "kernels_us": {k: v["avg_us"] for k, v in d["kern"].items() if v["launches"]},
        "step_ms_percentiles": d["step_ms_pct"],
        "decode_kernel_us_percentiles": d["decode_us_pct"],
        "kernel_breakdown": d["breakdown"],
        "rope": d["rope"],
        "cold": d["cold"],
        "verify": d.get("verify"),
        "roofline": {
            "bound": "hbm", "achieved": d["achieved"], "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": d["achieved"] / HBM_PEAK_GBS,
            "traffic": (traffic if traffic is not None else None),
            "kernel": d["kernel_name"],
            "bytes_per_launch": d["kv_bytes"] / args.steps,
        },
    }
    d["pool"].close()
    del d
    torch.cuda.empty_cache()
    if args.workload == "decode_m256":
        line["decode_m32"] = bench_decode_small(args, synth, pkv)
    if not args.no_prefill:
        line["prefill"] = bench_prefill(args, synth, pkv)
    if not args.no_forked:
        line["forked"] = bench_forked(args, synth, pkv, shared=False)
        line["forked_shared_prefix"] = bench_forked(args, synth, pkv, shared=True)
    if not args.no_cpu_baseline:
        import oracle
        line["cpu_baseline"] = cpu_baseline(args, wl, oracle)
        if not args.no_prefill:
            line["prefill"]["cpu_baseline"] = cpu_baseline_prefill(synth, oracle)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

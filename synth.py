"""Seeded synthetic inputs for paged-KV grouped-query attention.

This module only draws numbers: lengths, block placements and Q/K/V arrays.
It holds none of the attention or pool arithmetic, and it is the only code
that both the CPU oracle's callers and the HIP path's callers share.

Workloads (all synthetic; no dataset or trained weights are involved):

* tiny gate -- the pages' own exact-regime inputs ("nx_paged_kv_gate.nx
  source", the pg_lcg / pg_fill helpers and the fill order in main): a
  31-bit LCG s <- (s * 1103515245 + 12345) mod 2^31, each value
  (s mod 17) - 8 as a float, seed 20260709.
* Qwen3-4B-shaped attention ("nx_f32_gqa_attention.nx source", header: 32
  query heads share 8 kv heads, q_out 4096 / kv_out 1024, so head_dim 128):
  - decode, M=32, context lengths uniform on {512..4096};
  - decode, M=256, context lengths log-uniform on [1024, 16384];
  - chunked prefill, 8 sequences x (3584 cached + 512 new rows);
  - forked batch, one 2048-row prefix forked into 64 sequences.
  Values are N(0, sigma) float32 drawn per sequence from
  numpy.random.default_rng([seed, stream, index]) so that any one sequence
  can be regenerated on its own.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

QWEN3_4B_ATTN = dict(n_heads=32, n_kv_heads=8, head_dim=128)
BLOCK = 16

# stream tags for numpy SeedSequence entropy lists
_S_LEN, _S_PLACE, _S_HIST, _S_STEP = 0, 1, 2, 3


# --------------------------------------------------------------------------
# The pages' LCG (exact small integers in [-8, 8])
# --------------------------------------------------------------------------

class PagesLCG:
    """Stateful 31-bit LCG with the pages' multiplier, increment and mapping."""

    def __init__(self, seed: int = 20260709):
        self.s = int(seed)

    def fill(self, n: int) -> np.ndarray:
        out = np.empty(n, np.float32)
        s = self.s
        for i in range(n):
            s = (s * 1103515245 + 12345) & 0x7FFFFFFF
            out[i] = float((s % 17) - 8)
        self.s = s
        return out


@dataclasses.dataclass
class TinyGate:
    n_layers: int = 2
    n_heads: int = 4
    n_kv_heads: int = 2
    head_dim: int = 8
    block_size: int = 4
    n_blocks: int = 16
    max_tokens: int = 64
    scale: float = 0.25  # bit pattern 0x3E800000

    @property
    def q_dim(self):
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    def inputs(self):
        """Q/K/V for the three rounds and the two divergent forks, in the
        gate's fill order: (Q1,K1,V1) 5 rows, (Q2,K2,V2) 1 row, (Q3,K3,V3)
        3 rows, (QA,KA,VA) 2 rows, (QB,KB,VB) 2 rows."""
        g = PagesLCG(20260709)
        out = {}
        for name, n in (("1", 5), ("2", 1), ("3", 3), ("A", 2), ("B", 2)):
            q = g.fill(n * self.q_dim).reshape(n, self.q_dim)
            k = g.fill(n * self.kv_dim).reshape(n, self.kv_dim)
            v = g.fill(n * self.kv_dim).reshape(n, self.kv_dim)
            out[name] = (q, k, v)
        return out


# --------------------------------------------------------------------------
# Qwen3-4B-shaped workloads
# --------------------------------------------------------------------------

def _rng(seed, *tags):
    return np.random.default_rng([int(seed)] + [int(t) for t in tags])


def _normal(rng, shape, sigma, out=None):
    """N(0, sigma) float32 of `shape`; written into `out` (a C-contiguous
    float32 array with at least prod(shape) elements) when given, which
    draws exactly the same numbers without allocating."""
    if out is None:
        a = rng.standard_normal(shape, dtype=np.float32)
    else:
        n = int(np.prod(shape))
        a = out.reshape(-1)[:n].reshape(shape)
        rng.standard_normal(out=a, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


@dataclasses.dataclass
class DecodeWorkload:
    """M sequences with cached contexts, each decoding one token per step."""
    name: str
    M: int
    ctx: np.ndarray          # cached rows per sequence before the first step
    seed: int
    sigma: float = 1.0
    n_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    block_size: int = BLOCK
    max_steps: int = 64      # pool head-room for this many decode steps

    @property
    def q_dim(self):
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    @property
    def scale(self):
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def max_tokens(self):
        return int(self.ctx.max()) + self.max_steps + 1

    @property
    def n_blocks(self):
        b = self.block_size
        return int(sum((int(c) + self.max_steps + 1 + b - 1) // b
                       for c in self.ctx)) + self.M

    def free_order(self):
        """Random placement: the order in which the pool hands out ids."""
        return _rng(self.seed, _S_PLACE).permutation(self.n_blocks).astype(np.int64)

    def history(self, r, out=None):
        """(K, V) [ctx[r], kv_dim] float32 for sequence r (into out=(k, v)
        buffers when given)."""
        g = _rng(self.seed, _S_HIST, r)
        n = int(self.ctx[r])
        ok, ov = out if out is not None else (None, None)
        k = _normal(g, (n, self.kv_dim), self.sigma, ok)
        v = _normal(g, (n, self.kv_dim), self.sigma, ov)
        return k, v

    def step(self, t):
        """(Q [M, q_dim], K_new [M, kv_dim], V_new [M, kv_dim]) for step t."""
        g = _rng(self.seed, _S_STEP, t)
        k = _normal(g, (self.M, self.kv_dim), self.sigma)
        v = _normal(g, (self.M, self.kv_dim), self.sigma)
        q = _normal(g, (self.M, self.q_dim), self.sigma)
        return q, k, v

    def step_row(self, t, r):
        """Row r of step t, regenerated alone (same values as step(t)[.][r])."""
        q, k, v = self.step(t)
        return q[r], k[r], v[r]


def decode_m32(seed=2, max_steps=64):
    """M=32 sequences, context uniform on {512..4096}, values N(0,1)."""
    ctx = _rng(seed, _S_LEN).integers(512, 4096, size=32, endpoint=True)
    return DecodeWorkload("decode_m32_ctx512-4096", 32, ctx.astype(np.int64),
                          seed, max_steps=max_steps)


def decode_m256(seed=3, max_steps=64):
    """M=256 sequences, context log-uniform on [1024, 16384], values N(0,1)."""
    u = _rng(seed, _S_LEN).uniform(math.log(1024), math.log(16384), size=256)
    ctx = np.clip(np.round(np.exp(u)), 1024, 16384).astype(np.int64)
    return DecodeWorkload("decode_m256_ctx1k-16k_logu", 256, ctx, seed,
                          max_steps=max_steps)


@dataclasses.dataclass
class PrefillWorkload:
    """Sequences with a cached prefix, each appending and attending a chunk."""
    name: str
    M: int
    cached: int
    chunk: int
    seed: int
    sigma: float = 0.5
    n_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    block_size: int = BLOCK

    @property
    def q_dim(self):
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    @property
    def scale(self):
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def max_tokens(self):
        return self.cached + self.chunk

    @property
    def n_blocks(self):
        b = self.block_size
        return self.M * ((self.cached + self.chunk + b - 1) // b) + self.M

    def free_order(self):
        return _rng(self.seed, _S_PLACE).permutation(self.n_blocks).astype(np.int64)

    def history(self, r, out=None):
        g = _rng(self.seed, _S_HIST, r)
        ok, ov = out if out is not None else (None, None)
        k = _normal(g, (self.cached, self.kv_dim), self.sigma, ok)
        v = _normal(g, (self.cached, self.kv_dim), self.sigma, ov)
        return k, v

    def chunk_inputs(self, r):
        """(Q [chunk, q_dim], K_new [chunk, kv_dim], V_new) for sequence r."""
        g = _rng(self.seed, _S_STEP, r)
        k = _normal(g, (self.chunk, self.kv_dim), self.sigma)
        v = _normal(g, (self.chunk, self.kv_dim), self.sigma)
        q = _normal(g, (self.chunk, self.q_dim), self.sigma)
        return q, k, v


def prefill_8x3584p512(seed=4):
    return PrefillWorkload("prefill_8x(3584+512)", 8, 3584, 512, seed)


@dataclasses.dataclass
class ForkWorkload:
    """One prefix forked into n_forks sequences that then decode separately."""
    name: str
    prefix: int
    n_forks: int
    steps: int
    seed: int
    sigma: float = 1.0
    n_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    block_size: int = BLOCK

    @property
    def q_dim(self):
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    @property
    def scale(self):
        return float(np.float32(1.0 / math.sqrt(self.head_dim)))

    @property
    def max_tokens(self):
        return self.prefix + self.steps

    @property
    def n_blocks(self):
        b = self.block_size
        return ((self.prefix + b - 1) // b
                + self.n_forks * ((self.steps + b - 1) // b + 2) + 8)

    def free_order(self):
        return _rng(self.seed, _S_PLACE).permutation(self.n_blocks).astype(np.int64)

    def prefix_kv(self):
        g = _rng(self.seed, _S_HIST, 0)
        k = _normal(g, (self.prefix, self.kv_dim), self.sigma)
        v = _normal(g, (self.prefix, self.kv_dim), self.sigma)
        return k, v

    def fork_step(self, f, t):
        """(q [q_dim], k [kv_dim], v [kv_dim]) of fork f at decode step t."""
        g = _rng(self.seed, _S_STEP, f, t)
        k = _normal(g, (self.kv_dim,), self.sigma)
        v = _normal(g, (self.kv_dim,), self.sigma)
        q = _normal(g, (self.q_dim,), self.sigma)
        return q, k, v


def forked_2048x64(seed=5, steps=256, prefix=2048):
    return ForkWorkload("fork_2048x64", prefix, 64, steps, seed)


def parallel_map(fn, items, workers=8):
    """Map fn over items with a thread pool (numpy's generators drop the GIL)."""
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(fn, items))

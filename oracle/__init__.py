"""CPU oracle for paged-KV grouped-query attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never loads it; the two share no code.

The arithmetic lives in ``pkv_oracle.c`` (plain C, double accumulation); this
module compiles it with gcc and exposes it through ctypes with numpy arrays.
Every function cites the passage of the pages it follows in the C source.

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_*.py`` against closed forms, the pages' worked example,
the pages' known answers for the pool, invariants and a float64 library
attention routine.  None is left unpinned.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_pkv.so")

OK, BAD_DIM, BAD_GQA, ERR_SEQ, OOM, CAPACITY, BAD_ARG = range(7)


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle_pkv.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = C.CDLL(_LIB)
        P, I, F, I64 = C.c_void_p, C.c_int, C.c_float, C.c_int64
        sig = {
            "pkvo_attn_contig": (I, [P, P, P, I, I, I, I, I, I, F, P]),
            "pkvo_gqa_attention": (I, [P, P, P, I, I, I, I, F, P]),
            "pkvo_cache_new": (P, [I, I, I, I]),
            "pkvo_cache_free": (None, [P]),
            "pkvo_cache_len": (I, [P]),
            "pkvo_cache_advance": (I, [P, I]),
            "pkvo_attn_with_cache": (I, [P, P, P, I, I, I, I, P, I, I, F, P]),
            "pkvo_pool_new": (P, [I, I, I, I, I, I, I]),
            "pkvo_pool_free": (None, [P]),
            "pkvo_alloc_block": (I64, [P]),
            "pkvo_unref_block": (I, [P, I64]),
            "pkvo_set_free_order": (I, [P, P, I]),
            "pkvo_seq_new": (I, [P, I]),
            "pkvo_seq_free": (I, [P, I]),
            "pkvo_seq_fork": (I, [P, I]),
            "pkvo_seq_truncate": (I, [P, I, I]),
            "pkvo_ensure_append": (I, [P, P, I, I]),
            "pkvo_append_layer": (I, [P, P, I, I, I, P, P]),
            "pkvo_advance": (I, [P, P, I, I]),
            "pkvo_attn_paged": (I, [P, P, I, I, I, I, I, I, P, I, F, P]),
            "pkvo_attn_with_paged": (I, [P, P, P, I, I, I, I, P, I, I, I, F, P]),
            "pkvo_seq_len": (I, [P, I]),
            "pkvo_seq_pages": (I, [P, I, P, I]),
            "pkvo_refcounts": (I, [P, P]),
            "pkvo_free_stack": (I, [P, P, I]),
            "pkvo_read_row": (I, [P, I, I, I, P, P]),
            "pkvo_rope": (I, [P, I, I, I, P, C.c_double]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _ids(seqs) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(seqs, dtype=np.int32).reshape(-1))


# --------------------------------------------------------------------------
# Attention definition
# --------------------------------------------------------------------------

def attn_contig(Q, K, V, n_heads, n_kv_heads, head_dim, causal, scale):
    """softmax(Q K^T scale) V over explicit histories K, V [total_k, kv_dim].

    Q is [n_q, n_heads*head_dim]; returns (status, out [n_q, n_heads*head_dim]).
    """
    Q, K, V = _f32(Q), _f32(K), _f32(V)
    n_q = Q.shape[0]
    total_k = K.shape[0]
    out = np.zeros((n_q, n_heads * head_dim), np.float32)
    rc = lib().pkvo_attn_contig(_ptr(Q), _ptr(K), _ptr(V), n_q, total_k,
                                n_heads, n_kv_heads, head_dim, int(causal),
                                float(scale), _ptr(out))
    return rc, out


def rope(x, n_heads, head_dim, positions, log_base):
    """Rotary embedding (neox form) of rows x [n, n_heads*head_dim] at the
    given positions; log_base is ln(rotary base).  Returns (status, rotated
    copy)."""
    out = np.array(x, dtype=np.float32, copy=True, order="C")
    pos = np.ascontiguousarray(np.asarray(positions, dtype=np.int32).reshape(-1))
    n = out.shape[0]
    if pos.size != n:
        raise ValueError("one position per row")
    rc = lib().pkvo_rope(_ptr(out), n, n_heads, head_dim, _ptr(pos),
                         float(log_base))
    return rc, out


def gqa_attention(Q, K, V, n_tokens, n_q_heads, n_kv_heads, head_dim, scale):
    """The pages' unmasked contiguous GQA over one chunk; returns (status, out)."""
    Q, K, V = _f32(Q), _f32(K), _f32(V)
    out = np.zeros((max(n_tokens, 0), max(n_q_heads, 0) * max(head_dim, 0)),
                   np.float32)
    rc = lib().pkvo_gqa_attention(_ptr(Q), _ptr(K), _ptr(V), n_tokens,
                                  n_q_heads, n_kv_heads, head_dim,
                                  float(scale), _ptr(out))
    return rc, out


class Cache:
    """Contiguous per-sequence KV cache (the pages' contiguous twin)."""

    def __init__(self, n_layers, n_kv_heads, max_seq, head_dim):
        self._h = lib().pkvo_cache_new(n_layers, n_kv_heads, max_seq, head_dim)
        if not self._h:
            raise ValueError("bad cache dims")

    def __del__(self):
        if getattr(self, "_h", None):
            lib().pkvo_cache_free(self._h)
            self._h = None

    @property
    def seq_len(self):
        return lib().pkvo_cache_len(self._h)

    def advance(self, n):
        return lib().pkvo_cache_advance(self._h, n)

    def attn_with_cache(self, Q, K_new, V_new, n_tokens, n_heads, n_kv_heads,
                        head_dim, layer, causal, scale):
        Q, K_new, V_new = _f32(Q), _f32(K_new), _f32(V_new)
        out = np.zeros((n_tokens, n_heads * head_dim), np.float32)
        rc = lib().pkvo_attn_with_cache(_ptr(Q), _ptr(K_new), _ptr(V_new),
                                        n_tokens, n_heads, n_kv_heads, head_dim,
                                        self._h, layer, int(causal),
                                        float(scale), _ptr(out))
        return rc, out


class Pool:
    """Refcounted paged block pool with sequences addressed by small ids."""

    def __init__(self, n_blocks, block_size, n_layers, n_kv_heads, head_dim,
                 max_seqs=64, with_storage=True):
        self.n_blocks = n_blocks
        self.block_size = block_size
        self.n_layers = n_layers
        self.n_kv_heads = n_kv_heads
        self.head_dim = head_dim
        self._h = lib().pkvo_pool_new(n_blocks, block_size, n_layers,
                                      n_kv_heads, head_dim, max_seqs,
                                      int(with_storage))
        if not self._h:
            raise ValueError("bad pool dims")

    def __del__(self):
        if getattr(self, "_h", None):
            lib().pkvo_pool_free(self._h)
            self._h = None

    # block level
    def alloc_block(self):
        return lib().pkvo_alloc_block(self._h)

    def unref_block(self, b):
        return lib().pkvo_unref_block(self._h, b)

    def set_free_order(self, ids):
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int64))
        return lib().pkvo_set_free_order(self._h, _ptr(a), a.size)

    # sequence level
    def seq_new(self, max_tokens):
        return lib().pkvo_seq_new(self._h, max_tokens)

    def seq_free(self, s):
        return lib().pkvo_seq_free(self._h, s)

    def seq_fork(self, s):
        return lib().pkvo_seq_fork(self._h, s)

    def seq_truncate(self, s, new_len):
        return lib().pkvo_seq_truncate(self._h, s, new_len)

    def ensure_append(self, seqs, n):
        a = _ids(seqs)
        return lib().pkvo_ensure_append(self._h, _ptr(a), a.size, n)

    def append_layer(self, seqs, n, layer, K_new, V_new):
        a = _ids(seqs)
        K_new, V_new = _f32(K_new), _f32(V_new)
        return lib().pkvo_append_layer(self._h, _ptr(a), a.size, n, layer,
                                       _ptr(K_new), _ptr(V_new))

    def advance(self, seqs, n):
        a = _ids(seqs)
        return lib().pkvo_advance(self._h, _ptr(a), a.size, n)

    def attn_paged(self, seqs, n_q, layer, n_heads, n_kv_heads, head_dim, Q,
                   causal, scale):
        a = _ids(seqs)
        Q = _f32(Q)
        out = np.zeros((a.size * n_q, n_heads * head_dim), np.float32)
        rc = lib().pkvo_attn_paged(self._h, _ptr(a), a.size, n_q, layer,
                                   n_heads, n_kv_heads, head_dim, _ptr(Q),
                                   int(causal), float(scale), _ptr(out))
        return rc, out

    def attn_with_paged(self, Q, K_new, V_new, n_tokens, n_heads, n_kv_heads,
                        head_dim, seq, layer, causal, scale):
        Q, K_new, V_new = _f32(Q), _f32(K_new), _f32(V_new)
        out = np.zeros((n_tokens, n_heads * head_dim), np.float32)
        rc = lib().pkvo_attn_with_paged(_ptr(Q), _ptr(K_new), _ptr(V_new),
                                        n_tokens, n_heads, n_kv_heads, head_dim,
                                        self._h, seq, layer, int(causal),
                                        float(scale), _ptr(out))
        return rc, out

    # introspection
    def seq_len(self, s):
        return lib().pkvo_seq_len(self._h, s)

    def seq_pages(self, s):
        cap = self.n_blocks
        out = np.zeros(cap, np.int64)
        n = lib().pkvo_seq_pages(self._h, s, _ptr(out), cap)
        if n < 0:
            return None
        return out[:n].copy()

    def refcounts(self):
        out = np.zeros(self.n_blocks, np.int32)
        lib().pkvo_refcounts(self._h, _ptr(out))
        return out

    def free_stack(self):
        out = np.zeros(self.n_blocks, np.int64)
        n = lib().pkvo_free_stack(self._h, _ptr(out), self.n_blocks)
        return out[:n].copy()

    def read_row(self, s, layer, pos):
        kv_dim = self.n_kv_heads * self.head_dim
        k = np.zeros(kv_dim, np.float32)
        v = np.zeros(kv_dim, np.float32)
        rc = lib().pkvo_read_row(self._h, s, layer, pos, _ptr(k), _ptr(v))
        return rc, k, v

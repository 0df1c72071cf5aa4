"""paged_kv_gqa_layer_amd -- paged-KV grouped-query attention on AMD MI355X.

A thin Python layer over libpkv's C ABI (include/pkv.h).  It only marshals
arguments: every step of the path (append scatter, copy-on-append, decode,
split merge, prefill) runs in the library's gfx950 kernels.  PyTorch supplies
device memory and streams: tensors are passed by ``data_ptr()`` and the
stream defaults to ``torch.cuda.current_stream()``.

Names follow the C functions without the ``pkv_`` prefix.  Calls that return
a status raise :class:`PKVError` on failure unless ``check=False``.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import _lib
from ._lib import (BAD_ARG, BAD_DIM, BAD_GQA, CAPACITY, DEVICE, ERR_SEQ,
                   K_APPEND, K_COW, K_DECODE, K_MERGE, K_PREFILL, K_PREFIX,
                   K_VERIFY, OK, OOM, SIZE_MAX, STATE, UNSUPPORTED, Contig, PKVError)

__all__ = [
    "Pool", "ContigCache", "Rope", "PKVError", "lib", "pool_storage_bytes",
    "OK", "BAD_DIM", "BAD_GQA", "ERR_SEQ", "OOM", "CAPACITY", "BAD_ARG",
    "DEVICE", "UNSUPPORTED", "STATE", "K_APPEND", "K_DECODE", "K_MERGE", "K_PREFILL",
    "K_COW", "K_VERIFY", "K_PREFIX",
]


def lib():
    return _lib.load()


def _ids(seqs) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(seqs, dtype=np.int32).reshape(-1))


def _vp(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _stream(stream):
    if stream is None:
        import torch
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)


def _dptr(t, what, numel=None):
    """Device pointer of a contiguous float32 CUDA tensor (checked)."""
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch tensor" % what)
    if not t.is_cuda:
        raise ValueError("%s must be on the GPU" % what)
    if t.dtype != torch.float32:
        raise ValueError("%s must be float32" % what)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    if numel is not None and t.numel() != numel:
        raise ValueError("%s has %d elements, expected %d" % (what, t.numel(), numel))
    return C.c_void_p(t.data_ptr())


def _ws(ws):
    """(pointer, bytes) of a workspace: a contiguous CUDA tensor, or None."""
    if ws is None:
        return None, 0
    import torch
    if not isinstance(ws, torch.Tensor):
        raise TypeError("ws must be a torch tensor")
    if not ws.is_cuda:
        raise ValueError("ws must be on the GPU")
    if not ws.is_contiguous():
        raise ValueError("ws must be contiguous")
    return C.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def _check(rc, what, check=True):
    if check and rc != OK:
        raise PKVError(rc, what)
    return rc


def pool_storage_bytes(n_blocks, block_size, n_layers, n_kv_heads, head_dim):
    return lib().pkv_pool_storage_bytes(n_blocks, block_size, n_layers,
                                        n_kv_heads, head_dim)


class Rope:
    """Rotary table (``pkv_rope``) on the current GPU: neox-form turns at
    positions [0, max_positions); ``log_base`` = ln(rotary base)."""

    def __init__(self, head_dim, log_base, max_positions):
        self.head_dim = head_dim
        self.log_base = float(log_base)
        self.max_positions = max_positions
        self._free = lib().pkv_rope_free  # kept for interpreter shutdown
        self._h = lib().pkv_rope_new(head_dim, self.log_base, max_positions)
        if not self._h:
            raise ValueError("pkv_rope_new failed (bad arguments or HIP error)")

    def close(self):
        if getattr(self, "_h", None):
            self._free(self._h)
            self._h = None

    def __del__(self):
        self.close()


class Pool:
    """A refcounted paged KV pool (``pkv_pool``).

    ``device=None`` makes a metadata-only pool (no GPU needed).  Otherwise the
    pool's storage is a torch uint8 tensor on ``device`` owned by this object.
    """

    def __init__(self, n_blocks, block_size, n_layers, n_kv_heads, head_dim,
                 max_seqs=1024, device="cuda"):
        self.n_blocks = n_blocks
        self.block_size = block_size
        self.n_layers = n_layers
        self.n_kv_heads = n_kv_heads
        self.head_dim = head_dim
        self.max_seqs = max_seqs
        self.storage = None
        ptr, nbytes = None, 0
        if device is not None:
            import torch
            nbytes = pool_storage_bytes(n_blocks, block_size, n_layers,
                                        n_kv_heads, head_dim)
            if nbytes == 0:
                raise ValueError("bad pool dims")
            self.storage = torch.empty(nbytes, dtype=torch.uint8, device=device)
            ptr = self.storage.data_ptr()
        self._free = lib().pkv_pool_free  # kept for interpreter shutdown
        self._h = lib().pkv_pool_new(n_blocks, block_size, n_layers, n_kv_heads,
                                     head_dim, max_seqs, ptr, nbytes)
        if not self._h:
            raise ValueError("pkv_pool_new failed (bad sizes)")
        self.rope = None

    def set_rope(self, rope, check=True):
        """Turn rotary embedding on with a :class:`Rope` table, or off (None);
        the pool keeps a reference to the table."""
        rc = _check(lib().pkv_pool_set_rope(self._h, rope._h if rope else None),
                    "pool_set_rope", check)
        if rc == OK:
            self.rope = rope
        return rc

    def set_checks(self, level, check=True):
        """Debug state checks before device work (0 off, 1 host state and row
        descriptors, 2 also the device page-table mirror)."""
        return _check(lib().pkv_pool_set_checks(self._h, int(level)), "pool_set_checks",
                      check)

    def close(self):
        if getattr(self, "_h", None):
            self._free(self._h)
            self._h = None

    def __del__(self):
        self.close()

    # ----------------------------------------------------------- blocks
    def alloc_block(self):
        return lib().pkv_alloc_block(self._h)

    def unref_block(self, block, check=False):
        return _check(lib().pkv_unref_block(self._h, block), "unref_block", check)

    def set_free_order(self, ids, check=True):
        a = np.ascontiguousarray(np.asarray(ids, dtype=np.int64))
        return _check(lib().pkv_pool_set_free_order(self._h, _vp(a), a.size),
                      "set_free_order", check)

    # -------------------------------------------------------- sequences
    def seq_new(self, max_tokens):
        return lib().pkv_seq_new(self._h, max_tokens)

    def seq_free(self, seq, check=False):
        return _check(lib().pkv_seq_free(self._h, seq), "seq_free", check)

    def seq_fork(self, seq):
        return lib().pkv_seq_fork(self._h, seq)

    def seq_truncate(self, seq, new_len, check=False):
        return _check(lib().pkv_seq_truncate(self._h, seq, new_len),
                      "seq_truncate", check)

    # ------------------------------------------------------ step protocol
    def ensure_append(self, seqs, n_new, stream=None, check=False):
        a = _ids(seqs)
        st = _stream(stream) if self.storage is not None else None
        return _check(lib().pkv_ensure_append(self._h, _vp(a), a.size, n_new, st),
                      "ensure_append", check)

    def append_layer(self, seqs, n_new, layer, K_new, V_new, stream=None,
                     check=False):
        a = _ids(seqs)
        kv_dim = self.n_kv_heads * self.head_dim
        if self.storage is None:
            kp = vp = st = None
        else:
            kp = _dptr(K_new, "K_new", a.size * n_new * kv_dim)
            vp = _dptr(V_new, "V_new", a.size * n_new * kv_dim)
            st = _stream(stream)
        return _check(lib().pkv_append_layer(self._h, _vp(a), a.size, n_new, layer,
                                             kp, vp, st), "append_layer", check)

    def advance(self, seqs, n, check=False):
        a = _ids(seqs)
        return _check(lib().pkv_advance(self._h, _vp(a), a.size, n), "advance", check)

    # ---------------------------------------------------------- attention
    def decode_workspace_bytes(self, seqs, n_heads):
        a = _ids(seqs)
        return lib().pkv_decode_workspace_bytes(self._h, _vp(a), a.size, n_heads)

    def attn_paged_decode(self, seqs, layer, n_heads, n_kv_heads, head_dim, Q,
                          scale, out, ws=None, stream=None, check=False):
        a = _ids(seqs)
        q_dim = n_heads * head_dim
        qp = _dptr(Q, "Q", a.size * q_dim)
        op = _dptr(out, "out", a.size * q_dim)
        wp, wb = _ws(ws)
        return _check(lib().pkv_attn_paged_decode(
            self._h, _vp(a), a.size, layer, n_heads, n_kv_heads, head_dim, qp,
            float(scale), op, wp, wb, _stream(stream)), "attn_paged_decode", check)

    def attn_paged_decode_noalloc(self, seqs, layer, n_heads, n_kv_heads, head_dim,
                                  Q, scale, out, stream=None, check=False):
        """attn_paged_decode without a workspace and without allocating: the
        library's fixed per-GPU device array holds the descriptors and split
        partials (calls overlapping on one GPU race)."""
        a = _ids(seqs)
        q_dim = n_heads * head_dim
        qp = _dptr(Q, "Q", a.size * q_dim)
        op = _dptr(out, "out", a.size * q_dim)
        return _check(lib().pkv_attn_paged_decode_noalloc(
            self._h, _vp(a), a.size, layer, n_heads, n_kv_heads, head_dim, qp,
            float(scale), op, _stream(stream)), "attn_paged_decode_noalloc", check)

    def attn_with_paged_decode(self, seqs, layer, n_heads, n_kv_heads, head_dim,
                               Q, K_new, V_new, scale, out, ws=None, stream=None,
                               check=False):
        """append_layer of one row per sequence, then attn_paged_decode, as
        one call (the pages' append-then-attend wrapper)."""
        a = _ids(seqs)
        q_dim = n_heads * head_dim
        kv_dim = n_kv_heads * head_dim
        qp = _dptr(Q, "Q", a.size * q_dim)
        kp = _dptr(K_new, "K_new", a.size * kv_dim)
        vp = _dptr(V_new, "V_new", a.size * kv_dim)
        op = _dptr(out, "out", a.size * q_dim)
        wp, wb = _ws(ws)
        return _check(lib().pkv_attn_with_paged_decode(
            self._h, _vp(a), a.size, layer, n_heads, n_kv_heads, head_dim, qp, kp, vp,
            float(scale), op, wp, wb, _stream(stream)), "attn_with_paged_decode", check)

    def attn_with_paged_decode_shared(self, seqs, layer, n_heads, n_kv_heads, head_dim,
                                      Q, K_new, V_new, scale, out, ws=None, stream=None,
                                      check=False):
        """append_layer of one row per sequence, then
        attn_paged_decode_shared, as one call."""
        a = _ids(seqs)
        q_dim = n_heads * head_dim
        kv_dim = n_kv_heads * head_dim
        qp = _dptr(Q, "Q", a.size * q_dim)
        kp = _dptr(K_new, "K_new", a.size * kv_dim)
        vp = _dptr(V_new, "V_new", a.size * kv_dim)
        op = _dptr(out, "out", a.size * q_dim)
        wp, wb = _ws(ws)
        return _check(lib().pkv_attn_with_paged_decode_shared(
            self._h, _vp(a), a.size, layer, n_heads, n_kv_heads, head_dim, qp, kp, vp,
            float(scale), op, wp, wb, _stream(stream)), "attn_with_paged_decode_shared",
            check)

    def decode_shared_workspace_bytes(self, seqs, n_heads):
        a = _ids(seqs)
        return lib().pkv_decode_shared_workspace_bytes(self._h, _vp(a), a.size, n_heads)

    def attn_paged_decode_shared(self, seqs, layer, n_heads, n_kv_heads, head_dim,
                                 Q, scale, out, ws=None, stream=None, check=False):
        a = _ids(seqs)
        q_dim = n_heads * head_dim
        qp = _dptr(Q, "Q", a.size * q_dim)
        op = _dptr(out, "out", a.size * q_dim)
        wp, wb = _ws(ws)
        return _check(lib().pkv_attn_paged_decode_shared(
            self._h, _vp(a), a.size, layer, n_heads, n_kv_heads, head_dim, qp,
            float(scale), op, wp, wb, _stream(stream)), "attn_paged_decode_shared",
            check)

    def verify_workspace_bytes(self, seqs, n_q, n_heads):
        a = _ids(seqs)
        return lib().pkv_verify_workspace_bytes(self._h, _vp(a), a.size, n_q, n_heads)

    def attn_paged_verify(self, seqs, n_q, layer, n_heads, n_kv_heads, head_dim,
                          Q, scale, out, ws=None, stream=None, check=False):
        a = _ids(seqs)
        q_dim = n_heads * head_dim
        qp = _dptr(Q, "Q", a.size * n_q * q_dim)
        op = _dptr(out, "out", a.size * n_q * q_dim)
        wp, wb = _ws(ws)
        return _check(lib().pkv_attn_paged_verify(
            self._h, _vp(a), a.size, n_q, layer, n_heads, n_kv_heads, head_dim, qp,
            float(scale), op, wp, wb, _stream(stream)), "attn_paged_verify", check)

    def attn_paged_prefill(self, seqs, n_q, layer, n_heads, n_kv_heads,
                           head_dim, Q, causal, scale, out, stream=None,
                           check=False):
        a = _ids(seqs)
        q_dim = n_heads * head_dim
        qp = _dptr(Q, "Q", a.size * n_q * q_dim)
        op = _dptr(out, "out", a.size * n_q * q_dim)
        return _check(lib().pkv_attn_paged_prefill(
            self._h, _vp(a), a.size, n_q, layer, n_heads, n_kv_heads, head_dim,
            qp, int(causal), float(scale), op, _stream(stream)),
            "attn_paged_prefill", check)

    # ------------------------------------------------------ introspection
    def seq_len(self, seq):
        return lib().pkv_seq_len(self._h, seq)

    def seq_pages(self, seq):
        n = lib().pkv_seq_pages(self._h, seq, None, 0)
        if n < 0:
            return None
        out = np.zeros(max(n, 1), np.int64)
        lib().pkv_seq_pages(self._h, seq, _vp(out), n)
        return out[:n].copy()

    def refcounts(self):
        out = np.zeros(self.n_blocks, np.int32)
        lib().pkv_pool_refcounts(self._h, _vp(out))
        return out

    def free_stack(self):
        out = np.zeros(self.n_blocks, np.int64)
        n = lib().pkv_pool_free_stack(self._h, _vp(out), self.n_blocks)
        return out[:n].copy()

    # ------------------------------------------------------------- timing
    def profile_enable(self, on=True):
        return _check(lib().pkv_profile_enable(self._h, int(on)), "profile_enable")

    def profile_kernels(self, kernels=None):
        """Time only the given kernel ids (None: all) while profiling is on."""
        mask = 0xFFFFFFFF if kernels is None else sum(1 << int(k) for k in kernels)
        return _check(lib().pkv_profile_kernels(self._h, mask), "profile_kernels")

    def profile_samples(self, kernel):
        """Per-launch durations (ms) of one kernel id since profiling was enabled."""
        n = lib().pkv_profile_samples(self._h, kernel, None, 0)
        if n < 0:
            raise PKVError(-n, "profile_samples")
        out = np.zeros(max(n, 1), np.float32)
        n = lib().pkv_profile_samples(self._h, kernel, _vp(out), n)
        if n < 0:
            raise PKVError(-n, "profile_samples")
        return out[:n].astype(np.float64)

    def kernel_name(self, kernel):
        """The kernel form last launched under a kernel id ('' if none)."""
        n = lib().pkv_profile_kernel_name(self._h, kernel, None, 0)
        if n < 0:
            raise PKVError(-n, "profile_kernel_name")
        buf = C.create_string_buffer(n + 1)
        lib().pkv_profile_kernel_name(self._h, kernel, buf, n + 1)
        return buf.value.decode()

    def profile_read(self, kernel):
        ms = C.c_double(0.0)
        n = C.c_int64(0)
        _check(lib().pkv_profile_read(self._h, kernel, C.byref(ms), C.byref(n)),
               "profile_read")
        return ms.value, n.value


class ContigCache:
    """A contiguous KV cache on the GPU read by the same kernels
    (``pkv_contig``): [n_slots][n_layers][2][n_kv_heads][max_seq][head_dim]."""

    def __init__(self, n_slots, n_layers, n_kv_heads, max_seq, head_dim,
                 block_size=16, device="cuda", rope=None):
        import torch
        nbytes = lib().pkv_contig_bytes(n_slots, n_layers, n_kv_heads, max_seq,
                                        head_dim)
        if nbytes == 0:
            raise ValueError("bad cache dims")
        self.buf = torch.zeros(nbytes // 4, dtype=torch.float32, device=device)
        self.rope = rope  # keeps the table alive
        self.desc = Contig(self.buf.data_ptr(), n_slots, n_layers, n_kv_heads,
                           max_seq, head_dim, block_size,
                           rope._h if rope is not None else None)
        self.n_kv_heads = n_kv_heads
        self.head_dim = head_dim

    def append(self, slots, seq_lens, n_new, layer, K_new, V_new, stream=None,
               check=True):
        s, l = _ids(slots), _ids(seq_lens)
        kv_dim = self.n_kv_heads * self.head_dim
        return _check(lib().pkv_contig_append(
            C.byref(self.desc), _vp(s), _vp(l), s.size, n_new, layer,
            _dptr(K_new, "K_new", s.size * n_new * kv_dim),
            _dptr(V_new, "V_new", s.size * n_new * kv_dim), _stream(stream)),
            "contig_append", check)

    def decode_workspace_bytes(self, seq_lens, n_heads):
        l = _ids(seq_lens)
        return lib().pkv_contig_decode_workspace_bytes(
            _vp(l), l.size, n_heads, self.n_kv_heads, self.head_dim)

    def attn_decode(self, slots, seq_lens, layer, n_heads, Q, scale, out,
                    ws=None, stream=None, check=True):
        s, l = _ids(slots), _ids(seq_lens)
        q_dim = n_heads * self.head_dim
        wp, wb = _ws(ws)
        return _check(lib().pkv_attn_contig_decode(
            C.byref(self.desc), _vp(s), _vp(l), s.size, layer, n_heads,
            self.n_kv_heads, self.head_dim, _dptr(Q, "Q", s.size * q_dim),
            float(scale), _dptr(out, "out", s.size * q_dim), wp, wb,
            _stream(stream)), "attn_contig_decode", check)

    def verify_workspace_bytes(self, seq_lens, n_q, n_heads):
        l = _ids(seq_lens)
        return lib().pkv_contig_verify_workspace_bytes(
            _vp(l), l.size, n_q, n_heads, self.n_kv_heads, self.head_dim)

    def attn_verify(self, slots, seq_lens, n_q, layer, n_heads, Q, scale, out,
                    ws=None, stream=None, check=True):
        s, l = _ids(slots), _ids(seq_lens)
        q_dim = n_heads * self.head_dim
        wp, wb = _ws(ws)
        return _check(lib().pkv_attn_contig_verify(
            C.byref(self.desc), _vp(s), _vp(l), s.size, n_q, layer, n_heads,
            self.n_kv_heads, self.head_dim, _dptr(Q, "Q", s.size * n_q * q_dim),
            float(scale), _dptr(out, "out", s.size * n_q * q_dim), wp, wb,
            _stream(stream)), "attn_contig_verify", check)

    def attn_prefill(self, slots, seq_lens, n_q, layer, n_heads, Q, causal,
                     scale, out, stream=None, check=True):
        s, l = _ids(slots), _ids(seq_lens)
        q_dim = n_heads * self.head_dim
        return _check(lib().pkv_attn_contig_prefill(
            C.byref(self.desc), _vp(s), _vp(l), s.size, n_q, layer, n_heads,
            self.n_kv_heads, self.head_dim, _dptr(Q, "Q", s.size * n_q * q_dim),
            int(causal), float(scale), _dptr(out, "out", s.size * n_q * q_dim),
            _stream(stream)), "attn_contig_prefill", check)

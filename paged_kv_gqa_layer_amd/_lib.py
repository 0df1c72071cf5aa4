"""ctypes declarations of libpkv's C ABI (include/pkv.h).

Argument marshalling only.  The library is loaded from this package
directory; if it is missing the import fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

OK = 0
BAD_DIM = 1
BAD_GQA = 2
ERR_SEQ = 3
OOM = 4
CAPACITY = 5
BAD_ARG = 6
DEVICE = 7
UNSUPPORTED = 8
STATE = 9

K_APPEND, K_DECODE, K_MERGE, K_PREFILL, K_COW, K_VERIFY, K_PREFIX = range(7)

SIZE_MAX = (1 << 64) - 1


class Contig(C.Structure):
    """pkv_contig: a contiguous cache descriptor."""
    _fields_ = [("base_dev", C.c_void_p), ("n_slots", C.c_int32),
                ("n_layers", C.c_int32), ("n_kv_heads", C.c_int32),
                ("max_seq", C.c_int32), ("head_dim", C.c_int32),
                ("block_size", C.c_int32), ("rope", C.c_void_p)]


_P, _I32, _I64, _F, _SZ = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
_CP = C.POINTER(Contig)

SIGNATURES = {
    "pkv_strerror": (C.c_char_p, [_I32]),
    "pkv_pool_storage_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "pkv_pool_new": (_P, [_I32, _I32, _I32, _I32, _I32, _I32, _P, _SZ]),
    "pkv_pool_free": (None, [_P]),
    "pkv_rope_new": (_P, [_I32, C.c_double, _I32]),
    "pkv_rope_free": (None, [_P]),
    "pkv_pool_set_rope": (_I32, [_P, _P]),
    "pkv_pool_set_checks": (_I32, [_P, _I32]),
    "pkv_alloc_block": (_I64, [_P]),
    "pkv_unref_block": (_I32, [_P, _I64]),
    "pkv_pool_set_free_order": (_I32, [_P, _P, _I32]),
    "pkv_seq_new": (_I32, [_P, _I32]),
    "pkv_seq_free": (_I32, [_P, _I32]),
    "pkv_seq_fork": (_I32, [_P, _I32]),
    "pkv_seq_truncate": (_I32, [_P, _I32, _I32]),
    "pkv_ensure_append": (_I32, [_P, _P, _I32, _I32, _P]),
    "pkv_append_layer": (_I32, [_P, _P, _I32, _I32, _I32, _P, _P, _P]),
    "pkv_advance": (_I32, [_P, _P, _I32, _I32]),
    "pkv_decode_workspace_bytes": (_SZ, [_P, _P, _I32, _I32]),
    "pkv_attn_paged_decode": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32, _P,
                                     _F, _P, _P, _SZ, _P]),
    "pkv_attn_paged_decode_noalloc": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32,
                                             _P, _F, _P, _P]),
    "pkv_attn_with_paged_decode": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32,
                                          _P, _P, _P, _F, _P, _P, _SZ, _P]),
    "pkv_attn_paged_prefill": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32,
                                      _I32, _P, _I32, _F, _P, _P]),
    "pkv_attn_with_paged_decode_shared": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32,
                                                 _P, _P, _P, _F, _P, _P, _SZ, _P]),
    "pkv_decode_shared_workspace_bytes": (_SZ, [_P, _P, _I32, _I32]),
    "pkv_attn_paged_decode_shared": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32,
                                            _P, _F, _P, _P, _SZ, _P]),
    "pkv_verify_workspace_bytes": (_SZ, [_P, _P, _I32, _I32, _I32]),
    "pkv_attn_paged_verify": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                     _P, _F, _P, _P, _SZ, _P]),
    "pkv_contig_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "pkv_contig_append": (_I32, [_CP, _P, _P, _I32, _I32, _I32, _P, _P, _P]),
    "pkv_contig_decode_workspace_bytes": (_SZ, [_P, _I32, _I32, _I32, _I32]),
    "pkv_attn_contig_decode": (_I32, [_CP, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                      _P, _F, _P, _P, _SZ, _P]),
    "pkv_attn_contig_prefill": (_I32, [_CP, _P, _P, _I32, _I32, _I32, _I32,
                                       _I32, _I32, _P, _I32, _F, _P, _P]),
    "pkv_contig_verify_workspace_bytes": (_SZ, [_P, _I32, _I32, _I32, _I32, _I32]),
    "pkv_attn_contig_verify": (_I32, [_CP, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                      _I32, _P, _F, _P, _P, _SZ, _P]),
    "pkv_seq_len": (_I32, [_P, _I32]),
    "pkv_seq_pages": (_I32, [_P, _I32, _P, _I32]),
    "pkv_pool_refcounts": (_I32, [_P, _P]),
    "pkv_pool_free_stack": (_I32, [_P, _P, _I32]),
    "pkv_profile_enable": (_I32, [_P, _I32]),
    "pkv_profile_kernels": (_I32, [_P, C.c_uint32]),
    "pkv_profile_read": (_I32, [_P, _I32, C.POINTER(C.c_double),
                                C.POINTER(C.c_int64)]),
    "pkv_profile_samples": (_I32, [_P, _I32, _P, _I32]),
    "pkv_profile_kernel_name": (_I32, [_P, _I32, C.c_char_p, _I32]),
}

_lib = None


def load() -> C.CDLL:
    """Load libpkv.so from the package directory (raises if it is absent)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libpkv.so is not built (expected at %s); run "
                "`python -m paged_kv_gqa_layer_amd.build`" % LIB_PATH)
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class PKVError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = int(code)
        msg = load().pkv_strerror(self.code).decode()
        super().__init__("%s: %s (%d)" % (what, msg, self.code) if what else
                         "%s (%d)" % (msg, self.code))

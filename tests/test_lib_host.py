"""The C-ABI library on the CPU: it loads, exports what include/pkv.h
declares, and its host-side pool logic matches the oracle's state bit for bit
(reference counts, free stack, page tables, lengths, status codes) on the
pages' known answers and on seeded random operation sequences.  No kernel is
launched: the pools here are metadata-only.
"""
import os
import re

import numpy as np
import pytest

import oracle
import paged_kv_gqa_layer_amd as pkv
import synth
from conftest import ROOT, read_golden


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 25
    L = pkv.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(pkv._lib.SIGNATURES), "binding out of date"


def test_strerror_and_storage_bytes():
    L = pkv.lib()
    assert L.pkv_strerror(0) == b"ok"
    assert pkv.pool_storage_bytes(10, 16, 2, 8, 128) == 10 * 2 * 2 * 8 * 16 * 128 * 4
    assert pkv.pool_storage_bytes(0, 16, 2, 8, 128) == 0


def test_pool_new_rejects_bad_sizes():
    L = pkv.lib()
    assert not L.pkv_pool_new(0, 4, 1, 1, 4, 4, None, 0)
    assert not L.pkv_pool_new(4, 4, 1, 1, 4, 0, None, 0)
    # 64 mirror entries per sequence id must stay int32-addressable
    assert not L.pkv_pool_new(4, 4, 1, 1, 4, (1 << 25), None, 0)
    h = L.pkv_pool_new(4, 4, 1, 1, 4, (1 << 25) - 1, None, 0)
    assert h
    L.pkv_pool_free(h)


def test_pool_new_checks_storage_size_and_alignment():
    """The pool only records the storage pointer (no HIP call), so address
    values stand in for device memory here: 256-byte alignment and at least
    pkv_pool_storage_bytes bytes are required."""
    L = pkv.lib()
    need = pkv.pool_storage_bytes(4, 4, 1, 1, 4)
    base = 1 << 20
    for off, nbytes, ok in ((0, need, True), (0, need - 1, False), (16, need, False),
                            (128, need, False), (256, need, True)):
        h = L.pkv_pool_new(4, 4, 1, 1, 4, 4, base + off, nbytes)
        assert bool(h) == ok, (off, nbytes)
        if h:
            L.pkv_pool_free(h)


def test_seq_new_refuses_page_tables_past_int32_mirror_offsets():
    """max_seqs x (longest page table rounded up to 64 entries) must fit in
    int32: a sequence that would break that is refused with CAPACITY and the
    pool is left as it was."""
    max_seqs = 32768
    p = pkv.Pool(64, 16, 1, 8, 128, max_seqs=max_seqs, device=None)
    a = p.seq_new(1 << 20)               # 65536 pages: 32768 * 65536 = 2^31
    assert a == -pkv.CAPACITY
    assert p.seq_len(0) == -pkv.ERR_SEQ  # no sequence was made
    ok_tokens = (65536 - 64) * 16        # 65472 pages: 32768 * 65472 < 2^31
    a = p.seq_new(ok_tokens)
    assert a == 0
    assert p.seq_new(1 << 20) == -pkv.CAPACITY
    assert p.seq_new(16) == 1
    assert p.ensure_append([a], 100) == 0 and p.advance([a], 100) == 0
    assert p.seq_len(a) == 100


def test_unref_refuses_page_table_references():
    """unref_block drops only references taken by alloc_block; the library and
    the oracle refuse the rest the same way and keep the same state."""
    for impl in ("lib", "oracle"):
        p = (pkv.Pool(8, 4, 1, 1, 4, device=None) if impl == "lib"
             else oracle.Pool(8, 4, 1, 1, 4, with_storage=False))
        a = p.seq_new(64)
        assert p.ensure_append([a], 6) == 0 and p.advance([a], 6) == 0
        b0 = int(p.seq_pages(a)[0])
        f = p.seq_fork(a)
        assert f >= 0
        raw = int(p.alloc_block())
        st = (p.refcounts().tolist(), p.free_stack().tolist())
        assert p.unref_block(b0) == pkv.BAD_ARG, impl
        assert (p.refcounts().tolist(), p.free_stack().tolist()) == st
        assert p.unref_block(raw) == 0
        assert p.seq_free(f) == 0 and p.seq_free(a) == 0
        assert p.refcounts().tolist() == [0] * 8


def test_known_answers_from_pages():
    g = read_golden("pool_known_answers.txt")
    p = pkv.Pool(int(g["pool_blocks"]), 4, 1, 1, 4, device=None)
    allocs = [int(x) for x in g["allocs"].split()]
    assert [p.alloc_block() for _ in allocs] == allocs
    assert p.unref_block(int(g["unref"])) == 0
    assert p.alloc_block() == int(g["realloc"])


def _lib_state(p, seqs):
    return (p.refcounts().tolist(), p.free_stack().tolist(),
            [(p.seq_len(s), None if p.seq_pages(s) is None else p.seq_pages(s).tolist())
             for s in seqs])


def _oracle_state(o, seqs):
    return (o.refcounts().tolist(), o.free_stack().tolist(),
            [(o.seq_len(s), None if o.seq_pages(s) is None else o.seq_pages(s).tolist())
             for s in seqs])


def test_gate_pool_trace_matches_oracle():
    """The gate's pool operations (prefill 5, fork, diverge, truncate,
    re-append) give the same state in the library and the oracle."""
    gate = synth.TinyGate()
    o = oracle.Pool(gate.n_blocks, gate.block_size, gate.n_layers,
                    gate.n_kv_heads, gate.head_dim, with_storage=False)
    p = pkv.Pool(gate.n_blocks, gate.block_size, gate.n_layers,
                 gate.n_kv_heads, gate.head_dim, device=None)
    for impl in (o, p):
        a = impl.seq_new(gate.max_tokens)
        assert impl.ensure_append([a], 5) == 0
        for L in range(gate.n_layers):
            assert impl.append_layer([a], 5, L, None, None) == 0 if impl is p else True
        assert impl.advance([a], 5) == 0
        b = impl.seq_fork(a)
        assert b == 1
        for s in (a, b):
            assert impl.ensure_append([s], 2) == 0
            assert impl.advance([s], 2) == 0
        assert impl.seq_truncate(a, 5) == 0
        assert impl.ensure_append([a], 2) == 0
        assert impl.advance([a], 2) == 0
    assert _lib_state(p, [0, 1]) == _oracle_state(o, [0, 1])
    pa, pb = p.seq_pages(0), p.seq_pages(1)
    ref = p.refcounts()
    assert pa[0] == pb[0] and ref[pa[0]] == 2
    assert pa[1] != pb[1] and ref[pa[1]] == 1 and ref[pb[1]] == 1


@pytest.mark.parametrize("seed", range(8))
def test_random_ops_state_matches_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.choice([1, 2, 4, 16]))
    n_blocks = int(rng.integers(8, 64))
    max_seqs = 6
    o = oracle.Pool(n_blocks, B, 2, 1, 2, max_seqs=max_seqs, with_storage=False)
    p = pkv.Pool(n_blocks, B, 2, 1, 2, max_seqs=max_seqs, device=None)
    # odd seeds run with the debug state checks on: they must never fire on
    # states the operations produce, nor change any status
    p.set_checks(seed % 2)
    perm = rng.permutation(n_blocks)
    assert o.set_free_order(perm) == p.set_free_order(perm, check=False) == 0
    raw = []
    for step in range(200):
        op = int(rng.integers(0, 9))
        s = int(rng.integers(-1, max_seqs + 1))
        if op == 0:
            mt = int(rng.integers(-1, 80))
            assert o.seq_new(mt) == p.seq_new(mt)
        elif op == 1:
            assert o.seq_fork(s) == p.seq_fork(s)
        elif op == 2:
            nl = int(rng.integers(-1, 40))
            assert o.seq_truncate(s, nl) == p.seq_truncate(s, nl)
        elif op == 3:
            assert o.seq_free(s) == p.seq_free(s)
        elif op == 4:
            b1, b2 = o.alloc_block(), p.alloc_block()
            assert b1 == b2
            if b1 >= 0:
                raw.append(b1)
        elif op == 5:
            if raw and rng.random() < 0.7:
                b = raw.pop()
            else:  # an id that is free, out of range or held by a page
                # table (but not raw): both must refuse it
                free = o.free_stack().tolist()
                held = [int(x) for q in range(max_seqs)
                        for x in (o.seq_pages(q) if o.seq_pages(q) is not None else [])
                        if int(x) not in raw]
                b = int(rng.choice(free + held + [-1, n_blocks]))
            assert o.unref_block(b) == p.unref_block(b)
        else:
            M = int(rng.integers(0, 4))
            batch = [int(x) for x in rng.integers(-1, max_seqs, size=M)]
            n = int(rng.integers(0, 9))
            assert o.ensure_append(batch, n) == p.ensure_append(batch, n), (step, batch, n)
            if op >= 7:
                layer = int(rng.integers(-1, 3))
                assert (o.append_layer(batch, n, layer, np.zeros((max(M * n, 1), 2), np.float32),
                                       np.zeros((max(M * n, 1), 2), np.float32))
                        == p.append_layer(batch, n, layer, None, None)), (step, batch, n)
            nadv = n if rng.random() < 0.8 else int(rng.integers(0, 9))
            assert o.advance(batch, nadv) == p.advance(batch, nadv)
        assert _lib_state(p, range(max_seqs)) == _oracle_state(o, range(max_seqs)), step


def test_ensure_oom_is_atomic():
    p = pkv.Pool(5, 4, 1, 1, 4, device=None)
    a, b = p.seq_new(64), p.seq_new(64)
    assert p.ensure_append([a], 8) == 0 and p.advance([a], 8) == 0
    before = _lib_state(p, [a, b])
    assert p.ensure_append([a, b], 9) == pkv.OOM
    assert _lib_state(p, [a, b]) == before


def test_attention_front_checks_order():
    """Status codes of the attention entry points follow the pages' order
    (dims, grouping, sequence) before anything else; a metadata-only pool
    then refuses with BAD_ARG."""
    L = pkv.lib()
    p = pkv.Pool(4, 4, 1, 2, 4, device=None)
    s = np.array([p.seq_new(8)], np.int32)
    sp = s.ctypes.data_as(pkv._lib.C.c_void_p)
    dec = L.pkv_attn_paged_decode
    assert dec(p._h, sp, 0, 0, 4, 2, 4, None, 1.0, None, None, 0, None) == pkv.BAD_DIM
    assert dec(p._h, sp, 1, 0, 3, 2, 4, None, 1.0, None, None, 0, None) == pkv.BAD_GQA
    assert dec(p._h, sp, 1, 0, 4, 1, 4, None, 1.0, None, None, 0, None) == pkv.BAD_DIM
    bad = np.array([3], np.int32)
    assert dec(p._h, bad.ctypes.data_as(pkv._lib.C.c_void_p), 1, 0, 4, 2, 4, None,
               1.0, None, None, 0, None) == pkv.ERR_SEQ
    assert dec(p._h, sp, 1, 1, 4, 2, 4, None, 1.0, None, None, 0, None) == pkv.BAD_ARG
    assert dec(p._h, sp, 1, 0, 4, 2, 4, None, 1.0, None, None, 0, None) == pkv.BAD_ARG
    pre = L.pkv_attn_paged_prefill
    assert pre(p._h, sp, 1, 0, 0, 4, 2, 4, None, 1, 1.0, None, None) == pkv.BAD_DIM
    assert pre(p._h, sp, 1, 2, 0, 6, 4, 4, None, 1, 1.0, None, None) == pkv.BAD_GQA
    fused = L.pkv_attn_with_paged_decode
    assert fused(p._h, sp, 0, 0, 4, 2, 4, None, None, None, 1.0, None, None, 0,
                 None) == pkv.BAD_DIM
    assert fused(p._h, sp, 1, 0, 3, 2, 4, None, None, None, 1.0, None, None, 0,
                 None) == pkv.BAD_GQA
    assert fused(p._h, bad.ctypes.data_as(pkv._lib.C.c_void_p), 1, 0, 4, 2, 4, None,
                 None, None, 1.0, None, None, 0, None) == pkv.ERR_SEQ
    assert fused(p._h, sp, 1, 1, 4, 2, 4, None, None, None, 1.0, None, None, 0,
                 None) == pkv.BAD_ARG
    # rows not ensured, then (ensured) a metadata-only pool cannot attend
    assert fused(p._h, sp, 1, 0, 4, 2, 4, None, None, None, 1.0, None, None, 0,
                 None) == pkv.ERR_SEQ
    assert p.ensure_append(s, 1) == 0
    assert fused(p._h, sp, 1, 0, 4, 2, 4, None, None, None, 1.0, None, None, 0,
                 None) == pkv.BAD_ARG


def test_rope_table_argument_checks():
    """pkv_rope_new refuses bad shapes before touching the device;
    pkv_pool_set_rope(NULL) switches rotary embedding off on any pool."""
    L = pkv.lib()
    assert not L.pkv_rope_new(0, 9.2, 16)
    assert not L.pkv_rope_new(7, 9.2, 16)       # odd head_dim: no pairs
    assert not L.pkv_rope_new(8, 0.0, 16)
    assert not L.pkv_rope_new(8, -1.0, 16)
    assert not L.pkv_rope_new(8, float("inf"), 16)
    assert not L.pkv_rope_new(8, float("nan"), 16)
    assert not L.pkv_rope_new(8, 9.2, 0)
    L.pkv_rope_free(None)
    p = pkv.Pool(4, 4, 1, 1, 4, device=None)
    assert L.pkv_pool_set_rope(p._h, None) == pkv.OK
    assert L.pkv_pool_set_rope(None, None) == pkv.BAD_ARG


def test_binding_rejects_host_and_malformed_buffers():
    """Pointers handed to the library must be contiguous device buffers; the
    binding refuses host tensors before any call (a host pointer in a kernel
    would fault the GPU)."""
    import torch
    with pytest.raises(ValueError):
        pkv._ws(torch.empty(16, dtype=torch.uint8))
    with pytest.raises(TypeError):
        pkv._ws(np.empty(16, np.uint8))
    with pytest.raises(ValueError):
        pkv._dptr(torch.empty(4, dtype=torch.float32), "Q")
    assert pkv._ws(None) == (None, 0)
    assert pkv._dptr(None, "Q") is None


def _split(own, n_q):
    """The documented key split of a row with `own` keys and n_q new rows."""
    s = 256 if own < 2048 else 512 if own < 6144 else 1024 if own < 8192 else 2048
    return s if n_q <= 4 else 2 * s


@pytest.mark.parametrize("n_q", [1, 4, 8])
def test_split_plan_sizes(n_q):
    """Workspace sizes (partial slots x n_q x heads x (head_dim + 2) floats)
    follow the per-row split sizes at every threshold; a batch needs the sum
    of its rows' slots, independent of order."""
    L = pkv.lib()
    H, G, D = 32, 8, 128
    per_slot = n_q * H * (D + 2) * 4

    def ws(lens):
        a = np.asarray(lens, np.int32)
        p = a.ctypes.data_as(pkv._lib.C.c_void_p)
        if n_q == 1:
            return L.pkv_contig_decode_workspace_bytes(p, a.size, H, G, D)
        return L.pkv_contig_verify_workspace_bytes(p, a.size, n_q, H, G, D)

    edges = [0, 255, 256, 511, 2047 - n_q, 2048 - n_q, 2049 - n_q, 6143 - n_q, 6144 - n_q,
             6145 - n_q, 8191 - n_q, 8192 - n_q, 12288, 16383, 65536]
    slots = []
    for seq_len in edges:
        own = seq_len + n_q
        k = -(-own // _split(own, n_q))
        slots.append(k)
        assert ws([seq_len]) == (k * per_slot if k > 1 else 0), seq_len
    assert ws(edges) == sum(slots) * per_slot
    assert ws(edges[::-1]) == sum(slots) * per_slot


def test_set_checks_arguments():
    p = pkv.Pool(8, 4, 1, 1, 4, device=None)
    assert p.set_checks(0) == 0 and p.set_checks(2) == 0
    assert p.set_checks(3, check=False) == pkv.BAD_ARG
    assert p.set_checks(-1, check=False) == pkv.BAD_ARG
    assert pkv.lib().pkv_pool_set_checks(None, 1) == pkv.BAD_ARG
    assert pkv.lib().pkv_strerror(pkv.STATE) == b"pool state check failed"

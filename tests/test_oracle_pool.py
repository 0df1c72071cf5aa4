"""Pins for the oracle's paged pool (CPU only).

The pages fix a few known answers (allocation order, exhaustion, recycling,
the fork reference count) and three bit-exact invariants (paged ==
contiguous, fork == fresh replay, rewind == the other fork).  The rest of the
pool's behaviour is pinned by invariants that hold for any correct pool:
reference counts equal the number of references, the free stack holds
exactly the unreferenced ids, and every sequence reads back exactly the rows
that were appended to it (which a missing copy-on-append would break).
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden


def _ints(s):
    return [int(x, 0) for x in s.split()]


# ------------------------------------------------------------ known answers

def test_pool_known_answers_from_pages():
    g = read_golden("pool_known_answers.txt")
    p = oracle.Pool(int(g["pool_blocks"]), 4, 1, 1, 4, with_storage=False)
    got = [p.alloc_block() for _ in _ints(g["allocs"])]
    assert got == _ints(g["allocs"])
    assert p.unref_block(int(g["unref"])) == 0
    assert p.alloc_block() == int(g["realloc"])


def test_fork_shares_first_page_with_refcount_two():
    g = read_golden("pool_known_answers.txt")
    gate = synth.TinyGate()
    p = oracle.Pool(gate.n_blocks, gate.block_size, gate.n_layers,
                    gate.n_kv_heads, gate.head_dim)
    a = p.seq_new(gate.max_tokens)
    n = int(g["fork_prefill_rows"])
    assert p.ensure_append([a], n) == 0
    assert p.advance([a], n) == 0
    b = p.seq_fork(a)
    assert b >= 0
    assert p.refcounts()[p.seq_pages(a)[0]] == int(g["fork_first_page_refcount"])
    assert np.array_equal(p.seq_pages(a), p.seq_pages(b))


def test_gate_constants_match_fixture():
    g = read_golden("pool_known_answers.txt")
    gate = synth.TinyGate()
    assert (gate.n_layers, gate.n_heads, gate.n_kv_heads, gate.head_dim) == (
        int(g["gate_layers"]), int(g["gate_heads"]), int(g["gate_kv_heads"]),
        int(g["gate_head_dim"]))
    assert gate.n_blocks == int(g["gate_pool_blocks"])
    assert gate.max_tokens == int(g["gate_max_tokens"])
    assert np.float32(gate.scale).view(np.uint32) == int(g["gate_scale_bits"], 16)


# ------------------------------------------------------------- the gate

def _round_both(cache, pool, seq, qkv, n, gate):
    """One append round on the contiguous and the paged path; per layer the
    outputs must be bit-identical."""
    Q, K, V = qkv
    assert pool.ensure_append([seq], n) == 0
    outs = []
    for L in range(gate.n_layers):
        rc, oc = cache.attn_with_cache(Q, K, V, n, gate.n_heads, gate.n_kv_heads,
                                       gate.head_dim, L, True, gate.scale)
        assert rc == 0
        rc, op = pool.attn_with_paged(Q, K, V, n, gate.n_heads, gate.n_kv_heads,
                                      gate.head_dim, seq, L, True, gate.scale)
        assert rc == 0
        assert np.array_equal(oc.view(np.uint32), op.view(np.uint32))
        outs.append(op)
    assert cache.advance(n) == 0
    assert pool.advance([seq], n) == 0
    return outs


def _round_paged(pool, seq, qkv, n, gate):
    Q, K, V = qkv
    assert pool.ensure_append([seq], n) == 0
    outs = []
    for L in range(gate.n_layers):
        rc, op = pool.attn_with_paged(Q, K, V, n, gate.n_heads, gate.n_kv_heads,
                                      gate.head_dim, seq, L, True, gate.scale)
        assert rc == 0
        outs.append(op)
    assert pool.advance([seq], n) == 0
    return np.stack(outs)


def _round_contig(cache, qkv, n, gate):
    Q, K, V = qkv
    outs = []
    for L in range(gate.n_layers):
        rc, oc = cache.attn_with_cache(Q, K, V, n, gate.n_heads, gate.n_kv_heads,
                                       gate.head_dim, L, True, gate.scale)
        assert rc == 0
        outs.append(oc)
    assert cache.advance(n) == 0
    return np.stack(outs)


def _pool(gate):
    return oracle.Pool(gate.n_blocks, gate.block_size, gate.n_layers,
                       gate.n_kv_heads, gate.head_dim)


def _cache(gate):
    return oracle.Cache(gate.n_layers, gate.n_kv_heads, gate.max_tokens,
                        gate.head_dim)


def test_gate_equiv_paged_equals_contiguous():
    gate = synth.TinyGate()
    x = gate.inputs()
    pool, cache = _pool(gate), _cache(gate)
    s = pool.seq_new(gate.max_tokens)
    for name, n in (("1", 5), ("2", 1), ("3", 3)):
        _round_both(cache, pool, s, x[name], n, gate)
    assert pool.seq_len(s) == 9


def test_gate_fork_cow_and_rewind():
    gate = synth.TinyGate()
    x = gate.inputs()
    pool = _pool(gate)
    a = pool.seq_new(gate.max_tokens)
    _round_both(_cache(gate), pool, a, x["1"], 5, gate)
    b = pool.seq_fork(a)
    ref = pool.refcounts()
    pa = pool.seq_pages(a)
    assert ref[pa[0]] == 2 and ref[pa[1]] == 2

    opA = _round_paged(pool, a, x["A"], 2, gate)
    opB = _round_paged(pool, b, x["B"], 2, gate)
    pa, pb = pool.seq_pages(a), pool.seq_pages(b)
    ref = pool.refcounts()
    # block size 4: page 0 (rows 0-3) was full at the fork and stays shared;
    # page 1 held the partial tail (row 4) and was copied on append
    assert pa[0] == pb[0] and ref[pa[0]] == 2
    assert pa[1] != pb[1] and ref[pa[1]] == 1 and ref[pb[1]] == 1

    gA, gB = _cache(gate), _cache(gate)
    _round_contig(gA, x["1"], 5, gate)
    _round_contig(gB, x["1"], 5, gate)
    ocA = _round_contig(gA, x["A"], 2, gate)
    ocB = _round_contig(gB, x["B"], 2, gate)
    assert np.array_equal(opA.view(np.uint32), ocA.view(np.uint32))
    assert np.array_equal(opB.view(np.uint32), ocB.view(np.uint32))

    # rewind: truncate A to the fork point, append B's rows -> B's outputs
    assert pool.seq_truncate(a, 5) == 0
    opR = _round_paged(pool, a, x["B"], 2, gate)
    assert np.array_equal(opR.view(np.uint32), ocB.view(np.uint32))


def test_truncate_releases_pages_tail_first():
    p = oracle.Pool(8, 4, 1, 1, 4, with_storage=False)
    a = p.seq_new(32)
    assert p.ensure_append([a], 13) == 0 and p.advance([a], 13) == 0
    pages = p.seq_pages(a)
    assert list(pages) == [0, 1, 2, 3]
    b = p.seq_fork(a)
    assert list(p.refcounts()[:4]) == [2, 2, 2, 2]
    # b drops below the fork point: its pages 3, 2 lose one reference each
    assert p.seq_truncate(b, 6) == 0
    assert list(p.refcounts()[:4]) == [2, 2, 1, 1]
    assert list(p.seq_pages(b)) == [0, 1]
    # a drops to 4 rows: pages 3, 2, 1 are released in that order
    assert p.seq_truncate(a, 4) == 0
    ref = p.refcounts()
    assert list(ref[:4]) == [2, 1, 0, 0]
    fs = p.free_stack()
    assert list(fs[-2:]) == [3, 2]  # 2 was released last, so it pops first
    assert p.alloc_block() == 2


def test_truncate_bounds():
    p = oracle.Pool(8, 4, 1, 1, 4, with_storage=False)
    a = p.seq_new(32)
    assert p.ensure_append([a], 5) == 0 and p.advance([a], 5) == 0
    assert p.seq_truncate(a, 6) == oracle.BAD_ARG
    assert p.seq_truncate(a, -1) == oracle.BAD_ARG
    assert p.seq_truncate(a + 1, 0) == oracle.ERR_SEQ
    assert p.seq_truncate(a, 5) == 0


# ------------------------------------------------------------- failures

def _state(p, seqs):
    return (p.refcounts().tolist(), p.free_stack().tolist(),
            [(p.seq_len(s), None if p.seq_pages(s) is None else p.seq_pages(s).tolist())
             for s in seqs])


def test_ensure_oom_changes_nothing():
    p = oracle.Pool(5, 4, 1, 1, 4, with_storage=False)
    a, b = p.seq_new(64), p.seq_new(64)
    assert p.ensure_append([a], 8) == 0 and p.advance([a], 8) == 0  # 2 pages
    before = _state(p, [a, b])
    # b needs 3 pages and a needs 1: 4 > 3 free
    assert p.ensure_append([a, b], 9) == oracle.OOM
    assert _state(p, [a, b]) == before
    assert p.ensure_append([b], 9) == 0


def test_ensure_counts_cow_exactly_within_a_batch():
    """Two forks sharing a partial tail in one batch: the first copies, after
    which the second holds the old block alone and copies nothing, so one
    free id is enough."""
    p = oracle.Pool(3, 4, 1, 1, 4, with_storage=False)
    a = p.seq_new(16)
    assert p.ensure_append([a], 5) == 0 and p.advance([a], 5) == 0
    b = p.seq_fork(a)
    assert p.ensure_append([a, b], 1) == 0
    pa, pb = p.seq_pages(a), p.seq_pages(b)
    assert pa[1] == 2 and pb[1] == 1
    assert list(p.refcounts()) == [2, 1, 1]


def test_capacity_and_sequence_errors():
    p = oracle.Pool(8, 4, 1, 1, 4, with_storage=True)
    a = p.seq_new(6)
    assert p.ensure_append([a], 7) == oracle.CAPACITY
    assert p.ensure_append([a], 0) == oracle.BAD_DIM
    assert p.ensure_append([], 1) == oracle.BAD_DIM
    assert p.ensure_append([a, a], 1) == oracle.ERR_SEQ
    assert p.ensure_append([a + 5], 1) == oracle.ERR_SEQ
    k = np.zeros((2, 4), np.float32)
    # append without ensure
    assert p.append_layer([a], 2, 0, k, k) == oracle.ERR_SEQ
    assert p.ensure_append([a], 2) == 0
    assert p.append_layer([a], 2, 1, k, k) == oracle.BAD_ARG  # layer range
    assert p.append_layer([a], 2, 0, k, k) == 0
    assert p.advance([a], 5) == oracle.ERR_SEQ  # one page ensured: 4 slots
    assert p.advance([a], 2) == 0
    # append into a page shared with a fork
    b = p.seq_fork(a)
    assert b >= 0
    assert p.append_layer([a], 1, 0, k[:1], k[:1]) == oracle.ERR_SEQ
    assert p.unref_block(99) == oracle.BAD_ARG
    assert p.seq_new(0) == -oracle.BAD_ARG


def test_seq_ids_exhaust_and_recycle():
    p = oracle.Pool(4, 4, 1, 1, 4, max_seqs=2, with_storage=False)
    assert p.seq_new(8) == 0 and p.seq_new(8) == 1
    assert p.seq_new(8) == -oracle.CAPACITY
    assert p.seq_fork(0) == -oracle.CAPACITY
    assert p.seq_free(0) == 0
    assert p.seq_fork(1) == 0


# --------------------------------------------- randomized model comparison

class Model:
    """Token-list model: each sequence is the list of rows appended to it."""

    def __init__(self):
        self.rows = {}   # seq -> list of per-layer (k, v) rows


def _check_invariants(p, model, raw, n_blocks, B):
    ref = p.refcounts()
    want = np.zeros(n_blocks, np.int64)
    for s in model.rows:
        for b in p.seq_pages(s):
            want[b] += 1
    for b in raw:
        want[b] += 1
    assert np.array_equal(ref, want)
    fs = p.free_stack()
    assert len(set(fs.tolist())) == len(fs)
    assert set(fs.tolist()) == set(np.nonzero(ref == 0)[0].tolist())
    for s, rows in model.rows.items():
        assert p.seq_len(s) == len(rows)
        assert len(p.seq_pages(s)) == -(-len(rows) // B)
        for pos, per_layer in enumerate(rows):
            for L, (k, v) in enumerate(per_layer):
                rc, kk, vv = p.read_row(s, L, pos)
                assert rc == 0
                assert np.array_equal(kk, k) and np.array_equal(vv, v)


@pytest.mark.parametrize("seed", range(6))
def test_random_ops_match_token_list_model(seed):
    rng = np.random.default_rng(100 + seed)
    B, n_layers, G, D = 4, 2, 2, 3
    kv_dim = G * D
    n_blocks = 40
    p = oracle.Pool(n_blocks, B, n_layers, G, D, max_seqs=8)
    model = Model()
    raw = []
    for _ in range(120):
        op = rng.integers(0, 7)
        live = sorted(model.rows)
        if op == 0 or not live:
            s = p.seq_new(48)
            if s >= 0:
                model.rows[s] = []
        elif op == 1:
            s = int(rng.choice(live))
            c = p.seq_fork(s)
            if c >= 0:
                model.rows[c] = list(model.rows[s])
        elif op == 2:
            s = int(rng.choice(live))
            nl = int(rng.integers(0, len(model.rows[s]) + 1))
            assert p.seq_truncate(s, nl) == 0
            model.rows[s] = model.rows[s][:nl]
        elif op == 3 and len(live) > 1:
            s = int(rng.choice(live))
            assert p.seq_free(s) == 0
            del model.rows[s]
        elif op == 4:
            if raw and rng.random() < 0.5:
                assert p.unref_block(raw.pop()) == 0
            else:
                b = p.alloc_block()
                if b >= 0:
                    raw.append(b)
        else:
            k_sel = int(rng.integers(1, len(live) + 1))
            batch = [int(x) for x in rng.choice(live, size=k_sel, replace=False)]
            n = int(rng.integers(1, 6))
            before = _state(p, batch)
            rc = p.ensure_append(batch, n)
            if rc != 0:
                assert rc in (oracle.OOM, oracle.CAPACITY)
                assert _state(p, batch) == before
                continue
            new = [[(rng.integers(-8, 9, kv_dim).astype(np.float32),
                     rng.integers(-8, 9, kv_dim).astype(np.float32))
                    for _ in range(n_layers)] for _ in range(len(batch) * n)]
            for L in range(n_layers):
                K = np.stack([r[L][0] for r in new])
                V = np.stack([r[L][1] for r in new])
                assert p.append_layer(batch, n, L, K, V) == 0
            assert p.advance(batch, n) == 0
            for i, s in enumerate(batch):
                model.rows[s] = model.rows[s] + new[i * n:(i + 1) * n]
        _check_invariants(p, model, raw, n_blocks, B)


@pytest.mark.parametrize("seed", range(3))
def test_paged_attention_equals_contiguous_on_random_histories(seed):
    """Bit-exact: attention through the page table equals attention over the
    same rows held contiguously, for scattered placements and forks."""
    rng = np.random.default_rng(200 + seed)
    B, H, G, D = 4, 6, 2, 5
    kv_dim = G * D
    p = oracle.Pool(64, B, 1, G, D, max_seqs=8)
    p.set_free_order(rng.permutation(64))
    hist = {}
    a = p.seq_new(64)
    hist[a] = []
    for _ in range(5):
        batch = list(hist)
        n = int(rng.integers(1, 7))
        assert p.ensure_append(batch, n) == 0
        K = rng.integers(-8, 9, (len(batch) * n, kv_dim)).astype(np.float32)
        V = rng.integers(-8, 9, (len(batch) * n, kv_dim)).astype(np.float32)
        Q = rng.integers(-8, 9, (len(batch) * n, H * D)).astype(np.float32)
        assert p.append_layer(batch, n, 0, K, V) == 0
        rc, out = p.attn_paged(batch, n, 0, H, G, D, Q, True, 0.25)
        assert rc == 0
        for i, s in enumerate(batch):
            hist[s] = hist[s] + [(K[i * n + t], V[i * n + t]) for t in range(n)]
            Kc = np.stack([r[0] for r in hist[s]])
            Vc = np.stack([r[1] for r in hist[s]])
            rc, oc = oracle.attn_contig(Q[i * n:(i + 1) * n], Kc, Vc, H, G, D,
                                        True, 0.25)
            assert rc == 0
            assert np.array_equal(out[i * n:(i + 1) * n].view(np.uint32),
                                  oc.view(np.uint32))
        assert p.advance(batch, n) == 0
        parent = int(rng.choice(batch))
        c = p.seq_fork(parent)
        if c >= 0:
            hist[c] = list(hist[parent])


# ------------------------------------------- placement and block release

def test_set_free_order_sets_the_allocation_order():
    """After set_free_order(ids), allocations return ids[0], ids[1], ...,
    then -1; sequences take their pages in that order; a list that is not a
    permutation of exactly the free ids is refused and changes nothing."""
    rng = np.random.default_rng(7)
    n = 12
    p = oracle.Pool(n, 4, 1, 1, 4, with_storage=False)
    order = rng.permutation(n)
    assert p.set_free_order(order) == 0
    assert [p.alloc_block() for _ in range(n)] == order.tolist()
    assert p.alloc_block() == -1

    # with some ids taken, the order is over the free ones only
    p = oracle.Pool(n, 4, 1, 1, 4, with_storage=False)
    taken = [p.alloc_block() for _ in range(3)]
    assert taken == [0, 1, 2]
    free_now = list(range(3, n))
    stack = p.free_stack().tolist()
    for bad in (free_now[:-1],                      # one short
                free_now + [0],                     # a taken id added
                [0] + free_now[1:],                 # a taken id in place of a free one
                free_now[:-1] + [free_now[0]],      # a repeat
                free_now[:-1] + [n],                # out of range
                free_now[:-1] + [-1]):
        assert p.set_free_order(bad) == oracle.BAD_ARG
        assert p.free_stack().tolist() == stack
    order = [int(x) for x in rng.permutation(free_now)]
    assert p.set_free_order(order) == 0
    s = p.seq_new(64)
    assert p.ensure_append([s], 9) == 0            # 3 pages of 4 rows
    assert p.seq_pages(s).tolist() == order[:3]
    assert [p.alloc_block() for _ in range(2)] == order[3:5]
    # a released id is taken next (LIFO), before the rest of the order
    assert p.unref_block(taken[1]) == 0
    assert p.alloc_block() == taken[1]
    assert p.alloc_block() == order[5]


def test_unref_releases_only_alloc_references():
    """unref_block gives back references taken by alloc_block; references
    that page tables hold are released by truncate and free, and an unref
    that would take one is refused with nothing changed."""
    p = oracle.Pool(8, 4, 1, 1, 4, with_storage=False)
    a = p.seq_new(64)
    assert p.ensure_append([a], 6) == 0 and p.advance([a], 6) == 0
    b0, b1 = p.seq_pages(a).tolist()
    before = (p.refcounts().tolist(), p.free_stack().tolist())
    assert p.unref_block(b0) == oracle.BAD_ARG
    assert (p.refcounts().tolist(), p.free_stack().tolist()) == before
    f = p.seq_fork(a)                               # two holders, count 2
    assert p.refcounts()[b0] == 2
    assert p.unref_block(b0) == oracle.BAD_ARG
    assert p.refcounts()[b0] == 2
    raw = p.alloc_block()
    assert p.unref_block(raw) == 0                  # its own reference
    assert p.unref_block(raw) == oracle.BAD_ARG     # now free
    assert p.seq_free(f) == 0 and p.refcounts()[b0] == 1
    assert p.seq_truncate(a, 0) == 0
    assert p.refcounts()[b0] == 0 and p.refcounts()[b1] == 0
    assert p.free_stack().tolist()[-2:] == [b1, b0]  # last page released first

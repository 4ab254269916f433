"""The library's C++ radix tree (through the C ABI) against the oracle tree, on the CPU.

Index tables must match bit-exact, and so must the canonical tree dumps and the
counters, on all five workloads and on random operation sequences.
"""
import re
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synth
import radix_tree_prefix_amd as rs
from radix_tree_prefix_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# ---------------------------------------------------------------- the ABI surface
def test_library_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "rs.h")).read()
    hdr = re.sub(r"/\*.*?\*/", "", hdr, flags=re.S)
    declared = set(re.findall(r"\b(rs_[a-z0-9_]+)\s*\(", hdr))
    assert len(declared) >= 25
    for name in declared:
        assert hasattr(_lib.lib, name), name
    assert declared == set(_lib.EXPORTS)


def test_version_and_bad_create():
    assert b"gfx950" in _lib.lib.rs_version()
    with pytest.raises(rs.RsError):
        rs.Tree(100, page_size=16)
    with pytest.raises(rs.RsError):
        rs.Tree(0)


# ---------------------------------------------------------------- workloads
def _admit_both(wl):
    ot = oracle.RadixTree(wl.pool_slots)
    ct = rs.Tree(wl.pool_slots)
    o_new, c_new = [], []
    oracle.admit_history(ot, wl.history, lambda i, s, lo, sl: o_new.append((i, lo, sl.copy())))
    for i, s in enumerate(wl.history):
        row, node, m = ct.admit(s, len(s), 0)
        if len(s) > m:
            c_new.append((i, m, row[m:].copy()))
        ct.dec_lock_ref(node)
    ores = oracle.admit_batch(ot, wl)
    ld = ores["ld"]
    table = np.full((wl.B, ld), -1, np.int32)
    nodes = np.zeros(wl.B, np.int64)
    matched = np.zeros(wl.B, np.int64)
    for r in wl.requests:
        row, node, m = ct.admit(r.tokens, r.cached, r.new, out_row=table[r.row, :r.seq_len])
        nodes[r.row], matched[r.row] = node, m
    return ot, ct, ores, table, nodes, matched, o_new, c_new


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_tables_bit_exact(cfg):
    wl = synth.make(cfg)
    ot, ct, ores, table, nodes, matched, o_new, c_new = _admit_both(wl)
    np.testing.assert_array_equal(table, ores["table"])
    np.testing.assert_array_equal(nodes, ores["nodes"])
    np.testing.assert_array_equal(matched, ores["matched"])
    assert len(o_new) == len(c_new)
    for (i1, lo1, s1), (i2, lo2, s2) in zip(o_new, c_new):
        assert (i1, lo1) == (i2, lo2)
        np.testing.assert_array_equal(s1, s2)
    assert ct.dump() == ot.dump()
    cs, os_ = ct.stats(), ot.stats()
    for k in ("nodes", "tree_tokens", "evictable", "protected", "evicted_total", "clock"):
        assert cs[k] == os_[k], k
    assert cs["free_slots"] == os_["free"]


def test_tables_bit_exact_large_mixed_batch():
    """Full-size mixed batch: 4M-slot pool, 1,024-sequence history with eviction, 256 requests."""
    wl = synth.config5()
    ot, ct, ores, table, nodes, matched, o_new, c_new = _admit_both(wl)
    assert ot.evicted_total > 0
    np.testing.assert_array_equal(table, ores["table"])
    np.testing.assert_array_equal(nodes, ores["nodes"])
    np.testing.assert_array_equal(matched, ores["matched"])
    assert ct.dump() == ot.dump()
    cs, os_ = ct.stats(), ot.stats()
    assert (cs["evicted_total"], cs["tree_tokens"], cs["protected"]) == \
        (os_["evicted_total"], os_["tree_tokens"], os_["protected"])


# ---------------------------------------------------------------- random op sequences
seq_st = st.lists(st.integers(0, 2), min_size=0, max_size=10)
op_st = st.one_of(
    st.tuples(st.just("admit"), seq_st, st.integers(0, 3)),
    st.tuples(st.just("match"), seq_st, st.just(0)),
    st.tuples(st.just("lock"), seq_st, st.just(0)),
    st.tuples(st.just("unlock"), st.just([]), st.integers(0, 7)),
    st.tuples(st.just("evict"), st.just([]), st.integers(0, 20)),
    st.tuples(st.just("alloc"), st.just([]), st.integers(0, 6)),
    st.tuples(st.just("free"), st.just([]), st.integers(0, 7)),
    st.tuples(st.just("insert_held"), seq_st, st.just(0)),
)


@settings(max_examples=400, deadline=None)
@given(st.lists(op_st, min_size=1, max_size=40), st.integers(6, 30))
def test_random_ops_match_oracle(ops, pool):
    ot, ct = oracle.RadixTree(pool), rs.Tree(pool)
    locks, held = [], []
    for op, seq, k in ops:
        seq = np.array(seq, dtype=np.int32)
        if op == "admit":
            cached = len(seq)
            try:
                orow, onode, om = oracle.admit(ot, seq, cached, k)
                ook = True
            except oracle.NoSpace:
                ook = False
            try:
                crow, cnode, cm = ct.admit(seq, cached, k)
                cok = True
            except rs.NoSpaceError:
                cok = False
            assert ook == cok
            if ook:
                assert (onode, om) == (cnode, cm)
                np.testing.assert_array_equal(orow, crow)
                locks.append(onode)
                held.append(orow[cached:])
        elif op == "match":
            os_, on = ot.match_prefix(seq)
            cs, cn = ct.match_prefix(seq)
            assert on == cn
            np.testing.assert_array_equal(os_, cs)
        elif op == "lock":
            _a, on = ot.match_prefix(seq)
            _b, cn = ct.match_prefix(seq)
            assert on == cn
            ot.inc_lock_ref(on)
            ct.inc_lock_ref(cn)
            locks.append(on)
        elif op == "unlock" and locks:
            n = locks.pop(k % len(locks))
            ot.dec_lock_ref(n)
            ct.dec_lock_ref(n)
        elif op == "evict":
            assert ot.evict(k) == ct.evict(k)
        elif op == "alloc":
            try:
                a = ot.alloc(k)
                ook = True
            except oracle.NoSpace:
                ook = False
            try:
                b = ct.alloc(k)
                cok = True
            except rs.NoSpaceError:
                cok = False
            assert ook == cok
            if ook:
                np.testing.assert_array_equal(a, b)
                held.append(a)
        elif op == "free" and held:
            s = held.pop(k % len(held))
            ot.free_slots(s)
            ct.free_slots(s)
        elif op == "insert_held" and held and len(seq):
            # insert a sequence with slots the caller holds (some positions may be present already)
            s = held.pop()
            if len(s) >= len(seq):
                use, rest = s[:len(seq)], s[len(seq):]
                p1, n1, f1 = ot.insert(seq, use)
                p2, n2, f2 = ct.insert(seq, use)
                assert (p1, n1) == (p2, n2)
                np.testing.assert_array_equal(f1, f2)
                if len(rest):
                    held.append(rest)
            else:
                held.append(s)
        assert ct.dump() == ot.dump()
        cs, os_ = ct.stats(), ot.stats()
        assert (cs["evictable"], cs["protected"], cs["free_slots"], cs["tree_tokens"]) == \
            (os_["evictable"], os_["protected"], os_["free"], os_["tree_tokens"])


# ---------------------------------------------------------------- error paths
def test_error_codes():
    t = rs.Tree(8)
    row, node, m = t.admit(np.arange(6, dtype=np.int32), 6, 0)
    with pytest.raises(rs.NoSpaceError):          # 6 locked, 2 free: 3 cannot fit
        t.alloc(3)
    assert t.stats()["free_slots"] == 2
    t.dec_lock_ref(node)
    with pytest.raises(rs.RsError) as e:
        t.dec_lock_ref(node)                      # below zero
    assert e.value.code == _lib.RS_E_INVAL
    t.evict(100)
    with pytest.raises(rs.StaleError):
        t.inc_lock_ref(node)
    a = t.alloc(2)
    t.free_slots(a)
    with pytest.raises(rs.RsError):
        t.free_slots(a)                           # double free
    with pytest.raises(rs.RsError):
        t.insert(np.array([1, 2], np.int32), np.array([0, 1], np.int32))   # slots not allocated
    # admit that cannot fit drops its lock and holds nothing
    t2 = rs.Tree(4)
    r1, n1, _ = t2.admit(np.array([1, 2, 3], np.int32), 3, 0)
    with pytest.raises(rs.NoSpaceError):
        t2.admit(np.array([1, 2, 3, 9], np.int32), 3, 2)
    assert t2.stats()["protected"] == 3 and t2.stats()["free_slots"] == 1


def test_galloping_divergence_long_edges():
    """Divergence found at every position of long edges (window edges and inside windows)."""
    rng = np.random.default_rng(0)
    base = rng.integers(0, 1000, 4100).astype(np.int32)
    for cut in [0, 1, 2, 3, 6, 7, 8, 15, 31, 1000, 2047, 2048, 4095, 4099]:
        t, ot = rs.Tree(10000), oracle.RadixTree(10000)
        t.admit(base, len(base), 0)
        oracle.admit(ot, base, len(base), 0)
        q = base.copy()
        q[cut] += 1
        a, _ = t.match_prefix(q)
        b, _ = ot.match_prefix(q)
        assert len(a) == len(b) == cut
        assert t.dump() == ot.dump()

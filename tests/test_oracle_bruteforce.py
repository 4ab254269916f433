"""The oracle tree against brute force on tiny trees, and its invariants.

Random operation sequences over a 3-letter alphabet and short sequences:
every match is checked against the longest prefix shared with any resident
root-to-node path, and every eviction against a linear scan for the least
(priority, last_access, id) unlocked leaf, repeated leaf-inward.
"""
import copy

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle


def _path_tokens(t, nid):
    return np.concatenate([n.key for n in t.path(nid)]) if nid else np.zeros(0, np.int32)


def check_invariants(t, held):
    tree_tok = 0
    seen = set()
    prot = 0
    for nid, nd in t.nodes.items():
        if nd is t.root:
            continue
        assert len(nd.key) > 0 and len(nd.key) == len(nd.value)
        assert nd.parent.children[int(nd.key[0])] is nd
        assert nd.lock_ref >= sum(c.lock_ref for c in nd.children.values())
        for ft, c in nd.children.items():
            assert int(c.key[0]) == ft
        tree_tok += len(nd.key)
        prot += len(nd.key) if nd.lock_ref > 0 else 0
        for s in nd.value.tolist():
            assert s not in seen
            seen.add(s)
            assert not t.free[s]
    assert t.protected == prot
    assert t.evictable + t.protected == tree_tok
    assert t.num_free() + tree_tok + held == t.pool_slots


def brute_match_len(t, q):
    best = 0
    for nid in t.nodes:
        best = max(best, oracle.common_prefix_len(_path_tokens(t, nid), q))
    return best


def brute_evict(t, need):
    """Linear-scan eviction on a deep copy; returns (freed, ids evicted in order)."""
    c = copy.deepcopy(t)
    freed, order = 0, []
    while freed < need:
        cand = [n for n in c.nodes.values()
                if n is not c.root and not n.children and n.lock_ref == 0]
        if not cand:
            break
        x = min(cand, key=lambda n: (n.priority, n.last_access, n.id))
        freed += len(x.key)
        order.append(x.id)
        del x.parent.children[int(x.key[0])]
        del c.nodes[x.id]
    return freed, order


seq_st = st.lists(st.integers(0, 2), min_size=1, max_size=12)
op_st = st.one_of(
    st.tuples(st.just("insert"), seq_st),
    st.tuples(st.just("match"), seq_st),
    st.tuples(st.just("lock"), seq_st),
    st.tuples(st.just("unlock"), st.integers(0, 7)),
    st.tuples(st.just("evict"), st.integers(1, 20)),
)


@settings(max_examples=300, deadline=None)
@given(st.lists(op_st, min_size=1, max_size=30), st.integers(12, 40))
def test_random_ops_against_brute_force(ops, pool):
    t = oracle.RadixTree(pool)
    locks = []
    held = 0
    for op, arg in ops:
        if op == "insert":
            seq = np.array(arg, dtype=np.int32)
            try:
                oracle.admit_history(t, [seq])
            except oracle.NoSpace:
                pass
        elif op == "match":
            q = np.array(arg, dtype=np.int32)
            want = brute_match_len(t, q)
            got, nid = t.match_prefix(q)
            assert len(got) == want
            assert np.array_equal(_path_tokens(t, nid), q[:want])
            # the matched slots are the tree's slots along that path
            if want:
                assert np.array_equal(got, np.concatenate([n.value for n in t.path(nid)]))
        elif op == "lock":
            q = np.array(arg, dtype=np.int32)
            _g, nid = t.match_prefix(q)
            t.inc_lock_ref(nid)
            locks.append(nid)
        elif op == "unlock":
            if locks:
                t.dec_lock_ref(locks.pop(arg % len(locks)))
        elif op == "evict":
            want_freed, want_order = brute_evict(t, arg)
            before = set(t.nodes)
            freed = t.evict(arg)
            assert freed == want_freed
            assert before - set(t.nodes) == set(want_order)
        check_invariants(t, held)


def test_split_keeps_lower_id_and_lock():
    t = oracle.RadixTree(64)
    a = np.array([1, 2, 3, 4, 5], np.int32)
    oracle.admit_history(t, [a])
    _s, n = t.match_prefix(a)
    t.inc_lock_ref(n)
    got, up = t.match_prefix(a[:2])            # ends inside the edge: split after 2 tokens
    assert len(got) == 2 and up != n
    assert t.nodes[up].lock_ref == t.nodes[n].lock_ref == 1
    assert t.nodes[n].parent is t.nodes[up]
    assert t.protected == 5 and t.evictable == 0
    t.dec_lock_ref(n)
    assert t.protected == 0 and t.evictable == 5


def test_insert_over_present_tokens_frees_callers_duplicates():
    t = oracle.RadixTree(32)
    a = np.array([7, 8, 9], np.int32)
    oracle.admit_history(t, [a])               # slots 0,1,2
    mine = t.alloc(4)                          # 3,4,5,6 held by a caller that raced
    p, nid, fixed = t.insert(np.array([7, 8, 9, 10], np.int32), mine)
    assert p == 3
    assert fixed.tolist() == [0, 1, 2, 6]
    assert t.free[[3, 4, 5]].all() and not t.free[6]


def test_dec_lock_below_zero_and_stale_id():
    t = oracle.RadixTree(16)
    oracle.admit_history(t, [np.array([1, 2], np.int32)])
    _s, n = t.match_prefix(np.array([1, 2], np.int32))
    import pytest
    with pytest.raises(ValueError):
        t.dec_lock_ref(n)
    t.evict(100)
    with pytest.raises(oracle.Stale):
        t.inc_lock_ref(n)


def test_cascade_evicts_parent_after_children():
    t = oracle.RadixTree(64)
    base = [5, 5, 5]
    oracle.admit_history(t, [np.array(base + [1, 1], np.int32), np.array(base + [2, 2], np.int32)])
    assert t.stats()["nodes"] == 3
    freed = t.evict(100)
    assert freed == 7 and t.stats()["nodes"] == 0 and t.num_free() == 64

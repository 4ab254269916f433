"""Paged tree (page_size > 1): key truncation to whole pages, matches rounded down to a
page, children keyed on their first page, slots in whole pages.  The library against the
oracle on random operation sequences (bit-exact), the oracle against brute force, and
the page's rules on hand-built cases."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import radix_tree_prefix_amd as rs


def _both(pool, ps):
    return oracle.RadixTree(pool, ps), rs.Tree(pool, ps)


def test_rules_by_hand():
    """"A tree, not a map": keys truncated to a multiple of the page size, the match rounded
    down again, children keyed on the first page (a dict keyed on the page)."""
    for t in _both(64, 4):
        a = np.array([1, 2, 3, 4, 5, 6, 7, 8, 9, 10], np.int32)       # 10 tokens: 8 are kept
        s = t.alloc(10)
        assert list(s[:8]) == list(range(8)) and list(s[8:]) == [8, 9]
        pre, node, _f = t.insert(a, s)
        assert pre == 0
        t.free_slots(s[8:])                                       # the caller's partial page
        b = np.array([1, 2, 3, 9, 9, 9, 9, 9], np.int32)          # same first token, other first page
        pre, node_b, _f = t.insert(b, t.alloc(8))
        assert pre == 0                                           # no split inside a page
        got, _n = t.match_prefix(np.array([1, 2, 3, 4, 5, 6, 0, 0], np.int32))
        assert len(got) == 4 and list(got) == [0, 1, 2, 3]       # 6 shared tokens -> one page
        got, _n = t.match_prefix(np.array([1, 2, 3], np.int32))
        assert len(got) == 0                                      # less than a page
    o, c = _both(64, 4)
    for t in (o, c):
        t.insert(np.arange(1, 9, dtype=np.int32), t.alloc(8))
        t.insert(np.array([1, 2, 3, 9, 9, 9, 9, 9], np.int32), t.alloc(8))
        t.match_prefix(np.array([1, 2, 3, 4, 5, 6, 0, 0], np.int32))   # splits at the page boundary
    assert c.dump() == o.dump()
    lines = c.dump().splitlines()
    assert [l.split("|")[1].split()[:4] for l in lines if l.startswith("0 ")] == \
        [["1", "2", "3", "4"], ["1", "2", "3", "9"]]               # two root children, first pages differ


def test_alloc_takes_whole_pages_and_evicts_pages():
    o, c = _both(16, 4)
    for t in (o, c):
        assert list(t.alloc(5)) == [0, 1, 2, 3, 4]                # pages 0 and 1; 5..7 are taken too
    assert c.stats()["free_slots"] == o.stats()["free"] == 8
    for t in (o, c):
        with pytest.raises((oracle.NoSpace, rs.NoSpaceError)):
            t.alloc(9)                                            # 3 pages wanted, 2 free, nothing to evict


def test_paged_admission_continues_the_last_page():
    o, c = _both(64, 4)
    toks = np.arange(100, 110, dtype=np.int32)
    orow, onode, om = oracle.admit(o, toks, 6, 5)                 # cached 6 = a page and a half
    crow, cnode, cm = c.admit(toks, 6, 5)
    np.testing.assert_array_equal(orow, crow)
    assert (onode, om) == (cnode, cm) and om == 0
    # positions 0..3 in page 0 (inserted), 4..7 in page 1 (the request's), 8..10 in page 2
    assert list(crow) == list(range(11))
    assert c.dump() == o.dump() and c.stats()["tree_tokens"] == 4


seq_st = st.lists(st.integers(0, 2), min_size=0, max_size=14)
op_st = st.one_of(
    st.tuples(st.just("admit"), seq_st, st.integers(0, 5)),
    st.tuples(st.just("match"), seq_st, st.just(0)),
    st.tuples(st.just("lock"), seq_st, st.just(0)),
    st.tuples(st.just("unlock"), st.just([]), st.integers(0, 7)),
    st.tuples(st.just("evict"), st.just([]), st.integers(0, 20)),
    st.tuples(st.just("alloc"), st.just([]), st.integers(0, 9)),
    st.tuples(st.just("free"), st.just([]), st.integers(0, 7)),
    st.tuples(st.just("insert_held"), seq_st, st.just(0)),
)


@settings(max_examples=300, deadline=None)
@given(st.lists(op_st, min_size=1, max_size=40), st.integers(2, 10), st.sampled_from([2, 3, 4]))
def test_random_ops_match_oracle_paged(ops, pages, ps):
    pool = pages * ps
    ot, ct = _both(pool, ps)
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
                if k:
                    held.append(orow[cached:])
        elif op == "match":
            os_, on = ot.match_prefix(seq)
            cs, cn = ct.match_prefix(seq)
            assert on == cn and len(os_) % ps == 0
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
                if k:
                    held.append(a)
        elif op == "free" and held:
            s = held.pop(k % len(held))
            ot.free_slots(s)
            ct.free_slots(s)
        elif op == "insert_held" and held and len(seq) >= ps:
            # a run the caller holds, starting at a page: insert a sequence over it
            s = held[-1]
            if s[0] % ps == 0 and len(s) >= len(seq):
                held.pop()
                use = s[:len(seq)]
                p1, n1, f1 = ot.insert(seq, use)
                p2, n2, f2 = ct.insert(seq, use)
                assert (p1, n1) == (p2, n2)
                np.testing.assert_array_equal(f1, f2)
                n_al = len(seq) // ps * ps
                if len(s) > n_al:
                    held.append(s[n_al:])
        assert ct.dump() == ot.dump()
        cs, os_ = ct.stats(), ot.stats()
        assert (cs["evictable"], cs["protected"], cs["free_slots"], cs["tree_tokens"]) == \
            (os_["evictable"], os_["protected"], os_["free"], os_["tree_tokens"])


def _path_tokens(t, nid):
    return np.concatenate([n.key for n in t.path(nid)]) if nid else np.zeros(0, np.int32)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.lists(st.integers(0, 2), min_size=1, max_size=14), min_size=1, max_size=10),
       st.lists(st.integers(0, 2), min_size=0, max_size=14), st.sampled_from([2, 3, 4]))
def test_oracle_match_is_longest_page_aligned_prefix(seqs, q, ps):
    """Brute force: the match is the longest whole-page prefix shared with a resident path."""
    t = oracle.RadixTree(1200, ps)
    for s in seqs:
        s = np.array(s, np.int32)
        _row, node, _m = oracle.admit(t, s, len(s), 0)
        oracle.release_tail(t, _row)
        t.dec_lock_ref(node)
    q = np.array(q, np.int32)
    want = max([oracle.common_prefix_len(_path_tokens(t, nid), q) for nid in t.nodes] + [0]) // ps * ps
    got, nid = t.match_prefix(q)
    assert len(got) == want
    for nd in t.nodes.values():
        if nd is not t.root:
            assert len(nd.key) % ps == 0 and len(nd.key) > 0
            pg = nd.value.reshape(-1, ps)
            assert (pg[:, :1] % ps == 0).all() and (pg == pg[:, :1] + np.arange(ps)).all()
    # slot conservation: every allocated page is in the tree (admit + release_tail leave nothing held)
    assert t.num_free() + t.tree_tokens() == t.pool_slots


def test_schedule_on_paged_tree_matches_oracle():
    rng = np.random.default_rng(4)
    o, c = _both(1024, 4)
    for _ in range(6):
        s = rng.integers(0, 3, rng.integers(4, 40)).astype(np.int32)
        for t, adm in ((o, oracle.admit), (c, None)):
            if adm:
                row, node, _m = adm(t, s, len(s), 0)
                oracle.release_tail(t, row)
                t.dec_lock_ref(node)
            else:
                row, node, _m = t.admit(s, len(s), 0)
                n_al = len(s) // 4 * 4
                if n_al < len(s):
                    t.free_slots(row[n_al:n_al + 1])
                t.dec_lock_ref(node)
    assert c.dump() == o.dump()
    queue = [rng.integers(0, 3, rng.integers(0, 40)).astype(np.int32) for _ in range(30)]
    for policy in ("fcfs", "lpm", "dfs-weight"):
        got, want = c.schedule(queue, policy), oracle.schedule(o, queue, policy)
        np.testing.assert_array_equal(got[1], want[1])
        np.testing.assert_array_equal(got[0], want[0])


def test_page_size_must_divide_the_pool():
    with pytest.raises(rs.RsError):
        rs.Tree(10, 4)
    with pytest.raises(rs.RsError):
        rs.Tree(10, 0)


def test_two_tier_match_refuses_a_paged_tree():
    """The two-tier match walks one token at a time, so it needs page size 1 (the only size
    the host tier runs at): on a page-4 tree it is refused and changes nothing.  Without the
    refusal it would split inside a page and read past the caller's tokens."""
    t = rs.Tree(16, 4)
    row, node, _m = t.admit(np.arange(8, dtype=np.int32), 8, 0)
    before_dump, before_stats = t.dump(), t.stats()
    with pytest.raises(rs.RsError) as e:
        t.match2(np.arange(6, dtype=np.int32))
    assert e.value.code == rs._lib.RS_E_UNSUPPORTED
    assert t.dump() == before_dump and t.stats() == before_stats
    t.dec_lock_ref(node)


def test_two_tier_match_needs_the_host_tier():
    t = rs.Tree(16)
    t.admit(np.arange(8, dtype=np.int32), 8, 0)
    before = t.dump()
    with pytest.raises(rs.RsError) as e:
        t.match2(np.arange(6, dtype=np.int32))
    assert e.value.code == rs._lib.RS_E_INVAL
    assert t.dump() == before

"""Draft-tree verify step, host side: rs_draft_tree_build against the page's example and
the oracle (bit-exact)."""
import numpy as np
import pytest

import oracle
import radix_tree_prefix_amd as rs


def test_page_example_positions():
    # "Speculative decoding puts a tree inside the tree": depths [0, 1, 1, 2] after a
    # 7-token prompt give positions [7, 8, 8, 9]
    parents = np.array([[-1, 0, 0, 1]], np.int32)
    mask, pos, nt, ns = rs.draft_tree_build(parents, [7])
    assert list(pos[0]) == [7, 8, 8, 9]
    assert list(mask[0]) == [0b1, 0b11, 0b101, 0b1011]
    assert list(nt[0]) == [1, 3, -1, -1] and list(ns[0]) == [-1, 2, -1, -1]
    om, op, of, osb = oracle.speculative.draft_tree(parents[0], 7)
    assert op == [7, 8, 8, 9] and om == [1, 3, 5, 11] and of == [1, 3, -1, -1] and osb == [-1, 2, -1, -1]


def random_parents(rng, n):
    return np.array([-1] + [int(rng.integers(0, i)) for i in range(1, n)], np.int32)


@pytest.mark.parametrize("n", [1, 2, 16, 63, 64])
def test_build_against_oracle(n):
    rng = np.random.default_rng(n)
    B = 5
    parents = np.stack([random_parents(rng, n) for _ in range(B)])
    prefix = rng.integers(0, 5000, B).astype(np.int32)
    mask, pos, nt, ns = rs.draft_tree_build(parents, prefix)
    for b in range(B):
        om, op, of, osb = oracle.speculative.draft_tree(parents[b], int(prefix[b]))
        assert [int(x) for x in mask[b]] == om
        assert list(pos[b]) == op and list(nt[b]) == of and list(ns[b]) == osb


def test_build_rejects_bad_trees():
    with pytest.raises(rs.RsError):
        rs.draft_tree_build(np.array([[0, 0]], np.int32), [3])          # token 0 must be the root
    with pytest.raises(rs.RsError):
        rs.draft_tree_build(np.array([[-1, 1]], np.int32), [3])         # a parent must come earlier
    with pytest.raises(rs.RsError):
        rs.draft_tree_build(np.full((1, 65), 0, np.int32), [3])         # at most 64 tokens

"""Oracle for the draft-tree verify step: plain and slow.

TEST INFRASTRUCTURE ONLY (like the rest of oracle/): nothing in the product
imports it; the tests compare rs_draft_tree_build and rs_tree_verify_attention
against it.

What it follows: "SGLang: the tree, and the language nobody remembers"
(ai.thesatyajit.com), section "Speculative decoding puts a tree inside the
tree".  The verify tokens form a tree; each one attends to the prompt and to its
own ancestors only, so every branch is an independent continuation checked by one
target pass; a token's position is the prompt length plus its depth (the page's
example: depths [0, 1, 1, 2] after a 7-token prompt give positions [7, 8, 8, 9]);
the tree is also kept as first-child / next-sibling arrays.
Readings where the page is silent (the library documents the same): token 0 is the
root at depth 0 and every other token's parent comes earlier; a token sees itself;
children are listed in index order.
"""
from __future__ import annotations

import numpy as np

from .attention import attend


def ancestors_or_self(parents, i):
    """Indices on the path from token i up to the root, i included."""
    out = []
    while i >= 0:
        out.append(i)
        i = int(parents[i])
    return out


def draft_tree(parents, prefix_len):
    """(mask ints, positions, first child, next sibling) of one request's draft tree."""
    n = len(parents)
    mask = [sum(1 << j for j in ancestors_or_self(parents, i)) for i in range(n)]
    pos = [prefix_len + len(ancestors_or_self(parents, i)) - 1 for i in range(n)]
    children = [[c for c in range(n) if int(parents[c]) == p] for p in range(n)]
    first = [kids[0] if kids else -1 for kids in children]
    sibling = [-1] * n
    for kids in children:
        for a, b in zip(kids, kids[1:]):
            sibling[a] = b
    return mask, pos, first, sibling


def verify_attention(q, K_ctx, V_ctx, K_draft, V_draft, parents, sm_scale):
    """q [n, Hq, D] of the verify tokens; K/V_ctx [prefix, Hkv, D]; K/V_draft [n, Hkv, D].

    Token i attends to the whole prefix and to the verify tokens on its root path
    (itself included), materialised as its own key list.  Returns float64 outputs."""
    n = len(parents)
    out = []
    for i in range(n):
        path = sorted(ancestors_or_self(parents, i))
        K = np.concatenate([K_ctx, K_draft[path]])
        V = np.concatenate([V_ctx, V_draft[path]])
        o, _ = attend(q[i:i + 1], K, V, [len(K) - 1], sm_scale)
        out.append(o[0])
    return np.stack(out) if out else np.zeros((0,) + q.shape[1:])

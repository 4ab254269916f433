"""Oracle for the cache-aware ordering of a waiting queue: plain and slow.

TEST INFRASTRUCTURE ONLY (like the rest of oracle/): nothing in the product
imports it; the tests compare the library's rs_schedule against it.

What it follows: "SGLang: the tree, and the language nobody remembers"
(ai.thesatyajit.com), section "The scheduler is where the cache is won or lost".
 * Longest prefix match sorts the waiting queue by the number of prompt tokens
   already in the tree, most first.
 * A request whose real match is thin (at most 32 tokens) is looked up in a second
   radix tree built over the waiting queue; if 32 or more of its tokens are found
   there it is put at the very back (sort key +infinity), otherwise it is inserted
   into that queue tree.  The longest-prefix policy falls back to arrival order above
   128 waiting requests.
 * Depth-first weighting gives each tree node the number of waiting requests hanging
   off it and emits the queue in a weighted depth-first order.
Readings where the page is silent (the same ones the library documents): matching
for scheduling reads the tree without splitting or touching it; a request hangs off
the deepest node whose whole root path it matches; ties keep arrival order; heavier
subtrees first, equal weights by ascending first token, a node's own requests after
its subtrees.
"""
from __future__ import annotations

import numpy as np

from .tree import common_prefix_len

THIN = 32            # "IN_BATCH_PREFIX_CACHING_CHECK_THRESHOLD" and the deprioritise threshold
LPM_MAX_QUEUE = 128


def peek_match(tree, tokens):
    """(matched length, deepest node fully matched) without changing the tree."""
    tokens = np.asarray(tokens, dtype=np.int32)
    node, pos = tree.root, 0
    while tree._has_page(tokens, pos) and tree._ckey(tokens, pos) in node.children:
        child = node.children[tree._ckey(tokens, pos)]
        k = common_prefix_len(child.key, tokens[pos:]) // tree.ps * tree.ps
        pos += k
        if k < len(child.key):
            break
        node = child
    return pos, node


def _lpm(queue, matched):
    kept = []                  # the queue tree: thin requests not put back, in arrival order
    back = set()
    for i, tok in enumerate(queue):
        if matched[i] > THIN:
            continue
        in_queue = max((common_prefix_len(np.asarray(queue[j], np.int32), np.asarray(tok, np.int32))
                        for j in kept), default=0)
        if in_queue >= THIN:
            back.add(i)
        else:
            kept.append(i)
    key = lambda i: float("inf") if i in back else -matched[i]
    return sorted(range(len(queue)), key=key)          # Python's sort is stable


def _dfs_weight(tree, nodes):
    own = {}
    for i, nd in enumerate(nodes):
        own.setdefault(nd.id, []).append(i)

    def weight(nd):            # requests at this node or below it
        return len(own.get(nd.id, [])) + sum(weight(c) for c in nd.children.values())

    out = []

    def visit(nd):
        kids = [(weight(c), tree._ckey(c.key, 0), c) for c in nd.children.values()]
        kids = [k for k in kids if k[0] > 0]
        kids.sort(key=lambda k: (-k[0], k[1]))
        for _, _, c in kids:
            visit(c)
        out.extend(own.get(nd.id, []))

    visit(tree.root)
    return out


def schedule(tree, queue, policy="lpm"):
    """Returns (order, matched) for a list of token sequences."""
    peeks = [peek_match(tree, q) for q in queue]
    matched = [m for m, _ in peeks]
    if policy == "lpm" and len(queue) > LPM_MAX_QUEUE:
        policy = "fcfs"
    if policy == "fcfs":
        order = list(range(len(queue)))
    elif policy == "lpm":
        order = _lpm(queue, matched)
    elif policy == "dfs-weight":
        order = _dfs_weight(tree, [nd for _, nd in peeks])
    else:
        raise ValueError(policy)
    return np.array(order, np.int32), np.array(matched, np.int64)

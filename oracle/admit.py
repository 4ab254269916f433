"""Oracle admission: the request lifecycle on the oracle tree, and prefill accounting.

TEST INFRASTRUCTURE ONLY.  Nothing in the product imports this module.

Follows "How does SGLang work" (modernaiengineering.com), section "What
happens when a request arrives": match the longest prefix, lock it, prefill
only the rest, insert the new tokens, unlock.  Slot shortage evicts to fit
("Worked example, step by step"); when nothing can be evicted the request
waits, which here is the NoSpace exception.

Batch admission of one request with ``cached`` tokens to (re)establish and
``new`` tokens to compute: match tokens[:cached] and lock the node; allocate
slots for the unmatched cached part (re-prefill after an eviction); insert
the cached part and move the lock to the node it ends at; allocate the new
tokens' slots.  The request's index-table row is the ``cached + new`` slots.

With pages (page_size ps > 1) the tree holds whole pages only: the cached part's
slots come as whole pages, the last of which the request keeps when the cached
tokens end inside it; its new tokens continue that page before taking fresh pages.
"""
from __future__ import annotations

import numpy as np

from .tree import RadixTree, NoSpace  # noqa: F401


def admit(tree: RadixTree, tokens, cached: int, new: int):
    """Admit one request.  Returns (row slots int32 [cached+new], locked node id, matched len).

    The slots of positions matched..cached-1 are fresh and need their KV written
    (re-prefill); so do positions cached..cached+new-1.
    """
    tokens = np.asarray(tokens, dtype=np.int32)
    assert len(tokens) >= cached
    got, node = tree.match_prefix(tokens[:cached])
    m = len(got)
    tree.inc_lock_ref(node)
    row = np.empty(cached + new, dtype=np.int32)
    row[:m] = got
    ps = tree.ps
    tail = 0                        # slots left in the request's last page after `cached`
    try:
        if cached > m:
            row[m:cached] = tree.alloc(cached - m)
            if cached % ps:
                tail = ps - cached % ps
            _p, node2, fixed = tree.insert(tokens[:cached], row[:cached])
            row[:cached] = fixed
            tree.inc_lock_ref(node2)
            tree.dec_lock_ref(node)
            node = node2
        if new:
            k = min(new, tail)
            if k:
                row[cached:cached + k] = row[cached - 1] + 1 + np.arange(k)
            if new > k:
                row[cached + k:] = tree.alloc(new - k)
    except NoSpace:
        # the request waits: drop its lock and its own last page; whatever was
        # inserted stays cached
        if tail:
            tree.free_slots(row[cached - 1:cached])
        tree.dec_lock_ref(node)
        raise
    return row, node, m


def release_tail(tree: RadixTree, row):
    """Free the request's own last page: the positions past its last whole page, which the
    tree never holds (nothing to do with page size 1)."""
    n_al = len(row) // tree.ps * tree.ps
    if n_al < len(row):
        tree.free_slots(row[n_al:n_al + 1])


def release(tree: RadixTree, tokens, row, node):
    """End of a request: insert everything it computed, then unlock its old node."""
    tokens = np.asarray(tokens, dtype=np.int32)
    _p, _n, fixed = tree.insert(tokens[:len(row)], row)
    tree.dec_lock_ref(node)
    return fixed


def admit_history(tree: RadixTree, seqs, on_new=None):
    """Admit and release each sequence in order (prefill whatever is not cached).

    on_new(seq_index, tokens, lo, slots) is called for every fresh run of slots
    that needs KV written.  Returns the number of tokens prefilled.
    """
    prefilled = 0
    for i, s in enumerate(seqs):
        row, node, m = admit(tree, s, len(s), 0)
        if on_new is not None and len(s) > m:
            on_new(i, s, m, row[m:])
        prefilled += len(s) - m
        tree.dec_lock_ref(node)
    return prefilled


def admit_batch(tree: RadixTree, wl, on_new=None):
    """Admit every request of a workload in order and fill its index table.

    Returns dict(table int32 [B, ld] padded with -1, nodes, matched, reprefill).
    on_new(request, lo, slots) is called for every run of slots that needs KV
    written (re-prefilled cached positions and the new tokens).
    """
    B = wl.B
    ld = max(r.seq_len for r in wl.requests)
    table = np.full((B, ld), -1, dtype=np.int32)
    nodes = np.zeros(B, dtype=np.int64)
    matched = np.zeros(B, dtype=np.int64)
    reprefill = 0
    for r in wl.requests:
        row, node, m = admit(tree, r.tokens, r.cached, r.new)
        table[r.row, :len(row)] = row
        nodes[r.row] = node
        matched[r.row] = m
        reprefill += r.cached - m
        if on_new is not None:
            on_new(r, m, row[m:])
    return {"table": table, "nodes": nodes, "matched": matched, "reprefill": reprefill, "ld": ld}


# ----------------------------------------------------------------- accounting
def prefill_no_sharing(seqs) -> int:
    """Every request prefills its whole prompt."""
    return int(sum(len(s) for s in seqs))


def prefill_sequential(seqs, pool_slots=None) -> int:
    """Requests run one after another over one tree: each prefills what it did not match."""
    total = int(sum(len(s) for s in seqs))
    tree = RadixTree(pool_slots or max(total, 1))
    return admit_history(tree, seqs)


def prefill_fixed_prefix(seqs, prefix) -> int:
    """Only one hoisted block is cached (computed once); everything after it is per request."""
    tree = RadixTree(int(sum(len(s) for s in seqs)) + len(prefix))
    n = admit_history(tree, [prefix])
    for s in seqs:
        got, node = tree.match_prefix(s)
        n += len(s) - len(got)
    return n

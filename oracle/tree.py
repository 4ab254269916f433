"""Oracle radix tree over token prefixes: plain, slow, obviously correct.

TEST INFRASTRUCTURE ONLY.  Nothing in the product imports this module; only
tests/, the smoke check and the bench's CPU-baseline leg call it.

What it follows (pages as given, sections named):

* "SGLang: the tree, and the language nobody remembers" (ai.thesatyajit.com),
  section "A tree, not a map": a radix tree over token prefixes whose nodes
  carry a key (token run), a value (one KV slot per token), children keyed on
  the first token, lock_ref, last-access time and priority; a node splits at
  the divergence point; inc/dec of lock_ref moves len(key) between the
  evictable and protected totals on the 0<->1 edge; eviction pops evictable
  leaves off a heap and pushes a parent that became childless and unlocked.
* "SGLang" (bibekananda.in), sections "One tree for everybody" and "Eviction
  on a tree": walk from the root while tokens match, everything matched is
  reuse; eviction runs from the leaves inward.
* "How does SGLang work" (modernaiengineering.com), sections "What happens
  when a request arrives" (match, lock, prefill the rest, insert, unlock)
  and "Worked example, step by step" (least recently used unlocked leaf goes
  first, a node is evicted whole, nothing evictable means the request waits).

Paged variant, same page ("SGLang: the tree, ...", section "A tree, not a
map", the two details from the source): with page_size > 1 every key is
truncated to a multiple of the page size, a match is rounded down to one, and
a node's children are keyed on their first page (all page_size tokens).
Readings for it: slots come in whole pages (page p holds slots p*ps ..
p*ps+ps-1, lowest free pages first, a page is freed whole); a request's
tokens that do not fill a page stay with the request (its last page, which
later tokens continue) and are not inserted.

Two-tier variant, same page, section "What the C++ tree is actually for": a
host tier of slots beside the device pool; a node is on the device, on the
host or both; a match reports the device part and the host part with a node
per tier; writes to the host and loads back are transactions resolved by a
later commit (only the write's commit carries a success flag); device
eviction counts device-resident children only.  Readings for it: page size 1;
a write-through covers the root path and locks it until the commit; a device
leaf with a committed host copy leaves the device only, one without leaves the
tree with its host-only subtree; host eviction drops host-only leaves in the
device order; an insert over a host-only node gives it the caller's slots.

Readings where the pages are silent (each listed in the design notes):
page_size 1 unless asked; a logical clock that ticks once per match/insert call and
stamps every node the call visits; heap key (priority, last_access, node id)
with priority 0; splits in both match and insert, the new upper node taking
a fresh id and the lower node's lock_ref and last_access; lowest-free-first
slot allocation; insert over present tokens keeps the tree's slots and frees
the caller's differing ones; node ids are never reused, root = 0.
"""
from __future__ import annotations

import numpy as np


class NoSpace(Exception):
    """Allocation could not be satisfied even after evicting every evictable node."""


class Stale(Exception):
    """A node id that no longer names a node in the tree."""


class Node:
    __slots__ = ("id", "key", "value", "children", "parent", "lock_ref", "last_access", "priority", "host",
                 "pend")

    def __init__(self, nid, key, value, parent):
        self.id = nid
        self.key = np.asarray(key, dtype=np.int32)
        self.value = np.asarray(value, dtype=np.int32)    # device slots; empty: the node is on the host only
        self.host = np.zeros(0, np.int32)                  # host slots; empty: no host copy
        self.pend = 0                                      # ticket of a copy in flight, 0 if none
        self.children = {}          # first token -> Node
        self.parent = parent
        self.lock_ref = 0
        self.last_access = 0
        self.priority = 0


def common_prefix_len(a: np.ndarray, b: np.ndarray) -> int:
    """Number of leading positions where a and b agree."""
    n = min(len(a), len(b))
    if n == 0:
        return 0
    diff = np.flatnonzero(a[:n] != b[:n])
    return int(diff[0]) if len(diff) else n


class RadixTree:
    def __init__(self, pool_slots: int, page_size: int = 1):
        self.pool_slots = int(pool_slots)
        self.ps = int(page_size)
        assert self.ps >= 1 and self.pool_slots % self.ps == 0
        self.root = Node(0, [], [], None)
        self.nodes = {0: self.root}
        self.next_id = 1
        self.clock = 0
        self.free = np.ones(self.pool_slots, dtype=bool)   # True = slot is free
        self.evictable = 0
        self.protected = 0
        self.evicted_total = 0
        self.host_slots = 0                 # host tier off until enable_host
        self.host_free = np.zeros(0, bool)
        self.tickets = {}                   # ticket -> (kind, node id locked for it)
        self.next_ticket = 1

    # ---------------------------------------------------------------- helpers
    def _node(self, nid) -> Node:
        n = self.nodes.get(int(nid))
        if n is None:
            raise Stale(nid)
        return n

    def _new_id(self) -> int:
        i = self.next_id
        self.next_id += 1
        return i

    def _ckey(self, tokens, pos):
        """Child key of the edge starting at tokens[pos]: its first token (page size 1)
        or its first page."""
        if self.ps == 1:
            return int(tokens[pos])
        return tuple(int(x) for x in tokens[pos:pos + self.ps])

    def _has_page(self, tokens, pos):
        return pos + self.ps <= len(tokens)

    def _split(self, child: Node, k: int) -> Node:
        """Cut child's edge after k tokens; the new upper node is returned."""
        upper = Node(self._new_id(), child.key[:k], child.value[:k], child.parent)
        upper.lock_ref = child.lock_ref
        upper.last_access = child.last_access
        upper.priority = child.priority
        upper.host, upper.pend = child.host[:k], child.pend
        child.host = child.host[k:]
        upper.parent.children[self._ckey(child.key, 0)] = upper
        child.key = child.key[k:]
        child.value = child.value[k:]
        child.parent = upper
        upper.children[self._ckey(child.key, 0)] = child
        self.nodes[upper.id] = upper
        return upper

    # ---------------------------------------------------------------- match
    def match_prefix(self, tokens):
        """Longest cached prefix of `tokens`.  Returns (slots, node id)."""
        tokens = np.asarray(tokens, dtype=np.int32)
        self.clock += 1
        node, pos, got = self.root, 0, []
        while self._has_page(tokens, pos) and self._ckey(tokens, pos) in node.children:
            child = node.children[self._ckey(tokens, pos)]
            if not len(child.value):        # on the host only: not a device match
                break
            child.last_access = self.clock
            k = common_prefix_len(child.key, tokens[pos:]) // self.ps * self.ps
            if k < len(child.key):
                child = self._split(child, k)
            got.append(child.value)
            pos += k
            node = child
        slots = np.concatenate(got) if got else np.zeros(0, np.int32)
        return slots, node.id

    # ---------------------------------------------------------------- insert
    def insert(self, tokens, slots):
        """Insert tokens with their slots.  Returns (prefix_len, node id, slots).

        prefix_len tokens were already present; for them the tree's slots are
        kept, any differing caller slot is freed, and the returned slots array
        carries the tree's ids.  The remaining slots are adopted by a new leaf.
        """
        tokens = np.asarray(tokens, dtype=np.int32)
        slots = np.array(slots, dtype=np.int32, copy=True)
        assert len(tokens) == len(slots)
        n = len(tokens) // self.ps * self.ps          # whole pages only
        tokens = tokens[:n]
        # slots come in whole pages, aligned with the positions: slot of position j is
        # page * ps + j % ps, one page per group of ps positions
        pg = slots[:n].reshape(-1, self.ps) if n else np.zeros((0, self.ps), np.int32)
        assert (pg[:, :1] % self.ps == 0).all() and (pg == pg[:, :1] + np.arange(self.ps)).all(), \
            "slots are not whole pages"
        self.clock += 1
        node, pos = self.root, 0
        while self._has_page(tokens, pos) and self._ckey(tokens, pos) in node.children:
            child = node.children[self._ckey(tokens, pos)]
            child.last_access = self.clock
            k = common_prefix_len(child.key, tokens[pos:]) // self.ps * self.ps
            if k < len(child.key):
                child = self._split(child, k)
            seg = slots[pos:pos + k]
            if not len(child.value):        # on the host only: it takes the caller's device slots
                child.value = seg.copy()
                if child.lock_ref > 0:
                    self.protected += k
                else:
                    self.evictable += k
            differ = seg != child.value
            if differ.any():
                self._free(seg[differ])
                seg[differ] = child.value[differ]
            pos += k
            node = child
        prefix = pos
        if pos < n:
            leaf = Node(self._new_id(), tokens[pos:n], slots[pos:n], node)
            leaf.last_access = self.clock
            node.children[self._ckey(tokens, pos)] = leaf
            self.nodes[leaf.id] = leaf
            self.evictable += len(leaf.key)
            node = leaf
        return prefix, node.id, slots

    # ---------------------------------------------------------------- locks
    def inc_lock_ref(self, nid):
        node = self._node(nid)
        while node is not self.root:
            if node.lock_ref == 0:
                self.evictable -= len(node.value)
                self.protected += len(node.value)
            node.lock_ref += 1
            node = node.parent

    def dec_lock_ref(self, nid):
        node = self._node(nid)
        if node is not self.root and node.lock_ref <= 0:
            raise ValueError("dec_lock_ref below zero")
        while node is not self.root:
            if node.lock_ref == 1:
                self.evictable += len(node.value)
                self.protected -= len(node.value)
            node.lock_ref -= 1
            node = node.parent

    # ---------------------------------------------------------------- slots
    def _free(self, slots):
        """Free the pages that hold these slots (each page whole)."""
        pages = np.unique(np.asarray(slots, dtype=np.int64) // self.ps)
        first = pages * self.ps
        assert not self.free[first].any(), "double free"
        for p in pages:
            self.free[p * self.ps:(p + 1) * self.ps] = True

    def free_slots(self, slots):
        self._free(slots)

    def num_free(self) -> int:
        return int(self.free.sum())

    def alloc(self, n: int) -> np.ndarray:
        """n slots from the lowest free whole pages (ceil(n/ps) pages, page-major); evicts to
        fit; NoSpace if it cannot.  The unused end of the last page belongs to the caller too."""
        n = int(n)
        need = -(-n // self.ps) * self.ps
        have = self.num_free()
        if have < need:
            self.evict(need - have)
            if self.num_free() < need:
                raise NoSpace(n)
        pages = np.flatnonzero(self.free[::self.ps])[:need // self.ps]
        got = (pages[:, None] * self.ps + np.arange(self.ps)[None, :]).reshape(-1)
        self.free[got] = False
        return got[:n].astype(np.int32)

    # ---------------------------------------------------------------- evict
    @staticmethod
    def _device_leaf(nd):
        """On the device, unlocked, and no child on the device."""
        return len(nd.value) > 0 and nd.lock_ref == 0 and not any(len(c.value) for c in nd.children.values())

    def _evictable_leaves(self):
        return [nd for nd in self.nodes.values() if nd is not self.root and self._device_leaf(nd)]

    def evict(self, num_tokens: int) -> int:
        """Evict whole unlocked device leaves, least key first, until num_tokens are freed.  A
        node with a finished host copy stays, on the host only; any other leaves the tree."""
        import heapq
        heap = [(nd.priority, nd.last_access, nd.id) for nd in self._evictable_leaves()]
        heapq.heapify(heap)
        freed = 0
        while freed < num_tokens and heap:
            _p, _t, nid = heapq.heappop(heap)
            x = self.nodes[nid]
            self._free(x.value)
            freed += len(x.value)
            self.evictable -= len(x.value)
            parent = x.parent
            if len(x.host) and x.pend == 0:
                x.value = np.zeros(0, np.int32)
            else:
                self._drop_subtree(x)       # what is left below is on the host only: it goes too
                del parent.children[self._ckey(x.key, 0)]
                del self.nodes[nid]
            if parent is not self.root and self._device_leaf(parent):
                heapq.heappush(heap, (parent.priority, parent.last_access, parent.id))
        self.evicted_total += freed
        return freed

    # ---------------------------------------------------------------- host tier
    # "SGLang: the tree, ..." (ai.thesatyajit.com), "What the C++ tree is actually for": a
    # second tier in host memory; a match also reports how far it runs on the host, with
    # a node handle per tier; copies to the host (writing through) and back (loading) are
    # transactions that a later commit resolves; nodes are on the GPU, on the CPU or both.
    def enable_host(self, host_slots: int):
        assert self.ps == 1 and self.host_slots == 0 and host_slots > 0
        self.host_slots = int(host_slots)
        self.host_free = np.ones(self.host_slots, bool)

    def _host_leaves(self):
        return [nd for nd in self.nodes.values()
                if nd is not self.root and not len(nd.value) and not nd.children and nd.lock_ref == 0
                and nd.pend == 0]

    def evict_host(self, num_tokens: int) -> int:
        """Drop host-only leaves, least (priority, last_access, id) first, until num_tokens host
        slots are freed; a parent left a host-only leaf follows."""
        import heapq
        heap = [(nd.priority, nd.last_access, nd.id) for nd in self._host_leaves()]
        heapq.heapify(heap)
        freed = 0
        while freed < num_tokens and heap:
            _p, _t, nid = heapq.heappop(heap)
            x = self.nodes[nid]
            self.host_free[x.host] = True
            freed += len(x.host)
            parent = x.parent
            del parent.children[self._ckey(x.key, 0)]
            del self.nodes[nid]
            if (parent is not self.root and not len(parent.value) and not parent.children
                    and parent.lock_ref == 0 and parent.pend == 0):
                heapq.heappush(heap, (parent.priority, parent.last_access, parent.id))
        return freed

    def _drop_subtree(self, x):
        for c in list(x.children.values()):
            assert not len(c.value) and c.lock_ref == 0 and c.pend == 0
            self._drop_subtree(c)
            self.host_free[c.host] = True
            del self.nodes[c.id]
        x.children.clear()

    def _alloc_host(self, n):
        have = int(self.host_free.sum())
        if have < n:
            self.evict_host(n - have)
            if int(self.host_free.sum()) < n:
                raise NoSpace(n)
        got = np.flatnonzero(self.host_free)[:n]
        self.host_free[got] = False
        return got.astype(np.int32)

    def match2(self, tokens):
        """(device slots, host slots, device length, total length, device node, last node): the
        device match as match_prefix, continued through nodes that are on the host only."""
        tokens = np.asarray(tokens, dtype=np.int32)
        self.clock += 1
        node, pos, dev, host = self.root, 0, [], []
        dev_node, dev_len = self.root, 0
        while pos < len(tokens) and int(tokens[pos]) in node.children:
            child = node.children[int(tokens[pos])]
            child.last_access = self.clock
            k = common_prefix_len(child.key, tokens[pos:])
            if k < len(child.key):
                child = self._split(child, k)
            if len(child.value) and dev_len == pos:
                dev.append(child.value)
                dev_node, dev_len = child, pos + k
            else:
                host.append(child.host)
            pos += k
            node = child
        cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int32)
        return cat(dev), cat(host), dev_len, pos, dev_node.id, node.id

    def write_through(self, nid):
        """Host copies for the device nodes on nid's root path that have none: returns (device
        slots, host slots, ticket); the path stays locked until commit."""
        path = self.path(nid)
        assert all(len(nd.value) for nd in path), "write-through of a node not on the device"
        todo = [nd for nd in path if not len(nd.host) and nd.pend == 0]
        need = sum(len(nd.key) for nd in todo)
        if need > self.host_slots:                # can never fit: fail before evicting anything
            raise NoSpace(need)
        got = self._alloc_host(need)
        t = self.next_ticket
        self.next_ticket += 1
        src, dst, o = [], [], 0
        for nd in todo:
            nd.host = got[o:o + len(nd.key)]
            nd.pend = t
            o += len(nd.key)
            src.append(nd.value)
            dst.append(nd.host)
        self.inc_lock_ref(nid)
        self.tickets[t] = ("write", nid)
        cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int32)
        return cat(src), cat(dst), t

    def load_back(self, nid):
        """Device slots for the nodes on nid's root path that are on the host only: returns
        (host slots, device slots, ticket); the path stays locked until commit."""
        path = self.path(nid)
        todo = [nd for nd in path if not len(nd.value)]
        if sum(len(nd.key) for nd in todo) > self.pool_slots:   # can never fit
            raise NoSpace(sum(len(nd.key) for nd in todo))
        self.inc_lock_ref(nid)
        try:
            got = self.alloc(sum(len(nd.key) for nd in todo))
        except NoSpace:
            self.dec_lock_ref(nid)
            raise
        t = self.next_ticket
        self.next_ticket += 1
        src, dst, o = [], [], 0
        for nd in todo:
            nd.value = got[o:o + len(nd.key)]
            nd.pend = t
            o += len(nd.key)
            self.protected += len(nd.key)          # the path is locked
            src.append(nd.host)
            dst.append(nd.value)
        self.tickets[t] = ("load", nid)
        cat = lambda xs: np.concatenate(xs) if xs else np.zeros(0, np.int32)
        return cat(src), cat(dst), t

    def commit(self, ticket, success=True):
        """Resolve a copy.  A write-through that failed gives its host slots back; either way
        the path is unlocked.  Only the write-through's commit carries an outcome on the page: a
        load back is committed once its copy has run, and a failed one is refused."""
        kind, nid = self.tickets[ticket]
        if kind == "load" and not success:
            raise ValueError("a load back is committed after its copy has run")
        del self.tickets[ticket]
        for nd in list(self.nodes.values()):
            if nd is self.root or nd.pend != ticket:
                continue
            nd.pend = 0
            if not success:
                self.host_free[nd.host] = True
                nd.host = np.zeros(0, np.int32)
        self.dec_lock_ref(nid)

    # ---------------------------------------------------------------- views
    def path(self, nid):
        """Nodes from the root's child down to nid."""
        out, node = [], self._node(nid)
        while node is not self.root:
            out.append(node)
            node = node.parent
        return out[::-1]

    def tree_tokens(self) -> int:
        """Tokens on the device."""
        return sum(len(nd.value) for nd in self.nodes.values())

    def stats(self) -> dict:
        return {
            "nodes": len(self.nodes) - 1,
            "tree_tokens": self.tree_tokens(),
            "evictable": self.evictable,
            "protected": self.protected,
            "free": self.num_free(),
            "evicted_total": self.evicted_total,
            "clock": self.clock,
            "host_tokens": sum(len(nd.host) for nd in self.nodes.values()),
            "host_free": int(self.host_free.sum()),
        }

    def dump(self) -> str:
        """Canonical text: depth-first, children in ascending first-token order.

        One line per node: depth id lock_ref last_access len | key tokens | slots
        """
        lines = []

        def walk(nd, depth):
            for ft in sorted(nd.children):            # first tokens, or first pages as tuples
                c = nd.children[ft]
                line = "%d %d %d %d %d | %s | %s" % (
                    depth, c.id, c.lock_ref, c.last_access, len(c.key),
                    " ".join(map(str, c.key.tolist())), " ".join(map(str, c.value.tolist())))
                if self.host_slots:
                    line += " | %s | %d" % (" ".join(map(str, c.host.tolist())), c.pend)
                lines.append(line)
                walk(c, depth + 1)

        walk(self.root, 0)
        return "\n".join(lines) + ("\n" if lines else "")

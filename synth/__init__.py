"""Seeded synthetic workloads for the radix-tree prefix cache and its attention path.

This module is shared by the oracle side and the GPU side, so it holds only
input generation: token sequences shaped like the pages' workloads, the batch
layout, and the value tables from which Q, K and V rows are drawn.  It holds
none of the method's arithmetic: no matching, splitting, locking, allocation,
eviction or attention.

Workload shapes (the pages' workloads, reproduced with synthetic token ids):

* ``config1``: the two-document agent of "SGLang" (bibekananda.in),
  section "Why nesting is the point": a 900-token instruction block, two
  600-token documents shared by four requests each, 120 unique tokens per
  request.  One extend step over the 120 new tokens, fp32, 8/8 heads, d=64.
* ``config2``: the 40-call agent preamble of "SGLang" (llmdeepdive.com),
  section "Conceito": a 3,000-token shared preamble, 200 unique tokens per
  call, then one decode token each.  bf16, GQA 32/8, d=128.
* ``config3``: the multi-step shopping agent of "How does SGLang work"
  (modernaiengineering.com), section "The problem SGLang solves": a
  2,000-token instruction prefix, each step appending 200 tokens; step s
  extends 200 tokens over a cached 2,000+200(s-1).  bf16, GQA 32/8, d=128.
* ``config4``: a tree-of-thought search (the branching-search workload the
  same lesson lists among prefix-sharing programs): 4,096-token root, three
  fan-out-4 levels of 512 tokens, a 64-token leaf suffix and one decode
  token per leaf.  bf16, GQA 64/8, d=128.
* ``config5``: a large mixed batch drawn from a seeded random recursive tree
  of segments with Zipf(1.1) reuse, contexts log-uniform in [1k, 32k], half
  512-token chunked extends and half 1-token decodes, a 2^22-slot pool that
  a 1,024-sequence history overfills so that eviction runs.  bf16, GQA 64/8.

Values.  Every K/V row is a function of the token prefix that produced it
(the pages state that a token's KV entries depend only on that token and the
ones before it): a polynomial prefix hash, finalised with the SplitMix64
mixer, picks a row of a seeded N(0,1) table.  Q rows are drawn the same way
from their own table.  bf16 workloads round the tables to bf16
(round-to-nearest-even) once; every consumer reads the rounded values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

VOCAB = 32000
_M64 = (1 << 64) - 1
_HASH_BASE = 0x9E3779B97F4A7C15 | 1          # odd, so invertible mod 2^64
_SALT_K = 0x243F6A8885A308D3
_SALT_V = 0x13198A2E03707344
_SALT_Q = 0xA4093822299F31D0


# --------------------------------------------------------------------------
# workload description
# --------------------------------------------------------------------------
@dataclass
class Request:
    """One request of the batch.

    ``tokens`` holds ``cached + new`` ids: the first ``cached`` are expected
    to be (re)established in the cache at admission, the last ``new`` are
    the tokens this step computes (extend: new > 0 query tokens; decode:
    new == 1).  ``row`` is the request's row in the batch index table.
    """
    tokens: np.ndarray
    cached: int
    new: int
    kind: str
    row: int

    @property
    def seq_len(self) -> int:
        return self.cached + self.new


@dataclass
class Workload:
    name: str
    Hq: int
    Hkv: int
    D: int
    dtype: str                     # "f32" or "bf16"
    value_scale: float             # multiplier applied to the N(0,1) draws
    pool_slots: int
    history: list                  # token arrays admitted (then released) before the batch
    requests: list                 # list[Request], in admission order
    value_seed: int
    kv_table_rows: int = 65536
    q_table_rows: int = 8192
    meta: dict = field(default_factory=dict)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def B(self) -> int:
        return len(self.requests)

    def extend_requests(self):
        return [r for r in self.requests if r.kind == "extend"]

    def decode_requests(self):
        return [r for r in self.requests if r.kind == "decode"]


def _fresh(rng: np.random.Generator, n: int, avoid_first=()) -> np.ndarray:
    """n uniform token ids; the first is redrawn until it is not in avoid_first."""
    t = rng.integers(0, VOCAB, size=n, dtype=np.int64).astype(np.int32)
    if n and avoid_first:
        avoid = set(int(a) for a in avoid_first)
        while int(t[0]) in avoid:
            t[0] = np.int32(rng.integers(0, VOCAB))
    return t


def _cat(*parts) -> np.ndarray:
    return np.concatenate([np.asarray(p, dtype=np.int32) for p in parts]) if parts else np.zeros(0, np.int32)


# --------------------------------------------------------------------------
# configs
# --------------------------------------------------------------------------
def config1(seed: int = 1) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    instr = _fresh(rng, 900)
    docs = []
    for _ in range(2):
        docs.append(_fresh(rng, 600, [d[0] for d in docs]))
    tails = []
    for g in range(2):
        sib = []
        for _ in range(4):
            t = _fresh(rng, 120, [s[0] for s in sib])
            sib.append(t)
        tails.extend(sib)
    reqs, hist = [], []
    for r in range(8):
        pre = _cat(instr, docs[r // 4])
        hist.append(pre)
        reqs.append(Request(_cat(pre, tails[r]), cached=1500, new=120, kind="extend", row=r))
    return Workload("two-document agent extend (8 x 120 over a 1,500-token prefix, fp32, 8/8 heads, d64)",
                    Hq=8, Hkv=8, D=64, dtype="f32", value_scale=0.125, pool_slots=8192,
                    history=hist, requests=reqs, value_seed=1001, kv_table_rows=16384, q_table_rows=4096,
                    meta={"instr": instr, "docs": docs, "tails": tails})


def config2(seed: int = 2) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    pre = _fresh(rng, 3000)
    sufs = []
    for _ in range(40):
        sufs.append(_fresh(rng, 200, [s[0] for s in sufs]))
    reqs, hist = [], []
    for i in range(40):
        ctx = _cat(pre, sufs[i])
        hist.append(ctx)
        reqs.append(Request(_cat(ctx, _fresh(rng, 1)), cached=3200, new=1, kind="decode", row=i))
    return Workload("agent preamble decode (40 x 3,201, bf16, GQA 32/8, d128)",
                    Hq=32, Hkv=8, D=128, dtype="bf16", value_scale=1.0, pool_slots=16384,
                    history=hist, requests=reqs, value_seed=1002, meta={"preamble": pre})


def config3(seed: int = 3) -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    instr = _fresh(rng, 2000)
    hist = [instr]
    reqs = []
    firsts = []
    for u in range(64):
        s = int(rng.integers(1, 6))
        segs = [_fresh(rng, 200, firsts)]
        firsts.append(segs[0][0])
        for _ in range(s - 1):
            segs.append(_fresh(rng, 200))
        for k in range(1, s):
            hist.append(_cat(instr, *segs[:k]))
        reqs.append(Request(_cat(instr, *segs), cached=2000 + 200 * (s - 1), new=200, kind="extend", row=u))
    return Workload("multi-step agent extend (64 x 200 over 2,000-2,800 prefixes, bf16, GQA 32/8, d128)",
                    Hq=32, Hkv=8, D=128, dtype="bf16", value_scale=1.0, pool_slots=262144,
                    history=hist, requests=reqs, value_seed=1003, meta={"instr": instr})


def config4(seed: int = 4, reading: str = "A") -> Workload:
    rng = np.random.Generator(np.random.PCG64(seed))
    root = _fresh(rng, 4096)
    paths = [root]
    for _level in range(3):
        nxt = []
        for p in paths:
            kids = []
            for _ in range(4):
                kids.append(_fresh(rng, 512, [k[0] for k in kids]))
            nxt.extend(_cat(p, k) for k in kids)
        paths = nxt
    hist, reqs = [], []
    for i, p in enumerate(paths):
        if reading == "A":
            ctx = _cat(p, _fresh(rng, 64))
        else:                                   # level-3 nodes are the suffixes themselves
            ctx = p[:4096 + 2 * 512 + 64]
        hist.append(ctx)
        reqs.append(Request(_cat(ctx, _fresh(rng, 1)), cached=len(ctx), new=1, kind="decode", row=i))
    return Workload("tree-of-thought decode (64 x 5,697, bf16, GQA 64/8, d128)",
                    Hq=64, Hkv=8, D=128, dtype="bf16", value_scale=1.0, pool_slots=65536,
                    history=hist, requests=reqs, value_seed=1004, meta={"reading": reading})


def _loguniform_int(rng, lo, hi) -> int:
    return int(round(math.exp(rng.uniform(math.log(lo), math.log(hi)))))


def config5(seed: int = 5, n_requests: int = 256, n_history: int = 1024, pool_slots: int = 1 << 22,
            n_segments: int = 1024, max_ctx: int = 32768, min_ctx: int = 1024) -> Workload:
    """Large mixed batch.  The keyword sizes exist so that tests can draw a
    scaled-down instance with the same recipe; the defaults are the full one."""
    rng = np.random.Generator(np.random.PCG64(seed))
    # 1. catalogue: a random recursive tree of token segments
    parent = [-1]
    segs = [_fresh(rng, _loguniform_int(rng, 64, 4096))]
    child_firsts = {0: []}
    for k in range(1, n_segments):
        p = int(rng.integers(0, k))
        ln = _loguniform_int(rng, 64, 4096)
        t = _fresh(rng, ln, child_firsts[p])
        child_firsts[p].append(t[0])
        child_firsts[k] = []
        parent.append(p)
        segs.append(t)
    paths = []
    for k in range(n_segments):
        chain, j = [], k
        while j >= 0:
            chain.append(segs[j])
            j = parent[j]
        paths.append(_cat(*reversed(chain)))
    # 2. Zipf(1.1) popularity over ranks 1..K-1, mapped to catalogue nodes 1..K-1
    rank_to_node = rng.permutation(n_segments - 1) + 1
    w = np.arange(1, n_segments, dtype=np.float64) ** -1.1
    w /= w.sum()

    def draw(g, ext):
        L = _loguniform_int(g, min_ctx, max_ctx)
        node = int(rank_to_node[int(g.choice(n_segments - 1, p=w))])
        cached = L - ext
        path = paths[node]
        shared = min(len(path), cached)
        toks = _cat(path[:shared], _fresh(g, cached - shared), _fresh(g, ext))
        return toks, cached

    # 3. the batch: even requests extend 512 tokens, odd ones decode 1
    reqs = []
    n_ext = (n_requests + 1) // 2
    for r in range(n_requests):
        ext = 512 if r % 2 == 0 else 1
        toks, cached = draw(rng, ext)
        row = r // 2 if ext == 512 else n_ext + r // 2     # extend rows first, then decode rows
        reqs.append(Request(toks, cached=cached, new=ext, kind="extend" if ext == 512 else "decode", row=row))
    # 4. history from its own stream, admitted whole before the batch
    hrng = np.random.Generator(np.random.PCG64(1000 + seed))
    hist = []
    for _ in range(n_history):
        toks, _c = draw(hrng, 0)
        hist.append(toks)
    return Workload("mixed extend+decode batch (128 x 512-token extend + 128 decode, contexts 1k-32k, "
                    "bf16, GQA 64/8, d128, 4M-slot pool)" if n_requests == 256 else
                    f"mixed batch, scaled instance ({n_requests} requests, pool {pool_slots})",
                    Hq=64, Hkv=8, D=128, dtype="bf16", value_scale=1.0, pool_slots=pool_slots,
                    history=hist, requests=reqs, value_seed=1005)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def make(config: int, **kw) -> Workload:
    return CONFIGS[config](**kw)


# --------------------------------------------------------------------------
# values
# --------------------------------------------------------------------------
def _inv64(a: int) -> int:
    x = a
    for _ in range(6):                       # Newton: x <- x (2 - a x) mod 2^64
        x = (x * (2 - a * x)) & _M64
    assert (a * x) & _M64 == 1
    return x


_POW_CACHE: dict = {}


def _powers(n: int):
    got = _POW_CACHE.get("n", 0)
    if got < n:
        m = max(n, 2 * got, 4096)
        b = np.full(m, _HASH_BASE, dtype=np.uint64); b[0] = 1
        ib = np.full(m, _inv64(_HASH_BASE), dtype=np.uint64); ib[0] = 1
        _POW_CACHE.update(n=m, p=np.cumprod(b), ip=np.cumprod(ib))
    return _POW_CACHE["p"][:n], _POW_CACHE["ip"][:n]


def _mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output finaliser (Steele, Lea, Flood 2014), vectorised on uint64."""
    z = z.copy()
    z ^= z >> np.uint64(30)
    z *= np.uint64(0xBF58476D1CE4E5B9)
    z ^= z >> np.uint64(27)
    z *= np.uint64(0x94D049BB133111EB)
    z ^= z >> np.uint64(31)
    return z


def prefix_keys(tokens: np.ndarray) -> np.ndarray:
    """uint64 key of every prefix tokens[0..p]: sum_i (t_i+1) * B^(p-i) mod 2^64."""
    n = len(tokens)
    if n == 0:
        return np.zeros(0, np.uint64)
    p, ip = _powers(n)
    t = np.asarray(tokens, dtype=np.int64).astype(np.uint64) + np.uint64(1)
    return p * np.cumsum(t * ip)


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 (ties to even); returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) & np.uint32(0xFFFF0000)).view(np.float32)


class Values:
    """The seeded value tables of one workload (already rounded to its dtype).

    K/V row of the token at position p of a sequence = table[mix(key_p ^ salt) % rows];
    Q row likewise from the Q table.  All returned arrays are float32 holding
    exactly the values the device sees (bf16-representable for bf16 workloads).
    """

    def __init__(self, wl: Workload):
        self.wl = wl
        rng = np.random.Generator(np.random.PCG64(wl.value_seed))
        nkv, nq = wl.kv_table_rows, wl.q_table_rows
        wk = wl.Hkv * wl.D
        self.k_table = (rng.standard_normal((nkv, wk), dtype=np.float32) * np.float32(wl.value_scale))
        self.v_table = (rng.standard_normal((nkv, wk), dtype=np.float32) * np.float32(wl.value_scale))
        self.q_table = (rng.standard_normal((nq, wl.Hq * wl.D), dtype=np.float32) * np.float32(wl.value_scale))
        if wl.dtype == "bf16":
            self.k_table = _round_bf16(self.k_table)
            self.v_table = _round_bf16(self.v_table)
            self.q_table = _round_bf16(self.q_table)

    def kv_index(self, tokens: np.ndarray):
        key = prefix_keys(tokens)
        n = np.uint64(self.wl.kv_table_rows)
        return ((_mix64(key ^ np.uint64(_SALT_K)) % n).astype(np.int64),
                (_mix64(key ^ np.uint64(_SALT_V)) % n).astype(np.int64))

    def q_index(self, tokens: np.ndarray) -> np.ndarray:
        key = prefix_keys(tokens)
        return (_mix64(key ^ np.uint64(_SALT_Q)) % np.uint64(self.wl.q_table_rows)).astype(np.int64)

    def kv_rows(self, tokens: np.ndarray, lo: int = 0, hi: int | None = None):
        """K, V rows [n, Hkv, D] for positions lo..hi-1 of the sequence `tokens`."""
        hi = len(tokens) if hi is None else hi
        ik, iv = self.kv_index(tokens[:hi])
        s = (-1, self.wl.Hkv, self.wl.D)
        return self.k_table[ik[lo:hi]].reshape(s), self.v_table[iv[lo:hi]].reshape(s)

    def q_rows(self, tokens: np.ndarray, lo: int, hi: int) -> np.ndarray:
        """Q rows [n, Hq, D] for query positions lo..hi-1 of `tokens`."""
        iq = self.q_index(tokens[:hi])
        return self.q_table[iq[lo:hi]].reshape(-1, self.wl.Hq, self.wl.D)

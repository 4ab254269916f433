"""Pins of the oracle tree against the numbers the pages print.

Each test reads its values from a cited fixture under tests/golden/ and
reaches them through the oracle's own match / insert / lock / evict calls.
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden


def _ids(start, n):
    return np.arange(start, start + n, dtype=np.int32)


# ---------------------------------------------------------------- two-document agent
def test_two_document_agent_prefill_totals():
    g = read_golden("two_document_agent.txt")
    wl = synth.config1()
    assert len(wl.meta["instr"]) == int(g["instruction_tokens"])
    assert all(len(d) == int(g["document_tokens"]) for d in wl.meta["docs"])
    seqs = [r.tokens for r in wl.requests]
    assert len(seqs) == int(g["documents"]) * int(g["requests_per_document"])
    assert all(len(t) == int(g["unique_tokens"]) for t in wl.meta["tails"])

    none = oracle.prefill_no_sharing(seqs)
    instr = oracle.prefill_fixed_prefix(seqs, wl.meta["instr"])
    tree = oracle.prefill_sequential(seqs)
    assert none == int(g["prefill_no_sharing"])
    assert instr == int(g["prefill_instruction_only"])
    assert tree == int(g["prefill_radix_tree"])
    assert round(none / instr, 2) == float(g["ratio_instruction"])
    assert round(instr / tree, 2) == float(g["ratio_nested"])
    assert round(none / tree, 2) == float(g["ratio_total"])


def test_two_document_agent_history_plus_batch_equals_tree_total():
    """The extend workload's history (cached prefixes) plus its new tokens is the tree total."""
    g = read_golden("two_document_agent.txt")
    wl = synth.config1()
    t = oracle.RadixTree(wl.pool_slots)
    hist = oracle.admit_history(t, wl.history)
    res = oracle.admit_batch(t, wl)
    assert res["reprefill"] == 0
    assert hist + sum(r.new for r in wl.requests) == int(g["prefill_radix_tree"])
    assert all(m == 1500 for m in res["matched"])


# ---------------------------------------------------------------- agent step 5
def test_agent_step5_reuse():
    g = read_golden("agent_step5.txt")
    rng = np.random.Generator(np.random.PCG64(55))
    instr = rng.integers(0, 32000, int(g["instruction_tokens"])).astype(np.int32)
    steps = [rng.integers(0, 32000, int(g["step_tokens"])).astype(np.int32) for _ in range(int(g["step"]))]
    t = oracle.RadixTree(10000)
    for s in range(1, int(g["step"])):
        oracle.admit_history(t, [np.concatenate([instr, *steps[:s]])])
    prompt = np.concatenate([instr, *steps])
    got, _node = t.match_prefix(prompt)
    assert len(prompt) == int(g["prompt_tokens"])
    assert len(got) == int(g["reused_tokens"])
    assert round(100 * len(got) / len(prompt)) == int(g["reused_percent"])


def test_multistep_agent_workload_reuses_all_earlier_steps():
    wl = synth.config3()
    t = oracle.RadixTree(wl.pool_slots)
    oracle.admit_history(t, wl.history)
    res = oracle.admit_batch(t, wl)
    assert res["reprefill"] == 0
    for r in wl.requests:
        assert res["matched"][r.row] == r.cached


# ---------------------------------------------------------------- toy trie
def test_toy_trie_hits():
    g = read_golden("toy_trie.txt")
    reqs = [np.array([int(x) for x in s.split()], dtype=np.int32) for s in g["request"]]
    expect = [tuple(int(x) for x in e.split()) for e in g["expect"]]
    t = oracle.RadixTree(1000)
    got = []
    for r in reqs:
        slots, node = t.match_prefix(r)
        got.append((len(r), len(slots)))
        oracle.admit_history(t, [r])
    assert got == expect
    reused = sum(h for _, h in got)
    total = sum(n for n, _ in got)
    assert (reused, total) == (int(g["total_reused"]), int(g["total_tokens"]))
    assert round(100 * reused / total) == int(g["hit_percent"])


# ---------------------------------------------------------------- eviction example
def _eviction_setup(lock_a):
    g = read_golden("eviction_example.txt")
    S = _ids(0, int(g["shared_tokens"]))
    A = np.concatenate([S, _ids(10000, int(g["leaf_a"]))])
    B = np.concatenate([S, _ids(20000, int(g["leaf_b"]))])
    C = np.concatenate([S, _ids(30000, int(g["leaf_c"]))])
    t = oracle.RadixTree(int(g["capacity"]))
    oracle.admit_history(t, [A, B, C])
    assert t.tree_tokens() == int(g["tree_before"])
    nodes = {}
    for name, seq in (("A", A), ("B", B), ("C", C)):      # used in the order A, B, C
        _s, nodes[name] = t.match_prefix(seq)
    t.inc_lock_ref(nodes["C"])                             # C's request is still running
    if lock_a:
        t.inc_lock_ref(nodes["A"])
    D = np.concatenate([S, _ids(40000, int(g["new_tokens_d"]))])
    return g, t, D, nodes


def test_eviction_evicts_least_recent_unlocked_leaf():
    g, t, D, nodes = _eviction_setup(lock_a=False)
    row, nD, m = oracle.admit(t, D, int(g["shared_tokens"]), int(g["new_tokens_d"]))
    assert m == int(g["shared_tokens"])
    assert nodes["A"] not in t.nodes and nodes["B"] in t.nodes and nodes["C"] in t.nodes
    assert t.pool_slots - t.num_free() == int(g["used_after_evict_a"])
    assert t.tree_tokens() == int(g["used_after_evict_a"]) - int(g["new_tokens_d"])


def test_eviction_skips_locked_leaf():
    g, t, D, nodes = _eviction_setup(lock_a=True)
    oracle.admit(t, D, int(g["shared_tokens"]), int(g["new_tokens_d"]))
    assert nodes["A"] in t.nodes and nodes["B"] not in t.nodes
    assert t.pool_slots - t.num_free() == int(g["used_after_evict_b_when_a_locked"])


def test_eviction_all_locked_waits():
    g, t, D, nodes = _eviction_setup(lock_a=True)
    t.inc_lock_ref(nodes["B"])
    assert g["all_locked"] == "wait"
    before = t.dump()
    with pytest.raises(oracle.NoSpace):
        oracle.admit(t, D, int(g["shared_tokens"]), int(g["new_tokens_d"]))
    # nothing was evictable, so nothing changed except access times; the lock was dropped
    assert t.tree_tokens() == int(g["tree_before"])
    assert t.protected == int(g["tree_before"])
    assert len(before.splitlines()) == len(t.dump().splitlines())


# ---------------------------------------------------------------- preamble agent
def test_preamble_agent_accounting():
    g = read_golden("preamble_agent.txt")
    wl = synth.config2()
    calls, pre = int(g["calls"]), int(g["preamble_tokens"])
    assert wl.B == calls and len(wl.meta["preamble"]) == pre
    kv = int(g["kv_bytes_per_token"])
    assert round(pre * kv / 2**20) == int(g["once_mib"])
    assert round(calls * pre * kv / 2**30, 1) == float(g["copies_gib"])
    assert round((calls - 1) * pre * kv / 2**30) == int(g["recovered_gib"])
    # per layer: 64 KiB over 16 full-attention layers = K+V of 8 KV heads x 128 dims x 2 bytes
    per_layer = kv // int(g["full_attention_layers"])
    assert per_layer == 2 * wl.Hkv * wl.D * 2
    # the tree prefills the preamble once; without sharing every call prefills it
    pres = [r.tokens[:pre] for r in wl.requests]
    assert oracle.prefill_no_sharing(pres) == int(g["prefill_tokens_no_sharing"])
    assert oracle.prefill_sequential(pres) == pre
    num, den = (int(x) for x in g["prefill_saved_fraction"].split("/"))
    assert (oracle.prefill_no_sharing(pres) - oracle.prefill_sequential(pres)) * den == num * calls * pre


def test_unique_kv_tokens_decode_workloads():
    """Unique KV per decode batch: tree tokens after admission + the decode slots."""
    for cfg, want in ((2, 11040), (4, 51264)):
        wl = synth.make(cfg)
        t = oracle.RadixTree(wl.pool_slots)
        oracle.admit_history(t, wl.history)
        res = oracle.admit_batch(t, wl)
        used = set()
        for r in wl.requests:
            used.update(res["table"][r.row, :r.seq_len].tolist())
        assert len(used) == want == t.tree_tokens() + wl.B

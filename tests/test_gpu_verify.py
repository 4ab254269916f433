"""GPU parity of the draft-tree verify step: rs_tree_verify_attention against the oracle
(every verify token attends to the prompt and its own ancestors), a chain tree against
causal extend, rs_move_kv bit-exact, and the accept -> compact -> insert flow."""
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def _say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def torch_rs():
    import torch
    import radix_tree_prefix_amd as rs
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch, rs


def _bf16(x):
    return synth._round_bf16(np.asarray(x, np.float32))


def _dev(torch, a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dt)


def _parents(rng, n, chain=False):
    if chain:
        return np.arange(-1, n - 1, dtype=np.int32)
    return np.array([-1] + [int(rng.integers(0, i)) for i in range(1, n)], np.int32)


def _verify_case(torch, rs, Hq, Hkv, D, prefixes, n, seed, chain=False, far_below=False):
    """far_below: keys near +1 and queries near -16 in every dimension, so that every score
    sits far below zero (hundreds of log2-units)."""
    rng = np.random.default_rng(seed)
    B = len(prefixes)
    S = int(sum(prefixes)) + B * n + 17
    kp = _bf16(rng.standard_normal((S, Hkv, D)) * (0.5 if far_below else 1.0) + (1.0 if far_below else 0.0))
    vp = _bf16(rng.standard_normal((S, Hkv, D)))
    perm = rng.permutation(S).astype(np.int32)
    ld = max(prefixes) + n
    table = np.full((B, ld), -1, np.int32)
    off = 0
    for b, p in enumerate(prefixes):
        table[b, :p + n] = perm[off:off + p + n]
        off += p + n
    parents = np.stack([_parents(rng, n, chain) for _ in range(B)])
    mask, pos, _nt, _ns = rs.draft_tree_build(parents, np.array(prefixes, np.int32))
    q = _bf16(rng.standard_normal((B * n, Hq, D)) - (16.0 if far_below else 0.0))
    sm = 1 / np.sqrt(D)
    out = rs.tree_verify_attention(_dev(torch, q, torch.bfloat16), _dev(torch, kp, torch.bfloat16),
                                   _dev(torch, vp, torch.bfloat16), _dev(torch, table, torch.int32),
                                   _dev(torch, np.array(prefixes, np.int32), torch.int32),
                                   _dev(torch, mask.view(np.int64), torch.int64), sm)
    got = out.float().cpu().numpy()
    return dict(kp=kp, vp=vp, table=table, parents=parents, q=q, sm=sm, got=got, B=B, n=n, prefixes=prefixes)


@pytest.mark.parametrize("Hq,Hkv,D,n", [(8, 2, 128, 1), (8, 2, 128, 16), (64, 8, 128, 5), (64, 8, 128, 64),
                                        (32, 8, 64, 33), (128, 8, 128, 17), (8, 8, 64, 64)])
def test_tree_verify_against_oracle(torch_rs, Hq, Hkv, D, n):
    torch, rs = torch_rs
    prefixes = [0, 37, 1000]
    _say(f"tree verify Hq={Hq} Hkv={Hkv} D={D} n={n} prefixes={prefixes}")
    c = _verify_case(torch, rs, Hq, Hkv, D, prefixes, n, seed=n + D)
    worst = _worst_vs_oracle(c)
    assert worst <= TOL_BF16, worst


def _worst_vs_oracle(c):
    n, worst = c["n"], 0.0
    for b, p in enumerate(c["prefixes"]):
        row = c["table"][b]
        ref = oracle.speculative.verify_attention(c["q"][b * n:(b + 1) * n], c["kp"][row[:p]], c["vp"][row[:p]],
                                                  c["kp"][row[p:p + n]], c["vp"][row[p:p + n]], c["parents"][b],
                                                  c["sm"])
        worst = max(worst, float(np.abs(c["got"][b * n:(b + 1) * n] - ref).max()))
    return worst


@pytest.mark.parametrize("Hq,Hkv,D,n", [(64, 8, 128, 16), (8, 8, 64, 5)])
def test_tree_verify_scores_far_below_zero(torch_rs, Hq, Hkv, D, n):
    """Every score hundreds of log2-units below zero: weights taken against no reference
    point all underflow, and the rows must come from the pass with their true maximum."""
    torch, rs = torch_rs
    prefixes = [0, 37, 1000]
    _say(f"tree verify far below zero Hq={Hq} Hkv={Hkv} D={D} n={n}")
    c = _verify_case(torch, rs, Hq, Hkv, D, prefixes, n, seed=3 * n + D, far_below=True)
    worst = _worst_vs_oracle(c)
    assert worst <= TOL_BF16, worst


def test_chain_tree_is_causal_extend(torch_rs):
    """A draft tree that is one chain is the causal extend of its tokens: same kernel
    arithmetic in another mask mode, so the outputs agree bit for bit."""
    torch, rs = torch_rs
    prefixes, n, Hq, Hkv, D = [5, 300, 64], 24, 64, 8, 128
    _say(f"chain tree vs extend prefixes={prefixes} n={n}")
    c = _verify_case(torch, rs, Hq, Hkv, D, prefixes, n, seed=7, chain=True)
    B = len(prefixes)
    qo = np.arange(0, (B + 1) * n, n, dtype=np.int32)
    ext = rs.extend_attention(_dev(torch, c["q"], torch.bfloat16), _dev(torch, c["kp"], torch.bfloat16),
                              _dev(torch, c["vp"], torch.bfloat16), _dev(torch, c["table"], torch.int32),
                              _dev(torch, qo, torch.int32), _dev(torch, np.array(prefixes, np.int32), torch.int32),
                              _dev(torch, np.full(B, n, np.int32), torch.int32), n, c["sm"])
    np.testing.assert_array_equal(ext.float().cpu().numpy(), c["got"])


def test_move_kv_bit_exact(torch_rs):
    torch, rs = torch_rs
    _say("move_kv bf16/f32")
    rng = np.random.default_rng(3)
    for dt in (torch.bfloat16, torch.float32):
        S, Hkv, D, n = 2000, 8, 128, 300
        kp = torch.randn((S, Hkv, D), device="cuda").to(dt)
        vp = torch.randn((S, Hkv, D), device="cuda").to(dt)
        perm = rng.permutation(S).astype(np.int32)
        src, dst = perm[:n], perm[n:2 * n]
        k0, v0 = kp.cpu(), vp.cpu()
        rs.move_kv(kp, vp, _dev(torch, src, torch.int32), _dev(torch, dst, torch.int32))
        torch.cuda.synchronize()
        k1, v1 = k0.clone(), v0.clone()
        k1[torch.from_numpy(dst).long()] = k0[torch.from_numpy(src).long()]
        v1[torch.from_numpy(dst).long()] = v0[torch.from_numpy(src).long()]
        assert torch.equal(kp.cpu(), k1) and torch.equal(vp.cpu(), v1)


def test_accept_compact_insert(torch_rs):
    """Verify, accept one root-to-leaf path, compact its scattered KV into fresh slots
    (rs_move_kv), insert it into the tree: the next match returns those slots and
    their rows hold the accepted tokens' K/V."""
    torch, rs = torch_rs
    _say("accept -> compact -> insert")
    rng = np.random.default_rng(5)
    S, Hq, Hkv, D, n = 4096, 16, 4, 128, 12
    tree = rs.Tree(S)
    prompt = rng.integers(0, 32000, 200).astype(np.int32)
    row, node, _m = tree.admit(prompt, len(prompt), 0)
    draft_slots = tree.alloc(n)                      # scratch slots of the draft tokens
    kp = torch.zeros((S, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    kv_rows = _bf16(rng.standard_normal((2, len(prompt) + n, Hkv, D)))
    slots_all = np.concatenate([row, draft_slots]).astype(np.int32)
    rs.store_kv(kp, vp, _dev(torch, kv_rows[0], torch.bfloat16), _dev(torch, kv_rows[1], torch.bfloat16),
                _dev(torch, slots_all, torch.int32))
    parents = _parents(rng, n)
    mask, _pos, _nt, _ns = rs.draft_tree_build(parents[None], [len(prompt)])
    q = _bf16(rng.standard_normal((n, Hq, D)))
    table = slots_all[None]
    out = rs.tree_verify_attention(_dev(torch, q, torch.bfloat16), kp, vp, _dev(torch, table, torch.int32),
                                   _dev(torch, np.array([len(prompt)], np.int32), torch.int32),
                                   _dev(torch, mask.view(np.int64), torch.int64), 1 / np.sqrt(D))
    ref = oracle.speculative.verify_attention(q, kv_rows[0][:len(prompt)], kv_rows[1][:len(prompt)],
                                              kv_rows[0][len(prompt):], kv_rows[1][len(prompt):], parents,
                                              1 / np.sqrt(D))
    assert np.abs(out.float().cpu().numpy() - ref).max() <= TOL_BF16
    # accept the path to the deepest token
    leaf = max(range(n), key=lambda i: len(oracle.speculative.ancestors_or_self(parents, i)))
    path = sorted(oracle.speculative.ancestors_or_self(parents, leaf))
    dst = tree.alloc(len(path))
    rs.move_kv(kp, vp, _dev(torch, draft_slots[path], torch.int32), _dev(torch, dst, torch.int32))
    tree.free_slots(draft_slots)
    draft_tokens = rng.integers(0, 32000, n).astype(np.int32)
    accepted = np.concatenate([prompt, draft_tokens[path]])
    pre, new_node, fixed = tree.insert(accepted, np.concatenate([row, dst]))
    assert pre == len(prompt) and list(fixed[len(prompt):]) == list(dst)
    tree.dec_lock_ref(node)
    got_slots, _ = tree.match_prefix(accepted)
    assert list(got_slots[len(prompt):]) == list(dst)
    torch.cuda.synchronize()
    k_host = kp.float().cpu().numpy()
    np.testing.assert_array_equal(k_host[dst], kv_rows[0][len(prompt) + np.array(path)])

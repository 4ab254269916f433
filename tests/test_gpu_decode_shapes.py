"""Plan-driven (prefix-aware) decode over head shapes beyond the workloads': a seeded tree of
shared prefixes (a 700-token root, 3 branches of 300, 2 x 150 below each, then private tails
of 1-400 tokens), 37 requests, random bf16 K/V in a pool addressed through the tree's own
index tables.  Every request's output and lse against the oracle, in plan and flat mode.
Shapes: one query head per KV head, 16 and 128 query heads per KV head (the latter gives row
tiles of one request each), d64 and d128, so segments with 37 x G rows are cut into several
row tiles and unique tails of every length meet chunk boundaries."""
import sys

import numpy as np
import pytest

import oracle
from conftest import bf16_request_errors, BF16_MAX_ABS, BF16_REL_RMS, LSE_MAX_ABS

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def _bf16(x):
    import synth
    return synth._round_bf16(np.asarray(x, np.float32))


def _tree_batch(rng):
    root = rng.integers(0, 32000, 700)
    seqs = []
    for b in range(3):
        br = rng.integers(0, 32000, 300)
        for c in range(2):
            ch = rng.integers(0, 32000, 150)
            for _ in range(rng.integers(5, 8)):
                tail = rng.integers(0, 32000, int(rng.integers(1, 401)))
                seqs.append(np.concatenate([root, br, ch, tail]).astype(np.int32))
    return seqs[:37]


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 8, 128), (16, 1, 64), (64, 4, 128), (128, 1, 64), (32, 8, 64)])
def test_plan_decode_head_shapes(Hq, Hkv, D):
    import torch
    import radix_tree_prefix_amd as rs
    _say(f"plan decode shapes Hq={Hq} Hkv={Hkv} D={D}")
    rng = np.random.default_rng(Hq * 7 + Hkv + D)
    seqs = _tree_batch(rng)
    B = len(seqs)
    S = 1 << 16
    tree = rs.Tree(S)
    # history: every prompt once (its shared parts become tree nodes), then the batch admits
    # each prompt as cached plus one decode token
    for s in seqs:
        _r, node, _m = tree.admit(s, len(s), 0)
        tree.dec_lock_ref(node)
    L = np.array([len(s) + 1 for s in seqs], np.int32)
    ld = int(L.max())
    table = np.full((B, ld), -1, np.int32)
    nodes = np.zeros(B, np.int64)
    for b, s in enumerate(seqs):
        _r, nodes[b], _m = tree.admit(s, len(s), 1, out_row=table[b, :L[b]])
    kp = _bf16(rng.standard_normal((S, Hkv, D)).astype(np.float32))
    vp = _bf16(rng.standard_normal((S, Hkv, D)).astype(np.float32))
    q = _bf16(rng.standard_normal((B, Hq, D)).astype(np.float32))
    sm = 1 / np.sqrt(D)
    plan = rs.Plan(tree, nodes, L - 1, L, Hq, Hkv, D)
    assert plan.info["n_shared"] >= 3
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dt)
    kd, vd, qd = dev(kp, torch.bfloat16), dev(vp, torch.bfloat16), dev(q, torch.bfloat16)
    td, ld_ = dev(table, torch.int32), dev(L, torch.int32)
    ref = [oracle.attend(q[b:b + 1], kp[table[b, :L[b]]], vp[table[b, :L[b]]], [L[b] - 1], sm) for b in range(B)]
    for flat in (False, True):
        p = None if flat else plan
        ws = rs.DecodeWorkspace(p, B, ld, Hq, Hkv, D)
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        out = rs.decode_attention(qd, kd, vd, td, ld_, ld, sm, ws, plan=p,
                                  plan_dev=None if flat else rs.upload_plan(plan), lse=lse)
        torch.cuda.synchronize()
        got, gl = out.float().cpu().numpy(), lse.cpu().numpy()
        for b in range(B):
            mx, rel = bf16_request_errors(got[b], ref[b][0][0])
            assert mx <= BF16_MAX_ABS and rel <= BF16_REL_RMS, (flat, b, mx, rel)
            assert np.abs(gl[b] - ref[b][1][0]).max() <= LSE_MAX_ABS, (flat, b)

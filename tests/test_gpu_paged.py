"""GPU parity with index tables from a paged tree (page_size 16): the kernels read one
slot per position, so page-structured tables run through the same extend and decode
kernels; outputs against the oracle (K/V gathered through the same tables)."""
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


def test_paged_tree_extend_and_decode():
    import torch
    import radix_tree_prefix_amd as rs
    assert torch.cuda.is_available()
    ps, S, Hq, Hkv, D = 16, 1 << 14, 32, 8, 128
    _say(f"paged tree ps={ps}: extend + decode")
    rng = np.random.default_rng(21)
    tree = rs.Tree(S, ps)
    pool_k = np.zeros((S, Hkv, D), np.float32)
    pool_v = np.zeros((S, Hkv, D), np.float32)

    def fill(slots):                      # fresh K/V for newly written positions
        pool_k[slots] = synth._round_bf16(rng.standard_normal((len(slots), Hkv, D)).astype(np.float32))
        pool_v[slots] = synth._round_bf16(rng.standard_normal((len(slots), Hkv, D)).astype(np.float32))

    prompt = rng.integers(0, 32000, 333).astype(np.int32)
    row, node, m = tree.admit(prompt, len(prompt), 0)
    fill(row[m:])
    n_al = len(prompt) // ps * ps
    tree.free_slots(row[n_al:n_al + 1])   # the history request's own last page
    tree.dec_lock_ref(node)
    # batch: 3 extend requests (37..120 new tokens) and 4 decode requests over the prompt
    reqs = []
    for i in range(7):
        tail = rng.integers(0, 32000, int(rng.integers(5, 200))).astype(np.int32)
        toks = np.concatenate([prompt, tail])
        if i < 3:
            new = int(rng.integers(37, 121))
            toks = np.concatenate([toks, rng.integers(0, 32000, new).astype(np.int32)])
            cached = len(toks) - new
        else:
            new, cached = 1, len(toks) - 1
        row, node, m = tree.admit(toks, cached, new)
        assert m % ps == 0
        fill(row[m:])
        reqs.append((toks, cached, new, row, node))
    ld = max(len(r[0]) for r in reqs)
    table = np.full((len(reqs), ld), -1, np.int32)
    for b, r in enumerate(reqs):
        table[b, :len(r[3])] = r[3]
        pg = r[3][:len(r[3]) // ps * ps].reshape(-1, ps)
        assert (pg == pg[:, :1] + np.arange(ps)).all() and (pg[:, 0] % ps == 0).all()
    dev = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dt)
    kp, vp = dev(pool_k, torch.bfloat16), dev(pool_v, torch.bfloat16)
    sm = 1 / np.sqrt(D)
    # extend rows 0..2
    ext = reqs[:3]
    q_ext = synth._round_bf16(rng.standard_normal((sum(r[2] for r in ext), Hq, D)).astype(np.float32))
    qo = np.concatenate([[0], np.cumsum([r[2] for r in ext])]).astype(np.int32)
    out = rs.extend_attention(dev(q_ext, torch.bfloat16), kp, vp, dev(table[:3], torch.int32), dev(qo, torch.int32),
                              dev(np.array([r[1] for r in ext], np.int32), torch.int32),
                              dev(np.array([r[2] for r in ext], np.int32), torch.int32), max(r[2] for r in ext), sm)
    got = out.float().cpu().numpy()
    worst = 0.0
    for b, (toks, cached, new, row, _n) in enumerate(ext):
        o, _ = oracle.attend(q_ext[qo[b]:qo[b + 1]], pool_k[row], pool_v[row], cached + np.arange(new), sm)
        worst = max(worst, float(np.abs(got[qo[b]:qo[b + 1]] - o).max()))
    assert worst <= 2e-2, worst
    # decode rows 3..6 with a plan: each locked node covers the cached tokens' whole pages
    dec = reqs[3:]
    seq = np.array([len(r[0]) for r in dec], np.int32)
    cached_al = np.array([r[1] // ps * ps for r in dec], np.int32)
    plan = rs.Plan(tree, np.array([r[4] for r in dec], np.int64), cached_al, seq, Hq, Hkv, D)
    assert plan.info["n_shared"] >= 1
    q_dec = synth._round_bf16(rng.standard_normal((len(dec), Hq, D)).astype(np.float32))
    ws = rs.DecodeWorkspace(plan, len(dec), int(seq.max()), Hq, Hkv, D)
    outd = rs.decode_attention(dev(q_dec, torch.bfloat16), kp, vp, dev(table[3:], torch.int32), dev(seq, torch.int32),
                               int(seq.max()), sm, ws, plan=plan, plan_dev=rs.upload_plan(plan))
    gotd = outd.float().cpu().numpy()
    for b, (toks, cached, new, row, _n) in enumerate(dec):
        o, _ = oracle.attend(q_dec[b:b + 1], pool_k[row], pool_v[row], [len(row) - 1], sm)
        assert np.abs(gotd[b] - o[0]).max() <= 2e-2

"""Cache-aware scheduling on the GPU path: a scaled mixed batch (48 requests drawn like the
full one, a 256-sequence history overfilling a 2^20-slot pool so that eviction runs) is
ordered as a waiting queue by rs_schedule, admitted in that order, and stepped (store_kv,
extend, decode).  The order and the index tables must equal the oracle's (oracle.schedule,
then oracle.admit in that order) bit for bit, and every request's outputs the oracle's
attention, under both cache-aware policies ("The scheduler is where the cache is won or
lost", ai.thesatyajit.com; the toy of "Practice: try it yourself", modernaiengineering.com)."""
import sys

import numpy as np
import pytest

import oracle
from conftest import bf16_request_errors, BF16_MAX_ABS, BF16_REL_RMS, LSE_MAX_ABS

pytestmark = pytest.mark.gpu

SCALED = dict(n_requests=48, n_history=256, pool_slots=1 << 20)


def _say(msg):
    print(f"[gpu-test] {msg}", file=sys.stderr, flush=True)


@pytest.mark.parametrize("policy", ["lpm", "dfs-weight"])
def test_scheduled_batch_tables_and_outputs(policy):
    import torch
    import bench
    assert torch.cuda.is_available()
    _say(f"scheduled mixed batch ({policy}): setup")
    st = bench.setup(5, schedule=policy, **SCALED)
    wl = st.wl
    # the oracle: same history, same queue, same policy, admission in its own order
    _say(f"scheduled mixed batch ({policy}): oracle order and tables")
    t = oracle.RadixTree(wl.pool_slots)
    oracle.admit_history(t, wl.history)
    order, _m = oracle.schedule(t, [r.tokens[:r.cached] for r in wl.requests], policy)
    assert [int(i) for i in order] == st.admit_order
    assert st.admit_order != list(range(wl.B))            # the queue really was reordered
    ref = np.full((wl.B, max(r.seq_len for r in wl.requests)), -1, np.int32)
    for i in order:
        r = wl.requests[int(i)]
        row, _node, _hit = oracle.admit(t, r.tokens, r.cached, r.new)
        ref[r.row, :len(row)] = row
    np.testing.assert_array_equal(st.table[:, :ref.shape[1]], ref)
    assert (st.table[:, ref.shape[1]:] == -1).all()
    _say(f"scheduled mixed batch ({policy}): step")
    bench.step(st)
    torch.cuda.synchronize()
    got_e, got_d, got_l = st.out_ext.float().cpu().numpy(), st.out_dec.float().cpu().numpy(), st.lse_dec.cpu().numpy()
    qo = st.qo_indptr.cpu().numpy()
    bad = []
    for i, r in enumerate(st.ext):
        rows = np.unique(np.concatenate([[0], np.arange(15, r.new, 16), [r.new - 1]]))
        k, v = st.vals.kv_rows(r.tokens, 0, r.seq_len)
        q = st.vals.q_rows(r.tokens, r.cached, r.seq_len)[rows]
        o, _ = oracle.attend(q, k, v, r.cached + rows, wl.sm_scale)
        mx, rel = bf16_request_errors(got_e[qo[i] + rows], o)
        if mx > BF16_MAX_ABS or rel > BF16_REL_RMS:
            bad.append(("extend", i, mx, rel))
    for i, r in enumerate(st.dec):
        k, v = st.vals.kv_rows(r.tokens, 0, r.seq_len)
        q = st.vals.q_rows(r.tokens, r.seq_len - 1, r.seq_len)
        o, l = oracle.attend(q, k, v, [r.seq_len - 1], wl.sm_scale)
        mx, rel = bf16_request_errors(got_d[i], o[0])
        lerr = float(np.abs(got_l[i] - l[0]).max())
        if mx > BF16_MAX_ABS or rel > BF16_REL_RMS or lerr > LSE_MAX_ABS:
            bad.append(("decode", i, mx, rel, lerr))
    assert not bad, bad

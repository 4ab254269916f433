#!/usr/bin/env python3
"""Benchmark of RadixAttention's hot path on one MI355X.

One step = one pass of the device path over a resident batch: store the new
tokens' K/V into their pool slots, extend attention for the extend requests,
prefix-aware decode attention (plan-driven work items, then a log-sum-exp merge
kernel) for the decode requests.  The host tree admission, table build and plan build that produce
the batch are timed separately and reported (`host_ms`).

Default workload: the large mixed batch (128 x 512-token extends + 128 decodes,
contexts 1k-32k, GQA 64/8, d128, bf16, 4M-slot pool).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 5] [--no-cpu-baseline] [--no-extra]
                    [--flush]

--flush reads a 1 GiB buffer before every timed step, so that a workload small enough to
stay in L2 and the 256 MB MALL between steps is read from HBM each time; the step time is
then the sum of the per-kernel event times (the flush itself is not counted).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X dense fp32 (matrix and vector alike)


# ---------------------------------------------------------------------------- setup
class State:
    pass


def _chunks(n, size):
    for i in range(0, n, size):
        yield i, min(n, i + size)


def setup(cfg=5, device="cuda", build_plan=True, schedule=None, **wl_kw):
    """Admit a workload through librs and make its batch resident on the GPU.

    schedule=None admits the batch in request order; "lpm" / "dfs-weight" / "fcfs" admits it
    in the order rs_schedule gives its cached parts as a waiting queue on the tree the history
    left (st.admit_order); each request keeps its own table row either way."""
    import torch
    import radix_tree_prefix_amd as rs

    t_host = time.perf_counter()
    wl = synth.make(cfg, **wl_kw)
    vals = synth.Values(wl)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    S, Hq, Hkv, D = wl.pool_slots, wl.Hq, wl.Hkv, wl.D
    st = State()
    st.wl, st.vals, st.dt = wl, vals, dt
    st.tree = tree = rs.Tree(S)

    # history: admit and release every sequence; record every fresh run of slots
    runs = []
    t0 = time.perf_counter()
    for s in wl.history:
        row, node, m = tree.admit(s, len(s), 0)
        if len(s) > m:
            runs.append((s, m, len(s), row[m:].copy()))
        tree.dec_lock_ref(node)
    st.history_s = time.perf_counter() - t0

    # cache-aware ordering of the batch as a waiting queue (its cached parts) on this tree
    from radix_tree_prefix_amd._lib import pack_queue
    queue = [r.tokens[:r.cached] for r in wl.requests]
    packed = pack_queue(queue[:128])
    t0 = time.perf_counter()
    tree.schedule_packed(*packed, "lpm")
    st.sched_lpm_s = time.perf_counter() - t0
    packed = pack_queue(queue)
    t0 = time.perf_counter()
    tree.schedule_packed(*packed, "dfs-weight")
    st.sched_dfs_s = time.perf_counter() - t0
    st.sched_n = len(queue)

    # batch: admit every request (in the scheduler's order if asked), its slots straight into
    # its table row; table rows padded to 64 bytes, as an engine allocates its request-to-token pool
    order = list(range(wl.B))
    if schedule is not None:
        order = [int(i) for i in tree.schedule([r.tokens[:r.cached] for r in wl.requests], schedule)[0]]
    st.admit_order = order
    ld = -(-max(r.seq_len for r in wl.requests) // 16) * 16
    table = np.full((wl.B, ld), -1, np.int32)
    nodes = np.zeros(wl.B, np.int64)
    matched = np.zeros(wl.B, np.int64)
    t0 = time.perf_counter()
    for r in (wl.requests[i] for i in order):
        row, node, m = tree.admit(r.tokens, r.cached, r.new, out_row=table[r.row, :r.seq_len])
        nodes[r.row], matched[r.row] = node, m
        if r.cached > m:
            runs.append((r.tokens, m, r.cached, row[m:r.cached]))
    st.admit_s = time.perf_counter() - t0
    st.table, st.nodes, st.matched, st.ld = table, nodes, matched, ld

    # K/V of every written slot (last writer wins when an evicted slot was reused)
    sl, ik, iv = [], [], []
    for toks, lo, hi, slots in runs:
        a, b = vals.kv_index(toks[:hi])
        sl.append(slots); ik.append(a[lo:hi]); iv.append(b[lo:hi])
    sl = np.concatenate(sl) if sl else np.zeros(0, np.int32)
    ik = np.concatenate(ik) if ik else np.zeros(0, np.int64)
    iv = np.concatenate(iv) if iv else np.zeros(0, np.int64)
    _, first = np.unique(sl[::-1], return_index=True)
    keep = len(sl) - 1 - first
    sl, ik, iv = sl[keep], ik[keep], iv[keep]

    st.k_pool = torch.zeros((S, Hkv, D), dtype=dt, device=device)
    st.v_pool = torch.zeros((S, Hkv, D), dtype=dt, device=device)
    ktab = torch.from_numpy(vals.k_table).to(device=device, dtype=dt)
    vtab = torch.from_numpy(vals.v_table).to(device=device, dtype=dt)
    qtab = torch.from_numpy(vals.q_table).to(device=device, dtype=dt)
    for a, b in _chunks(len(sl), 1 << 18):
        s_dev = torch.from_numpy(sl[a:b]).to(device)
        kn = ktab.index_select(0, torch.from_numpy(ik[a:b]).to(device)).view(-1, Hkv, D)
        vn = vtab.index_select(0, torch.from_numpy(iv[a:b]).to(device)).view(-1, Hkv, D)
        rs.store_kv(st.k_pool, st.v_pool, kn, vn, s_dev)

    # the step's inputs: new tokens' K/V and slots, queries, lengths, tables
    ext = sorted(wl.extend_requests(), key=lambda r: r.row)
    dec = sorted(wl.decode_requests(), key=lambda r: r.row)
    if ext and dec:
        assert max(r.row for r in ext) < min(r.row for r in dec), "extend rows must precede decode rows"
    st.ext, st.dec = ext, dec
    new_slots, new_ik, new_iv, q_ext_idx, q_dec_idx = [], [], [], [], []
    for r in wl.requests:
        a, b = vals.kv_index(r.tokens[:r.seq_len])
        new_slots.append(table[r.row, r.cached:r.seq_len]); new_ik.append(a[r.cached:]); new_iv.append(b[r.cached:])
    for r in ext:
        q_ext_idx.append(vals.q_index(r.tokens[:r.seq_len])[r.cached:])
    for r in dec:
        q_dec_idx.append(vals.q_index(r.tokens[:r.seq_len])[r.seq_len - 1:])
    new_slots = np.concatenate(new_slots)
    st.n_new = len(new_slots)
    st.new_slots = torch.from_numpy(new_slots).to(device)
    st.k_new = ktab.index_select(0, torch.from_numpy(np.concatenate(new_ik)).to(device)).view(-1, Hkv, D)
    st.v_new = vtab.index_select(0, torch.from_numpy(np.concatenate(new_iv)).to(device)).view(-1, Hkv, D)
    st.table_dev = torch.from_numpy(table).to(device)
    n_ext = len(ext)
    if ext:
        st.q_ext = qtab.index_select(0, torch.from_numpy(np.concatenate(q_ext_idx)).to(device)).view(-1, Hq, D)
        st.out_ext = torch.empty_like(st.q_ext)
        lens = np.array([r.new for r in ext], np.int32)
        st.ext_tokens = int(lens.sum())
        st.max_ext = int(lens.max())
        st.qo_indptr = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(device)
        st.prefix_lens = torch.from_numpy(np.array([r.cached for r in ext], np.int32)).to(device)
        st.extend_lens = torch.from_numpy(lens).to(device)
        st.ext_order = torch.from_numpy(rs.extend_order([r.cached for r in ext], lens)).to(device)
        st.table_ext = st.table_dev[:n_ext]
    if dec:
        st.q_dec = qtab.index_select(0, torch.from_numpy(np.concatenate(q_dec_idx)).to(device)).view(-1, Hq, D)
        st.out_dec = torch.empty_like(st.q_dec)
        st.lse_dec = torch.empty((len(dec), Hq), dtype=torch.float32, device=device)
        sl_ = np.array([r.seq_len for r in dec], np.int32)
        st.dec_seq_lens = torch.from_numpy(sl_).to(device)
        st.max_seq = int(sl_.max())
        st.table_dec = st.table_dev[n_ext:]
        st.plan = st.plan_dev = None
        t0 = time.perf_counter()
        if build_plan:
            st.plan = rs.Plan(tree, nodes[n_ext:], np.array([r.cached for r in dec], np.int32), sl_, Hq, Hkv, D)
            st.plan_dev = rs.upload_plan(st.plan, device)
        st.plan_s = time.perf_counter() - t0
        st.ws = rs.DecodeWorkspace(st.plan, len(dec), st.max_seq, Hq, Hkv, D, device)
        st.ws_flat = rs.DecodeWorkspace(None, len(dec), st.max_seq, Hq, Hkv, D, device)
    torch.cuda.synchronize()
    st.host_s = time.perf_counter() - t_host
    return st


def run_store(st):
    import radix_tree_prefix_amd as rs
    rs.store_kv(st.k_pool, st.v_pool, st.k_new, st.v_new, st.new_slots)


def run_extend(st):
    import radix_tree_prefix_amd as rs
    if st.ext:
        rs.extend_attention(st.q_ext, st.k_pool, st.v_pool, st.table_ext, st.qo_indptr, st.prefix_lens,
                            st.extend_lens, st.max_ext, st.wl.sm_scale, out=st.out_ext, order=st.ext_order)


def run_decode(st, flat=False):
    import radix_tree_prefix_amd as rs
    if st.dec:
        if flat or st.plan is None:
            rs.decode_attention(st.q_dec, st.k_pool, st.v_pool, st.table_dec, st.dec_seq_lens, st.max_seq,
                                st.wl.sm_scale, st.ws_flat, out=st.out_dec, lse=st.lse_dec)
        else:
            rs.decode_attention(st.q_dec, st.k_pool, st.v_pool, st.table_dec, st.dec_seq_lens, st.max_seq,
                                st.wl.sm_scale, st.ws, plan=st.plan, plan_dev=st.plan_dev, out=st.out_dec,
                                lse=st.lse_dec)


def step(st):
    run_store(st)
    run_extend(st)
    run_decode(st)


# ---------------------------------------------------------------------------- work counts
def extend_flops(st):
    """Exact causal flops: 4*D per (query head, visible key) pair."""
    wl = st.wl
    tot = 0
    for r in st.ext:
        P, E = r.cached, r.new
        pairs = E * P + E * (E + 1) // 2
        tot += pairs
    return 4 * wl.D * wl.Hq * tot


def decode_unique_bytes(st):
    """Distinct KV positions the decode batch reads x bytes per position (K and V, all KV heads)."""
    esz = 2 if st.wl.dtype == "bf16" else 4
    slots = set()
    for r in st.dec:
        slots.update(st.table[r.row, :r.seq_len].tolist())
    return len(slots) * 2 * st.wl.Hkv * st.wl.D * esz


def decode_flat_bytes(st):
    esz = 2 if st.wl.dtype == "bf16" else 4
    return sum(r.seq_len for r in st.dec) * 2 * st.wl.Hkv * st.wl.D * esz


# ---------------------------------------------------------------------------- timing
def time_fn(fn, iters, warmup, flush=None):
    """Median and mean device time (ms) of fn over iters launches, events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    ts = []
    for _ in range(iters):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    return float(np.median(ts)), float(np.mean(ts))


def make_flush(device="cuda", nbytes=1 << 30):
    """Reads a 1 GiB buffer so that L2 and the 256 MB MALL hold none of the next op's inputs.

    A read, not a fill: a fill leaves the caches full of dirty lines whose write-back to HBM
    then runs during the timed op and competes with its reads (on the small decode workloads
    that added 7-35 us to ops of 30-110 us)."""
    import torch
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=device)
    acc = torch.empty((), dtype=torch.float32, device=device)      # same dtype: one reduction kernel, no cast copy

    def flush():
        torch.sum(buf, dim=0, out=acc)
    return flush


def cpu_baseline(st, budget_s=20.0):
    """The oracle (fp64 numpy, per-request materialised KV) on a bounded sample of the batch."""
    import oracle
    wl, vals = st.wl, st.vals
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    toks = 0
    sampled_ext = sampled_dec = 0
    order = []
    for i in range(max(len(st.ext), len(st.dec))):
        if i < len(st.dec):
            order.append(st.dec[i])
        if i < len(st.ext):
            order.append(st.ext[i])
    for r in order:
        if time.perf_counter() - t0 > budget_s:
            break
        k, v = vals.kv_rows(r.tokens, 0, r.seq_len)
        q = vals.q_rows(r.tokens, r.cached if r.kind == "extend" else r.seq_len - 1, r.seq_len)
        pos = np.arange(r.seq_len - len(q), r.seq_len)
        oracle.attend(q, k, v, pos, wl.sm_scale)
        toks += len(q)
        if r.kind == "extend":
            sampled_ext += 1
        else:
            sampled_dec += 1
    dt = time.perf_counter() - t0
    return {"value": toks / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{sampled_ext} extend + {sampled_dec} decode requests of the batch "
                      f"({toks} query tokens, {dt:.1f} s, KV regenerated per request, fp64 numpy)"}


EXTEND_KERNEL = "extend_bf16_kernel<128, false, 4, 2>"
VERIFY_KERNEL = "extend_bf16_kernel<128, true, 4, 1>"
# the decode kernel is instantiated per cache policy (<128, true> streams with the non-temporal
# one); a workload runs one of them, and the pattern names whichever it is
DECODE_KERNEL = "decode_bf16_kernel<128, *>"
MERGE_KERNEL = "decode_merge_kernel<128>"
F32_KERNEL = "extend_f32_kernel<64, 4>"


def code_hash(path):
    """SHA-256 of a C++ source with its // and /* */ comments and all whitespace removed, so that
    editing a comment does not count as changing the kernels."""
    import hashlib
    import re
    src = open(path).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return hashlib.sha256(re.sub(r"\s+", "", src).encode()).hexdigest()


def kernel_record(kernels, pattern):
    """(name, record) of the one kernel in `kernels` whose name matches `pattern` (an exact
    name, or an fnmatch pattern such as DECODE_KERNEL), else (pattern, None)."""
    import fnmatch
    if pattern in kernels:
        return pattern, kernels[pattern]
    hits = [n for n in kernels if fnmatch.fnmatchcase(n, pattern)]
    return (hits[0], kernels[hits[0]]) if len(hits) == 1 else (pattern, None)


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` (a name or pattern) on `workload` ("5", "1", "2", "3",
    "4", "verify") from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs (scaled by a plain
    copy's reading), or None when the kernel source has changed since they were taken or they
    do not cover the pair."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    name, k = kernel_record(rec["workloads"].get(str(workload), {}).get("kernels", {}), kernel)
    if code_hash(os.path.join(here, rec["source"])) != rec["code_sha256"] or k is None:
        return None
    return {"bytes": k["read_bytes"] + k["write_bytes"], "read": k["read_bytes"], "write": k["write_bytes"],
            "kernel": name}


# ---------------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the per-kernel runs of the other configs")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--flush", action="store_true",
                    help="read 1 GiB before every timed step (for workloads that fit in the caches)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    ap.add_argument("--host-tier", action="store_true",
                    help="only run the host tier's copy measurement (write-through and load back)")
    ap.add_argument("--verify", action="store_true",
                    help="only run the draft-tree verify measurement (cache-flushed)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the path has no cross-GPU step); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "no GPU visible"
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}), flush=True)
        return
    if args.host_tier:
        print(json.dumps(host_tier_extra()), flush=True)
        return
    if args.verify:
        print(json.dumps(verify_extra(make_flush())), flush=True)
        return
    print(f"[bench] setup config {args.config}", file=sys.stderr, flush=True)
    st = setup(args.config)
    print(f"[bench] setup done in {st.host_s:.1f}s (history {st.history_s:.2f}s, admit {st.admit_s:.3f}s)",
          file=sys.stderr, flush=True)

    # the timed region: exactly K steps
    for _ in range(args.warmup):
        step(st)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    flush = make_flush() if args.flush else None
    t0 = time.perf_counter()
    for e in ev:
        if flush is not None:
            flush()
        e[0].record()
        run_store(st)
        e[1].record()
        run_extend(st)
        e[2].record()
        run_decode(st)
        e[3].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ext_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    dec_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    store_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    if flush is not None:            # the flushes sit between the steps: count the kernels only
        ms_step = store_ms + ext_ms + dec_ms
    tokens = (st.ext_tokens if st.ext else 0) + len(st.dec)
    value = tokens / (ms_step / 1e3)

    flops = extend_flops(st) if st.ext else 0
    ub = decode_unique_bytes(st) if st.dec else 0
    ext_tf = flops / (ext_ms / 1e3) / 1e12 if st.ext else 0.0
    dec_gbs = ub / (dec_ms / 1e3) / 1e9 if st.dec else 0.0
    if st.ext:
        kern, peak = (EXTEND_KERNEL, BF16_PEAK_TFLOPS) if st.wl.dtype == "bf16" else (F32_KERNEL, FP32_PEAK_TFLOPS)
        roof = {"bound": "mfma", "kernel": kern, "achieved": round(ext_tf, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(ext_tf / peak, 4),
                "traffic": None, "algorithmic_per_launch": flops, "avg_launch_ms": round(ext_ms, 4)}
        tr = measured_traffic(roof["kernel"], args.config)
        if tr is not None:
            roof["traffic"] = tr["bytes"]
            roof["traffic_unit"] = "bytes/launch (HBM read+write, rocprofv3 FETCH_SIZE+WRITE_SIZE)"
            roof["traffic_read_write"] = [tr["read"], tr["write"]]
    else:
        roof = {"bound": "hbm", "kernel": DECODE_KERNEL, "achieved": round(dec_gbs, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                "traffic": None, "algorithmic_per_launch": ub, "avg_launch_ms": round(dec_ms, 4)}
        tr = measured_traffic(roof["kernel"], args.config)
        if tr is not None:
            roof["traffic"] = tr["bytes"]
            roof["kernel"] = tr["kernel"]
    out = {
        "metric": "decode+extend attention tokens/s and achieved HBM GB/s (% peak), 1 MI355X",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": st.wl.dtype, "data": "synthetic",
        "config": {"workload": st.wl.name, "batch": st.wl.B, "extend_tokens": st.ext_tokens if st.ext else 0,
                   "decode_requests": len(st.dec), "pool_slots": st.wl.pool_slots},
        "roofline": roof,
        "parts_ms": {"store_kv": round(store_ms, 4), "extend": round(ext_ms, 4), "decode": round(dec_ms, 4)},
        "host_ms": {"history_admission": round(st.history_s * 1e3, 2), "batch_admission": round(st.admit_s * 1e3, 3),
                    "decode_plan": round(getattr(st, "plan_s", 0.0) * 1e3, 3),
                    f"schedule_lpm_{min(st.sched_n, 128)}": round(st.sched_lpm_s * 1e3, 3),
                    f"schedule_dfs_weight_{st.sched_n}": round(st.sched_dfs_s * 1e3, 3)},
    }
    if st.dec:
        out["decode_hbm"] = {"achieved": round(dec_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "unique_kv_bytes": ub,
                             "flat_kv_bytes": decode_flat_bytes(st)}
        tr = measured_traffic(DECODE_KERNEL, args.config)
        trm = measured_traffic(MERGE_KERNEL, args.config)
        out["decode_hbm"]["traffic_decode_kernel"] = tr["bytes"] if tr is not None else None
        out["decode_hbm"]["traffic_merge_kernel"] = trm["bytes"] if trm is not None else None
    if not args.no_extra:
        out["other_configs"] = extra_configs()
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(st, args.cpu_budget)
    print(json.dumps(out), flush=True)


def extra_configs():
    """Per-kernel numbers of the smaller workloads (cache-flushed medians)."""
    import torch
    res = {}
    flush = make_flush()
    for cfg in (2, 4, 3, 1):
        print(f"[bench] extra config {cfg}", file=sys.stderr, flush=True)
        st = setup(cfg)
        d = {"workload": st.wl.name}
        if st.dec:
            med, _ = time_fn(lambda: run_decode(st), 30, 5, flush)
            medf, _ = time_fn(lambda: run_decode(st, flat=True), 30, 5, flush)
            ub = decode_unique_bytes(st)
            d.update({"decode_plan_us": round(med * 1e3, 2), "decode_flat_us": round(medf * 1e3, 2),
                      "unique_kv_bytes": ub, "hbm_gbs_unique": round(ub / (med / 1e3) / 1e9, 1),
                      "hbm_frac": round(ub / (med / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                      "tokens_per_s": round(len(st.dec) / (med / 1e3), 1)})
            for name, kern in (("traffic_decode_kernel", DECODE_KERNEL), ("traffic_merge_kernel", MERGE_KERNEL)):
                tr = measured_traffic(kern, cfg)
                d[name] = tr["bytes"] if tr is not None else None
        if st.ext:
            med, _ = time_fn(lambda: run_extend(st), 20, 3, flush)
            f = extend_flops(st)
            tf = f / (med / 1e3) / 1e12
            d.update({"extend_us": round(med * 1e3, 2), "flops": f, "tflops": round(tf, 2),
                      "tokens_per_s": round(st.ext_tokens / (med / 1e3), 1)})
            if st.wl.dtype == "bf16":
                d["mfma_frac"] = round(tf / BF16_PEAK_TFLOPS, 4)
                tr = measured_traffic(EXTEND_KERNEL, cfg)
                d["traffic_extend_kernel"] = tr["bytes"] if tr is not None else None
            else:                    # fp32 on 32x32x2 fp32 MFMAs: against the fp32 matrix peak
                d["fp32_frac"] = round(tf / FP32_PEAK_TFLOPS, 4)
                tr = measured_traffic(F32_KERNEL, cfg)
                d["traffic_extend_kernel"] = tr["bytes"] if tr is not None else None
        res[str(cfg)] = d
        del st
        torch.cuda.empty_cache()
    print("[bench] extra: draft-tree verify", file=sys.stderr, flush=True)
    res["verify"] = verify_extra(flush)
    torch.cuda.empty_cache()
    print("[bench] extra: host tier copies", file=sys.stderr, flush=True)
    res["host_tier"] = host_tier_extra()
    torch.cuda.empty_cache()
    return res


def host_tier_extra(tokens=65536, Hkv=8, D=128, seed=1013):
    """Two-tier cache: a 64k-token prefix written through to pinned host pools and loaded
    back, with the pairs the tree hands out (rs_copy_kv over the bus), beside a contiguous
    copy of the same bytes as the bus's own rate; and the tree calls' host time."""
    import time
    import torch
    import radix_tree_prefix_amd as rs
    S = H = 2 * tokens
    g = torch.Generator(device="cuda").manual_seed(seed)
    dk = torch.randn((S, Hkv, D), device="cuda", dtype=torch.bfloat16, generator=g)
    dv = torch.randn((S, Hkv, D), device="cuda", dtype=torch.bfloat16, generator=g)
    hk = rs.host_pool((H, Hkv, D), torch.bfloat16)
    hv = rs.host_pool((H, Hkv, D), torch.bfloat16)
    tree = rs.Tree(S)
    tree.enable_host(H)
    rng = np.random.default_rng(seed)
    toks = rng.integers(0, 32000, tokens).astype(np.int32)
    for i in range(0, tokens, 4096):              # the prefix arrives in 16 chunks: 16 nodes
        row, node, _m = tree.admit(toks[:i + 4096], i + 4096, 0)
        tree.dec_lock_ref(node)
    t0 = time.perf_counter()
    d, h, tk = tree.write_through(node)
    t_wt = time.perf_counter() - t0
    d_dev, h_dev = torch.from_numpy(d).cuda(), torch.from_numpy(h).cuda()
    d2h = lambda: rs.copy_kv(hk, hv, dk, dv, h_dev, d_dev)
    med_d2h, _ = time_fn(d2h, 10, 2)
    tree.commit(tk, True)
    tree.evict(S)
    t0 = time.perf_counter()
    src, dst, tk = tree.load_back(node)
    t_lb = time.perf_counter() - t0
    s_dev, t_dev = torch.from_numpy(src).cuda(), torch.from_numpy(dst).cuda()
    h2d = lambda: rs.copy_kv(dk, dv, hk, hv, t_dev, s_dev)
    med_h2d, _ = time_fn(h2d, 10, 2)
    tree.commit(tk, True)
    nbytes = 2 * len(d) * Hkv * D * 2
    flat_dev = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    flat_host = rs.host_pool((nbytes // 2,), torch.bfloat16)
    med_cd2h, _ = time_fn(lambda: flat_host.copy_(flat_dev, non_blocking=True), 10, 2)
    med_ch2d, _ = time_fn(lambda: flat_dev.copy_(flat_host, non_blocking=True), 10, 2)
    gbs = lambda ms: round(nbytes / (ms / 1e3) / 1e9, 1)
    return {"workload": f"host tier: {tokens:,}-token prefix in 16 nodes, K+V bf16 GQA {Hkv}x{D} "
                        f"({nbytes / 2**20:.0f} MiB), pinned host pools",
            "write_through_us": round(med_d2h * 1e3, 1), "write_through_gbs": gbs(med_d2h),
            "load_back_us": round(med_h2d * 1e3, 1), "load_back_gbs": gbs(med_h2d),
            "contiguous_d2h_gbs": gbs(med_cd2h), "contiguous_h2d_gbs": gbs(med_ch2d),
            "tree_write_through_ms": round(t_wt * 1e3, 3), "tree_load_back_ms": round(t_lb * 1e3, 3)}


def verify_extra(flush, B=256, prefix=32768, n=16, Hq=64, Hkv=8, D=128, seed=1009):
    """Draft-tree verify at the size the pages price the full mask at (256 requests, 32k
    context, 16 verify tokens): seeded random draft trees and bf16 K/V/Q, each request's
    context in its own run of slots, inputs resident.  HBM-bound on the unique KV bytes."""
    import torch
    import radix_tree_prefix_amd as rs
    g = torch.Generator(device="cuda").manual_seed(seed)
    rng = np.random.default_rng(seed)
    S = B * (prefix + n)
    kp = torch.randn((S, Hkv, D), device="cuda", dtype=torch.bfloat16, generator=g)
    vp = torch.randn((S, Hkv, D), device="cuda", dtype=torch.bfloat16, generator=g)
    q = torch.randn((B * n, Hq, D), device="cuda", dtype=torch.bfloat16, generator=g)
    table = torch.arange(S, dtype=torch.int32, device="cuda").view(B, prefix + n)
    parents = np.stack([np.array([-1] + [int(rng.integers(0, i)) for i in range(1, n)], np.int32)
                        for _ in range(B)])
    mask, pos, _nt, _ns = rs.draft_tree_build(parents, np.full(B, prefix, np.int32))
    mask_dev = torch.from_numpy(mask.view(np.int64)).cuda()
    prefix_dev = torch.full((B,), prefix, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    run = lambda: rs.tree_verify_attention(q, kp, vp, table, prefix_dev, mask_dev, 1 / np.sqrt(D), out=out)
    med, _ = time_fn(run, 20, 3, flush)
    ub = S * 2 * Hkv * D * 2
    depth1 = (pos - prefix + 1).astype(np.int64)          # keys seen among the verify tokens
    flops = int(((prefix + depth1).sum()) * Hq * 4 * D)
    tr = measured_traffic(VERIFY_KERNEL, "verify")
    return {"workload": f"draft-tree verify ({B} x {prefix:,} cached + {n} verify tokens, random trees, bf16, "
                        f"GQA {Hq}/{Hkv}, d{D})",
            "traffic_verify_kernel": tr["bytes"] if tr is not None else None,
            "verify_us": round(med * 1e3, 2), "unique_kv_bytes": ub,
            "hbm_gbs_unique": round(ub / (med / 1e3) / 1e9, 1),
            "hbm_frac": round(ub / (med / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(flops / (med / 1e3) / 1e12, 2),
            "tokens_per_s": round(B * n / (med / 1e3), 1)}


if __name__ == "__main__":
    main()

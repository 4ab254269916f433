"""GPU parity: the HIP path (through the C ABI) against the oracle, element by element.

bf16 outputs must be within max-abs 2e-2 of the float64 oracle, fp32 within 1e-4.
Index tables are compared bit-exact.  Each test prints what it runs before any
GPU work so a failure names its case.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
from conftest import bf16_request_errors, BF16_MAX_ABS, BF16_REL_RMS, LSE_MAX_ABS

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}


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


def _to_dev(torch, a, dt):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda", dtype=dt)


def _oracle_request(st, r, rows=None):
    """Oracle output for one request of a bench State: KV regenerated from its own tokens."""
    k, v = st.vals.kv_rows(r.tokens, 0, r.seq_len)
    lo = r.cached if r.kind == "extend" else r.seq_len - 1
    pos = np.arange(lo, r.seq_len)
    q = st.vals.q_rows(r.tokens, lo, r.seq_len)
    if rows is not None:
        q, pos = q[rows], pos[rows]
    return oracle.attend(q, k, v, pos, st.wl.sm_scale)


def _oracle_table(wl):
    t = oracle.RadixTree(wl.pool_slots)
    oracle.admit_history(t, wl.history)
    return oracle.admit_batch(t, wl)["table"]


def _check_table(st):
    """Bit-exact against the oracle's table; the bench pads rows (to 64 bytes) with -1."""
    ref = _oracle_table(st.wl)
    assert st.table.shape[1] >= ref.shape[1] and st.table.shape[1] % 16 == 0
    np.testing.assert_array_equal(st.table[:, :ref.shape[1]], ref)
    assert (st.table[:, ref.shape[1]:] == -1).all()


# ------------------------------------------------------------------ small kernels
def test_store_kv_scatter(torch_rs):
    torch, rs = torch_rs
    _say("store_kv bf16/f32 scatter")
    rng = np.random.default_rng(0)
    for dt in (torch.bfloat16, torch.float32):
        S, Hkv, D, n = 1000, 8, 128, 333
        kp = torch.zeros((S, Hkv, D), dtype=dt, device="cuda")
        vp = torch.zeros_like(kp)
        slots = rng.permutation(S)[:n].astype(np.int32)
        kn = torch.randn((n, Hkv, D), device="cuda").to(dt)
        vn = torch.randn((n, Hkv, D), device="cuda").to(dt)
        rs.store_kv(kp, vp, kn, vn, _to_dev(torch, slots, torch.int32))
        torch.cuda.synchronize()
        ref_k = torch.zeros((S, Hkv, D), dtype=dt)
        ref_k[torch.from_numpy(slots).long()] = kn.cpu()
        assert torch.equal(kp.cpu(), ref_k)
        ref_v = torch.zeros((S, Hkv, D), dtype=dt)
        ref_v[torch.from_numpy(slots).long()] = vn.cpu()
        assert torch.equal(vp.cpu(), ref_v)


def test_merge_states_closed_form(torch_rs):
    torch, rs = torch_rs
    _say("merge_states vs oracle merge")
    rng = np.random.default_rng(1)
    rows, D = 300, 128
    oa, ob = rng.standard_normal((rows, D)), rng.standard_normal((rows, D))
    la, lb = rng.standard_normal(rows) * 5, rng.standard_normal(rows) * 5
    lb[:10] = -np.inf                       # an empty side contributes nothing
    for dt, name in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        oa_, ob_ = (_bf16(oa), _bf16(ob)) if name == "bf16" else (oa.astype(np.float32), ob.astype(np.float32))
        o = rs.merge_states(_to_dev(torch, oa_, dt), _to_dev(torch, la.astype(np.float32), torch.float32),
                            _to_dev(torch, ob_, dt), _to_dev(torch, lb.astype(np.float32), torch.float32),
                            lse=(lse := torch.empty(rows, dtype=torch.float32, device="cuda")))
        ro, rl = oracle.merge_states(oa_, la.astype(np.float32), ob_, lb.astype(np.float32))
        err = np.abs(o.float().cpu().numpy() - ro).max()
        assert err <= (TOL[name] if name == "bf16" else 1e-5), (name, err)
        assert np.abs(lse.cpu().numpy() - rl).max() < 1e-4


# ------------------------------------------------------------------ synthetic random pools
def _random_case(torch, Hq, Hkv, D, lens, dtname, seed, scale=1.0):
    """Random pool, a random slot table, lens = [(prefix, extend)]."""
    rng = np.random.default_rng(seed)
    L = [p + e for p, e in lens]
    S = sum(L) + 17
    kp = rng.standard_normal((S, Hkv, D)).astype(np.float32) * scale
    vp = rng.standard_normal((S, Hkv, D)).astype(np.float32) * scale
    if dtname == "bf16":
        kp, vp = _bf16(kp), _bf16(vp)
    perm = rng.permutation(S).astype(np.int32)
    ld = max(max(L), 1)
    table = np.full((len(lens), ld), -1, np.int32)
    off = 0
    for b, n in enumerate(L):
        table[b, :n] = perm[off:off + n]
        off += n
    return kp, vp, table


def _extend_case(torch, rs, Hq, Hkv, D, lens, dtname, seed):
    dt = torch.bfloat16 if dtname == "bf16" else torch.float32
    kp, vp, table = _random_case(torch, Hq, Hkv, D, lens, dtname, seed)
    rng = np.random.default_rng(seed + 100)
    ext = np.array([e for _, e in lens], np.int32)
    q = rng.standard_normal((int(ext.sum()), Hq, D)).astype(np.float32)
    if dtname == "bf16":
        q = _bf16(q)
    qo = np.concatenate([[0], np.cumsum(ext)]).astype(np.int32)
    sm = 1 / np.sqrt(D)
    out = rs.extend_attention(_to_dev(torch, q, dt), _to_dev(torch, kp, dt), _to_dev(torch, vp, dt),
                              _to_dev(torch, table, torch.int32), _to_dev(torch, qo, torch.int32),
                              _to_dev(torch, np.array([p for p, _ in lens], np.int32), torch.int32),
                              _to_dev(torch, ext, torch.int32), int(max(ext.max(), 1)), sm)
    got = out.float().cpu().numpy()
    worst = 0.0
    for b, (p, e) in enumerate(lens):
        if e == 0:
            continue
        row = table[b, :p + e]
        o, _ = oracle.attend(q[qo[b]:qo[b + 1]], kp[row], vp[row], p + np.arange(e), sm)
        worst = max(worst, float(np.abs(got[qo[b]:qo[b + 1]] - o).max()))
    return worst


@pytest.mark.parametrize("Hq,Hkv,D", [(16, 4, 128), (8, 8, 128), (64, 8, 128), (8, 2, 64), (24, 8, 128),
                                      (64, 4, 128), (128, 1, 64)])
def test_extend_bf16_ragged(torch_rs, Hq, Hkv, D):
    torch, rs = torch_rs
    lens = [(0, 1), (0, 37), (1, 5), (63, 64), (64, 129), (200, 0), (517, 33), (1000, 300)]
    _say(f"extend bf16 Hq={Hq} Hkv={Hkv} D={D} lens={lens}")
    err = _extend_case(torch, rs, Hq, Hkv, D, lens, "bf16", seed=Hq + D)
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 8, 64), (8, 2, 128), (24, 8, 64), (64, 4, 128), (128, 1, 64)])
def test_extend_f32_ragged(torch_rs, Hq, Hkv, D):
    torch, rs = torch_rs
    lens = [(0, 1), (0, 70), (65, 3), (130, 64), (333, 0)]
    _say(f"extend f32 Hq={Hq} Hkv={Hkv} D={D}")
    err = _extend_case(torch, rs, Hq, Hkv, D, lens, "f32", seed=7)
    assert err <= TOL["f32"], err


def _planted_case(torch, rs, sm, lens, seed, dtname="bf16"):
    """Extend where one late key of each request is a scaled copy of its first query row,
    so that row's late score stands far above every score of the first key tile."""
    Hq, Hkv, D = 8, 2, 128
    rng = np.random.default_rng(seed)
    L = [p + e for p, e in lens]
    S = sum(L) + 5
    kp = _bf16(rng.standard_normal((S, Hkv, D)).astype(np.float32) * 0.1)
    vp = _bf16(rng.standard_normal((S, Hkv, D)).astype(np.float32))
    ext = np.array([e for _, e in lens], np.int32)
    q = _bf16(rng.standard_normal((int(ext.sum()), Hq, D)).astype(np.float32))
    qo = np.concatenate([[0], np.cumsum(ext)]).astype(np.int32)
    perm = rng.permutation(S).astype(np.int32)
    table = np.full((len(lens), max(L)), -1, np.int32)
    off = 0
    for b, n in enumerate(L):
        table[b, :n] = perm[off:off + n]
        off += n
        p = lens[b][0]
        kp[table[b, p - 7]] = q[qo[b], 0:Hq:Hq // Hkv]     # key p-7 of KV head h = query 0's head h*G
    return _extend_vs_oracle(torch, rs, q, kp, vp, table, lens, sm, dtname)


def _extend_vs_oracle(torch, rs, q, kp, vp, table, lens, sm, dtname):
    """Extend over the given pools and index table, every row against oracle.attend."""
    ext = np.array([e for _, e in lens], np.int32)
    qo = np.concatenate([[0], np.cumsum(ext)]).astype(np.int32)
    dt = torch.bfloat16 if dtname == "bf16" else torch.float32
    out = rs.extend_attention(_to_dev(torch, q, dt), _to_dev(torch, kp, dt),
                              _to_dev(torch, vp, dt), _to_dev(torch, table, torch.int32),
                              _to_dev(torch, qo, torch.int32),
                              _to_dev(torch, np.array([p for p, _ in lens], np.int32), torch.int32),
                              _to_dev(torch, ext, torch.int32), int(ext.max()), sm)
    got = out.float().cpu().numpy()
    worst = 0.0
    for b, (p, e) in enumerate(lens):
        row = table[b, :p + e]
        o, _ = oracle.attend(q[qo[b]:qo[b + 1]], kp[row], vp[row], p + np.arange(e), sm)
        worst = max(worst, float(np.abs(got[qo[b]:qo[b + 1]] - o).max()))
    return worst


@pytest.mark.parametrize("sm", [0.35, 0.6, 1.0])
def test_extend_late_dominant_key(torch_rs, sm):
    """A late score far above every other (about 0.35, 0.6 or 1.0 x 185 log2-units, and
    far above the first tile's maximum): weights up to ~2^110 stay finite and exact
    relative to each other; at sm=1 they overflow fp32, and the rows are recomputed with
    their true maximum."""
    torch, rs = torch_rs
    lens = [(100, 50), (700, 37), (3000, 64)]
    _say(f"extend planted dominant key sm_scale={sm} lens={lens}")
    err = _planted_case(torch, rs, sm, lens, seed=11)
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("sm", [0.35, 1.0])
def test_extend_f32_late_dominant_key(torch_rs, sm):
    """The fp32 path on the same planted batch: the softmax reference of the affected rows
    has to move on a late tile (scores ~65 or ~185 log2-units above the first tile's)."""
    torch, rs = torch_rs
    lens = [(100, 50), (700, 37), (3000, 64)]
    _say(f"extend f32 planted dominant key sm_scale={sm} lens={lens}")
    err = _planted_case(torch, rs, sm, lens, seed=11, dtname="f32")
    assert err <= TOL["f32"], err


@pytest.mark.parametrize("dtname", ["bf16", "f32"])
def test_extend_all_scores_far_below_zero(torch_rs, dtname):
    """Every score of every row sits about 260 log2-units below zero (queries near -16, keys
    near +1 in every dimension), so weights taken against no reference all underflow to 0:
    the rows must come out of a pass with their true maximum as the reference."""
    torch, rs = torch_rs
    Hq, Hkv, D = 8, 2, 128
    lens = [(0, 70), (100, 50), (700, 37), (3000, 64)]
    _say(f"extend {dtname} scores far below zero lens={lens}")
    rng = np.random.default_rng(19)
    L = [p + e for p, e in lens]
    S = sum(L) + 5
    kp = _bf16((1.0 + 0.5 * rng.standard_normal((S, Hkv, D))).astype(np.float32))
    vp = _bf16(rng.standard_normal((S, Hkv, D)).astype(np.float32))
    q = _bf16((-16.0 + rng.standard_normal((sum(e for _, e in lens), Hq, D))).astype(np.float32))
    perm = rng.permutation(S).astype(np.int32)
    table = np.full((len(lens), max(L)), -1, np.int32)
    off = 0
    for b, n in enumerate(L):
        table[b, :n] = perm[off:off + n]
        off += n
    err = _extend_vs_oracle(torch, rs, q, kp, vp, table, lens, 1 / np.sqrt(D), dtname)
    assert err <= TOL[dtname], err


def test_extend_prefix_zero_is_textbook_causal(torch_rs):
    """No cached prefix: plain causal attention, against torch SDPA in fp64 on the CPU."""
    torch, rs = torch_rs
    import torch.nn.functional as F
    _say("extend prefix 0 vs SDPA")
    Hq, Hkv, D, n = 32, 8, 128, 300
    rng = np.random.default_rng(3)
    q, k, v = (_bf16(rng.standard_normal(s).astype(np.float32)) for s in ((n, Hq, D), (n, Hkv, D), (n, Hkv, D)))
    table = np.arange(n, dtype=np.int32)[None]
    out = rs.extend_attention(_to_dev(torch, q, torch.bfloat16), _to_dev(torch, k, torch.bfloat16),
                              _to_dev(torch, v, torch.bfloat16), _to_dev(torch, table, torch.int32),
                              _to_dev(torch, np.array([0, n], np.int32), torch.int32),
                              _to_dev(torch, np.array([0], np.int32), torch.int32),
                              _to_dev(torch, np.array([n], np.int32), torch.int32), n, 1 / np.sqrt(D))
    ref = F.scaled_dot_product_attention(torch.from_numpy(q).double().permute(1, 0, 2)[None],
                                         torch.from_numpy(k).double().permute(1, 0, 2)[None],
                                         torch.from_numpy(v).double().permute(1, 0, 2)[None],
                                         is_causal=True, enable_gqa=True)[0].permute(1, 0, 2).numpy()
    assert np.abs(out.float().cpu().numpy() - ref).max() <= TOL["bf16"]


def _decode_case(torch, rs, Hq, Hkv, D, Ls, dtname, seed):
    dt = torch.bfloat16 if dtname == "bf16" else torch.float32
    kp, vp, table = _random_case(torch, Hq, Hkv, D, [(L - 1, 1) for L in Ls], dtname, seed)
    rng = np.random.default_rng(seed + 1)
    q = rng.standard_normal((len(Ls), Hq, D)).astype(np.float32)
    if dtname == "bf16":
        q = _bf16(q)
    sm = 1 / np.sqrt(D)
    ws = rs.DecodeWorkspace(None, len(Ls), max(Ls), Hq, Hkv, D)
    lse = torch.empty((len(Ls), Hq), dtype=torch.float32, device="cuda")
    out = rs.decode_attention(_to_dev(torch, q, dt), _to_dev(torch, kp, dt), _to_dev(torch, vp, dt),
                              _to_dev(torch, table, torch.int32), _to_dev(torch, np.array(Ls, np.int32), torch.int32),
                              max(Ls), sm, ws, lse=lse)
    got, gl = out.float().cpu().numpy(), lse.cpu().numpy()
    worst = wl = 0.0
    for b, L in enumerate(Ls):
        row = table[b, :L]
        o, l = oracle.attend(q[b:b + 1], kp[row], vp[row], [L - 1], sm)
        worst = max(worst, float(np.abs(got[b] - o[0]).max()))
        wl = max(wl, float(np.abs(gl[b] - l[0]).max()))
    return worst, wl


@pytest.mark.parametrize("Hq,Hkv,D", [(32, 8, 128), (64, 8, 128), (8, 8, 128), (8, 2, 64)])
def test_decode_flat_bf16(torch_rs, Hq, Hkv, D):
    torch, rs = torch_rs
    Ls = [1, 2, 63, 64, 255, 256, 257, 1000, 3201]
    _say(f"decode flat bf16 Hq={Hq} Hkv={Hkv} D={D} Ls={Ls}")
    err, lerr = _decode_case(torch, rs, Hq, Hkv, D, Ls, "bf16", seed=Hq * 3 + D)
    assert err <= TOL["bf16"], err
    assert lerr <= 1e-2, lerr


def test_decode_f32(torch_rs):
    torch, rs = torch_rs
    Ls = [1, 5, 64, 65, 700]
    _say("decode f32")
    err, lerr = _decode_case(torch, rs, 16, 4, 128, Ls, "f32", seed=11)
    assert err <= TOL["f32"], err
    assert lerr <= 1e-4


def test_decode_single_key_returns_value(torch_rs):
    torch, rs = torch_rs
    _say("decode L=1 returns v0")
    Hq, Hkv, D = 32, 8, 128
    rng = np.random.default_rng(5)
    v = _bf16(rng.standard_normal((1, Hkv, D)).astype(np.float32))
    k = _bf16(rng.standard_normal((1, Hkv, D)).astype(np.float32))
    q = _bf16(rng.standard_normal((1, Hq, D)).astype(np.float32))
    ws = rs.DecodeWorkspace(None, 1, 1, Hq, Hkv, D)
    out = rs.decode_attention(_to_dev(torch, q, torch.bfloat16), _to_dev(torch, k, torch.bfloat16),
                              _to_dev(torch, v, torch.bfloat16), _to_dev(torch, np.zeros((1, 1), np.int32), torch.int32),
                              _to_dev(torch, np.array([1], np.int32), torch.int32), 1, 1 / np.sqrt(D), ws)
    got = out.float().cpu().numpy()[0]
    for h in range(Hq):
        np.testing.assert_array_equal(got[h], v[0, h // (Hq // Hkv)])


@pytest.mark.parametrize("dtname", ["bf16", "f32"])
def test_decode_flat_cuts_requests_longer_than_max_seq_len(torch_rs, dtname):
    """Without a plan the device cannot check seq_lens against max_seq_len: a request that
    claims more keys than max_seq_len is cut to its first max_seq_len keys, so every read
    stays inside its table row and its partials inside their workspace range.  (The table
    is a view into a larger buffer, so even a read past a row would stay in memory.)"""
    torch, rs = torch_rs
    Hq, Hkv, D, M = 16, 4, 128, 512
    Ls = [300, 700, 512, 1000]
    _say(f"decode flat {dtname}, seq_lens {Ls} cut to max_seq_len {M}")
    dt = torch.bfloat16 if dtname == "bf16" else torch.float32
    rng = np.random.default_rng(21)
    S = 4 * M + 8
    kp = rng.standard_normal((S, Hkv, D)).astype(np.float32)
    vp = rng.standard_normal((S, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((len(Ls), Hq, D)).astype(np.float32)
    if dtname == "bf16":
        kp, vp, q = _bf16(kp), _bf16(vp), _bf16(q)
    big = np.full((len(Ls) + 1, M), -1, np.int32)
    big[:len(Ls)] = rng.permutation(S)[:len(Ls) * M].reshape(len(Ls), M)
    table = _to_dev(torch, big, torch.int32)[:len(Ls)]
    ws = rs.DecodeWorkspace(None, len(Ls), M, Hq, Hkv, D)
    lse = torch.empty((len(Ls), Hq), dtype=torch.float32, device="cuda")
    out = rs.decode_attention(_to_dev(torch, q, dt), _to_dev(torch, kp, dt), _to_dev(torch, vp, dt), table,
                              _to_dev(torch, np.array(Ls, np.int32), torch.int32), M, 1 / np.sqrt(D), ws, lse=lse)
    got, gl = out.float().cpu().numpy(), lse.cpu().numpy()
    for b, L in enumerate(Ls):
        n = min(L, M)
        row = big[b, :n]
        o, l = oracle.attend(q[b:b + 1], kp[row], vp[row], [n - 1], 1 / np.sqrt(D))
        assert np.abs(got[b] - o[0]).max() <= TOL[dtname], (b, L)
        assert np.abs(gl[b] - l[0]).max() <= (1e-2 if dtname == "bf16" else 1e-4), (b, L)


# ------------------------------------------------------------------ the workloads
def _bench():
    import bench
    return bench


def test_config1_two_document_agent_extend_f32(torch_rs):
    torch, rs = torch_rs
    _say("config 1 (fp32 extend, two-document agent)")
    b = _bench()
    st = b.setup(1)
    _check_table(st)
    b.step(st)
    torch.cuda.synchronize()
    got = st.out_ext.cpu().numpy()
    qo = st.qo_indptr.cpu().numpy()
    worst = 0.0
    for i, r in enumerate(st.ext):
        o, _ = _oracle_request(st, r)
        worst = max(worst, float(np.abs(got[qo[i]:qo[i + 1]] - o).max()))
    assert worst <= TOL["f32"], worst


@pytest.mark.parametrize("cfg", [2, 4])
def test_decode_workloads_plan_and_flat(torch_rs, cfg):
    torch, rs = torch_rs
    _say(f"config {cfg} decode (plan and flat)")
    b = _bench()
    st = b.setup(cfg)
    _check_table(st)
    ref = [_oracle_request(st, r) for r in st.dec]
    for flat in (False, True):
        st.out_dec.zero_()
        b.run_store(st)
        b.run_decode(st, flat=flat)
        torch.cuda.synchronize()
        got, gl = st.out_dec.float().cpu().numpy(), st.lse_dec.cpu().numpy()
        errs = [bf16_request_errors(got[i], o[0]) for i, (o, _) in enumerate(ref)]
        lerr = max(float(np.abs(gl[i] - l[0]).max()) for i, (_, l) in enumerate(ref))
        assert max(e[0] for e in errs) <= BF16_MAX_ABS, (flat, errs)
        assert max(e[1] for e in errs) <= BF16_REL_RMS, (flat, errs)
        assert lerr <= LSE_MAX_ABS, (flat, lerr)


def test_decode_plan_repeat_bit_identical(torch_rs):
    """Repeated plan-driven launches (decode and merge kernels, one workspace) agree bit for bit."""
    torch, rs = torch_rs
    _say("config 4 decode plan x5 bit identity")
    b = _bench()
    st = b.setup(4)
    b.run_store(st)
    outs = []
    for _ in range(5):
        b.run_decode(st)
        outs.append((st.out_dec.clone(), st.lse_dec.clone()))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def test_decode_consecutive_launches_merge_their_own_partials(torch_rs):
    """Partials live in the workspace across launches: each launch, with other queries
    (scaled by powers of two, exact in bf16), must merge only its own partials, in plan mode
    and in flat mode."""
    torch, rs = torch_rs
    _say("config 4 decode: three launches with different queries, plan and flat")
    b = _bench()
    st = b.setup(4)
    b.run_store(st)
    q0 = st.q_dec.clone()
    kv = [st.vals.kv_rows(r.tokens, 0, r.seq_len) for r in st.dec]
    qs = [st.vals.q_rows(r.tokens, r.seq_len - 1, r.seq_len) for r in st.dec]
    for scale in (1.0, -0.5, 2.0, 1.0):
        st.q_dec.copy_(q0 * scale)
        for flat in (False, True):
            b.run_decode(st, flat=flat)
            torch.cuda.synchronize()
            got, gl = st.out_dec.float().cpu().numpy(), st.lse_dec.cpu().numpy()
            for i, r in enumerate(st.dec):
                o, l = oracle.attend(qs[i] * scale, kv[i][0], kv[i][1], [r.seq_len - 1], st.wl.sm_scale)
                mx, rel = bf16_request_errors(got[i], o[0])
                assert mx <= BF16_MAX_ABS and rel <= BF16_REL_RMS, (scale, flat, i, mx, rel)
                assert np.abs(gl[i] - l[0]).max() <= LSE_MAX_ABS, (scale, flat, i)


def test_config3_multistep_agent_extend(torch_rs):
    torch, rs = torch_rs
    _say("config 3 extend bf16 (64 users)")
    b = _bench()
    st = b.setup(3)
    _check_table(st)
    b.step(st)
    torch.cuda.synchronize()
    got = st.out_ext.float().cpu().numpy()
    qo = st.qo_indptr.cpu().numpy()
    errs = []
    for i, r in enumerate(st.ext):
        o, _ = _oracle_request(st, r)
        errs.append(bf16_request_errors(got[qo[i]:qo[i + 1]], o))
    assert max(e[0] for e in errs) <= BF16_MAX_ABS, errs
    assert max(e[1] for e in errs) <= BF16_REL_RMS, errs


@pytest.fixture(scope="module")
def mixed_batch(torch_rs):
    """The full-size mixed batch in the bench's launch configuration, stepped once."""
    torch, rs = torch_rs
    b = _bench()
    _say("config 5 full size (setup)")
    st = b.setup(5)
    _say("config 5: step")
    b.step(st)
    torch.cuda.synchronize()
    st.got_ext = st.out_ext.float().cpu().numpy()
    st.got_dec = st.out_dec.float().cpu().numpy()
    st.got_lse = st.lse_dec.cpu().numpy()
    return st


def test_config5_tables_bit_exact(mixed_batch):
    _say("config 5: tables vs oracle")
    _check_table(mixed_batch)


def test_config5_every_decode_request(mixed_batch):
    """All 128 decode requests (contexts 1k-32k) against the oracle: outputs within the
    per-request bf16 bounds (max-abs and relative RMS) and lse within 1e-2."""
    st = mixed_batch
    _say(f"config 5: all {len(st.dec)} decode requests vs oracle")
    bad = []
    for i, r in enumerate(st.dec):
        o, l = _oracle_request(st, r)
        mx, rel = bf16_request_errors(st.got_dec[i], o[0])
        lerr = float(np.abs(st.got_lse[i] - l[0]).max())
        if mx > BF16_MAX_ABS or rel > BF16_REL_RMS or lerr > LSE_MAX_ABS:
            bad.append((i, r.seq_len, mx, rel, lerr))
    assert not bad, bad


@pytest.mark.parametrize("half", [0, 1])
def test_config5_every_extend_request(mixed_batch, half):
    """Every extend request (64 per half) against the oracle on its first row and the last
    row of every 16-token block: every q-tile of the kernel, at every head grouping it
    supports, has at least one of its rows checked (the last row of a block sees the most
    keys of its block)."""
    st = mixed_batch
    n = len(st.ext)
    idx = range(half * n // 2, (half + 1) * n // 2)
    _say(f"config 5: extend requests {idx.start}..{idx.stop - 1} vs oracle")
    qo = st.qo_indptr.cpu().numpy()
    bad = []
    for i in idx:
        r = st.ext[i]
        rows = np.unique(np.concatenate([[0], np.arange(15, r.new, 16), [r.new - 1]]))
        o, _ = _oracle_request(st, r, rows)
        mx, rel = bf16_request_errors(st.got_ext[qo[i] + rows], o)
        if mx > BF16_MAX_ABS or rel > BF16_REL_RMS:
            bad.append((i, r.seq_len, mx, rel))
    assert not bad, bad


@pytest.mark.parametrize("cfg", [3, 1])
def test_extend_order_changes_no_result(torch_rs, cfg):
    """The longest-first start order only reorders workgroups: outputs are bit-identical
    (bf16 engine on the multi-step agent, fp32 kernel on the two-document agent)."""
    torch, rs = torch_rs
    _say(f"config {cfg} extend with and without the work order")
    b = _bench()
    st = b.setup(cfg)
    b.run_store(st)
    b.run_extend(st)
    with_order = st.out_ext.clone()
    rs.extend_attention(st.q_ext, st.k_pool, st.v_pool, st.table_ext, st.qo_indptr, st.prefix_lens,
                        st.extend_lens, st.max_ext, st.wl.sm_scale, out=st.out_ext)
    torch.cuda.synchronize()
    assert torch.equal(with_order, st.out_ext)
    assert sorted(st.ext_order.cpu().tolist()) == list(range(len(st.ext)))

"""Decode plans (host side, no GPU): every request's context is covered exactly once,
shared segments really share slots, and the unique-KV accounting matches the oracle tree."""
import numpy as np
import pytest

import oracle
import synth
import radix_tree_prefix_amd as rs


def _admit(wl):
    t = rs.Tree(wl.pool_slots)
    for s in wl.history:
        _r, n, _m = t.admit(s, len(s), 0)
        t.dec_lock_ref(n)
    ld = max(r.seq_len for r in wl.requests)
    table = np.full((wl.B, ld), -1, np.int32)
    nodes = np.zeros(wl.B, np.int64)
    for r in wl.requests:
        _r, n, _m = t.admit(r.tokens, r.cached, r.new, out_row=table[r.row, :r.seq_len])
        nodes[r.row] = n
    return t, table, nodes


def _decode_view(img):
    n_items, B, G, P = img[1], img[2], img[3], img[4]
    items = img[img[5]:img[5] + 8 * n_items].reshape(n_items, 8)
    item_req = img[img[6]:img[7]].reshape(-1, 4)
    part_ptr = img[img[7]:img[7] + B + 1]
    return items, item_req, part_ptr


def check_plan(wl, t, table, nodes, reqs, base_row):
    Hq, Hkv, D = wl.Hq, wl.Hkv, wl.D
    cached = np.array([r.cached for r in reqs], np.int32)
    seq = np.array([r.seq_len for r in reqs], np.int32)
    p = rs.Plan(t, nodes[base_row:base_row + len(reqs)], cached, seq, Hq, Hkv, D)
    img = p.image()
    assert img[0] == 0x52535031 and img[2] == len(reqs) and img[3] == Hq // Hkv
    items, item_req, part_ptr = _decode_view(img)
    sub = table[base_row:base_row + len(reqs)]
    cover = [np.zeros(s, np.int32) for s in seq]
    owner = {}
    for it_idx, (k0, k1, rep, nreq, off, _a, _b, _c) in enumerate(items):
        assert 0 <= k0 < k1 and 1 <= nreq and nreq * (Hq // Hkv) <= 128
        for j in range(nreq):
            b, pidx, nparts, _z = item_req[off + j]
            assert k1 <= seq[b]
            cover[b][k0:k1] += 1
            # the representative row's slots are this request's slots
            np.testing.assert_array_equal(sub[rep, k0:k1], sub[b, k0:k1])
            # a request's partials are numbered consecutively from part_ptr[b], each once
            assert part_ptr[b] <= pidx < part_ptr[b + 1] and nparts == part_ptr[b + 1] - part_ptr[b]
            assert pidx not in owner
            owner[pidx] = b
    for b in range(len(reqs)):
        assert (cover[b] == 1).all(), b
    assert part_ptr[0] == 0 and part_ptr[-1] == img[4] == len(owner)
    assert img[6] % 4 == 0                      # item_req is read as 16-byte vectors
    uniq = set()
    for b in range(len(reqs)):
        uniq.update(sub[b, :seq[b]].tolist())
    assert p.info["unique_kv_tokens"] == len(uniq)
    assert p.info["flat_kv_tokens"] == int(seq.sum())
    return p


@pytest.mark.parametrize("cfg,n_shared,unique", [(2, 1, 11040), (4, 21, 51264)])
def test_plan_decode_workloads(cfg, n_shared, unique):
    wl = synth.make(cfg)
    t, table, nodes = _admit(wl)
    p = check_plan(wl, t, table, nodes, wl.requests, 0)
    assert p.info["n_shared"] == n_shared
    assert p.info["unique_kv_tokens"] == unique


def test_plan_mixed_batch_decode_half():
    wl = synth.config5()
    t, table, nodes = _admit(wl)
    dec = sorted(wl.decode_requests(), key=lambda r: r.row)
    n_ext = len(wl.extend_requests())
    p = check_plan(wl, t, table, nodes, dec, n_ext)
    assert p.info["n_shared"] >= 1


def test_plan_identical_requests_and_unshared():
    """Two requests with the same context, one sharing a prefix, one sharing nothing."""
    t = rs.Tree(1000)
    rng = np.random.default_rng(1)
    a = rng.integers(0, 100, 300).astype(np.int32)
    c = np.concatenate([a[:120], rng.integers(100, 200, 50).astype(np.int32)])
    d = rng.integers(200, 300, 77).astype(np.int32)
    seqs = [a, a, c, d]
    for s in seqs:
        _r, n, _m = t.admit(s, len(s), 0)
        t.dec_lock_ref(n)
    table = np.full((4, 301), -1, np.int32)
    nodes = np.zeros(4, np.int64)
    for i, s in enumerate(seqs):
        _r, nodes[i], _m = t.admit(s, len(s), 1, out_row=table[i, :len(s) + 1])

    class W:
        Hq, Hkv, D = 8, 2, 128

    class R:
        def __init__(self, s):
            self.cached, self.seq_len = len(s), len(s) + 1
    p = check_plan(W, t, table, nodes, [R(s) for s in seqs], 0)
    # a..a share 300 (120 of it also with c); d is alone
    assert p.info["n_shared"] == 2
    assert p.info["unique_kv_tokens"] == 300 + 50 + 77 + 4


def test_plan_rejects_bad_inputs():
    t = rs.Tree(100)
    _r, n, _m = t.admit(np.arange(10, dtype=np.int32), 10, 1)
    with pytest.raises(rs.RsError):
        rs.Plan(t, [n], [9], [11], 8, 2, 128)           # cached_lens disagrees with the node
    with pytest.raises(rs.RsError):
        rs.Plan(t, [n], [10], [9], 8, 2, 128)           # seq_len < cached
    with pytest.raises(rs.StaleError):
        rs.Plan(t, [12345], [10], [11], 8, 2, 128)

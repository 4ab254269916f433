"""Pins of the oracle attention.

* prefix 0 is textbook causal attention: torch's scaled_dot_product_attention
  in float64 on the CPU (grouped heads through its own enable_gqa mapping);
* prefix > 0 is the same library routine with a bottom-right causal mask;
* one key gives back that key's value row; equal keys give the mean of the
  visible values;
* splitting the keys in two and merging the halves by log-sum-exp gives the
  unsplit result;
* KV gathered from shared pool slots equals KV regenerated from each request's
  own tokens (a token's KV depends only on its prefix), so the attention over
  the shared pool equals per-request recomputation exactly.
"""
import numpy as np
import torch
import torch.nn.functional as F

import oracle
import synth


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa(q, K, V, prefix, sm_scale):
    """torch reference: q [n, Hq, D] at positions prefix..prefix+n-1 over K, V [L, Hkv, D]."""
    n, Hq, D = q.shape
    L, Hkv, _ = K.shape
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]          # [1, Hq, n, D]
    kt = torch.from_numpy(K).permute(1, 0, 2)[None]
    vt = torch.from_numpy(V).permute(1, 0, 2)[None]
    mask = torch.arange(L)[None, :] <= (prefix + torch.arange(n))[:, None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=sm_scale,
                                       enable_gqa=(Hq != Hkv))
    return o[0].permute(1, 0, 2).numpy()


def test_prefix_zero_is_causal_sdpa():
    rng = np.random.default_rng(0)
    for Hq, Hkv, D, L in ((4, 4, 16, 9), (8, 2, 32, 33), (6, 3, 8, 1)):
        q, K, V = _rand(rng, L, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
        s = 1 / np.sqrt(D)
        o, _ = oracle.attend(q, K, V, np.arange(L), s)
        qt = torch.from_numpy(q).permute(1, 0, 2)[None]
        kt = torch.from_numpy(K).permute(1, 0, 2)[None]
        vt = torch.from_numpy(V).permute(1, 0, 2)[None]
        ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=s,
                                             enable_gqa=(Hq != Hkv))[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_extend_over_prefix_is_bottom_right_masked_sdpa():
    rng = np.random.default_rng(1)
    for Hq, Hkv, D, P, n in ((8, 2, 16, 37, 11), (4, 4, 8, 5, 1), (16, 4, 32, 100, 29)):
        L = P + n
        q, K, V = _rand(rng, n, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
        s = 0.3
        o, _ = oracle.attend(q, K, V, P + np.arange(n), s)
        np.testing.assert_allclose(o, _sdpa(q, K, V, P, s), rtol=0, atol=1e-12)


def test_single_key_returns_its_value_and_lse_is_its_logit():
    rng = np.random.default_rng(2)
    q, K, V = _rand(rng, 1, 4, 8), _rand(rng, 1, 2, 8), _rand(rng, 1, 2, 8)
    o, lse = oracle.attend(q, K, V, [0], 0.5)
    for h in range(4):
        np.testing.assert_array_equal(o[0, h], V[0, h // 2])
        assert abs(lse[0, h] - 0.5 * q[0, h] @ K[0, h // 2]) < 1e-12


def test_equal_keys_average_visible_values():
    rng = np.random.default_rng(3)
    L, Hq, Hkv, D = 17, 4, 1, 8
    K = np.repeat(_rand(rng, 1, Hkv, D), L, axis=0)
    V = _rand(rng, L, Hkv, D)
    q = _rand(rng, L, Hq, D)
    o, lse = oracle.attend(q, K, V, np.arange(L), 0.25)
    for p in range(L):
        np.testing.assert_allclose(o[p, 0], V[:p + 1, 0].mean(axis=0), atol=1e-12)
        np.testing.assert_allclose(lse[p, 0], 0.25 * q[p, 0] @ K[0, 0] + np.log(p + 1), atol=1e-12)


def test_lse_merge_of_split_equals_unsplit():
    rng = np.random.default_rng(4)
    L, Hq, Hkv, D = 50, 8, 2, 16
    q, K, V = _rand(rng, 1, Hq, D), _rand(rng, L, Hkv, D), _rand(rng, L, Hkv, D)
    o, lse = oracle.attend(q, K, V, [L - 1], 0.2)
    for a in (1, 7, 25, 49):
        oa, la = oracle.attend(q, K[:a], V[:a], [a - 1], 0.2)
        ob, lb = oracle.attend(q, K[a:], V[a:], [L - 1 - a], 0.2)
        om, lm = oracle.merge_states(oa, la, ob, lb)
        np.testing.assert_allclose(om, o, atol=1e-12)
        np.testing.assert_allclose(lm, lse, atol=1e-12)


def test_lse_is_log_partition_function():
    rng = np.random.default_rng(5)
    q, K, V = _rand(rng, 3, 2, 4), _rand(rng, 6, 1, 4), _rand(rng, 6, 1, 4)
    _o, lse = oracle.attend(q, K, V, [2, 4, 5], 1.0)
    for i, p in enumerate([2, 4, 5]):
        for h in range(2):
            z = sum(np.exp(q[i, h] @ K[j, 0]) for j in range(p + 1))
            assert abs(lse[i, h] - np.log(z)) < 1e-12


def test_shared_pool_equals_per_request_recomputation():
    """The pages' invariant: KV of a token depends only on its prefix, so the
    pool rows the tree shares are exactly each request's own KV."""
    wl = synth.config1()
    vals = synth.Values(wl)
    t = oracle.RadixTree(wl.pool_slots)
    k_pool = np.full((wl.pool_slots, wl.Hkv, wl.D), np.nan, np.float32)
    v_pool = np.full_like(k_pool, np.nan)

    def fill_hist(_i, toks, lo, slots):
        k, v = vals.kv_rows(toks, lo, len(toks))
        k_pool[slots], v_pool[slots] = k, v

    def fill_batch(r, lo, slots):
        k, v = vals.kv_rows(r.tokens, lo, r.seq_len)
        k_pool[slots], v_pool[slots] = k, v

    oracle.admit_history(t, wl.history, fill_hist)
    res = oracle.admit_batch(t, wl, fill_batch)
    for r in wl.requests[:3]:
        row = res["table"][r.row, :r.seq_len]
        k_own, v_own = vals.kv_rows(r.tokens)
        np.testing.assert_array_equal(k_pool[row], k_own)
        np.testing.assert_array_equal(v_pool[row], v_own)
        q = vals.q_rows(r.tokens, r.cached, r.seq_len)
        pos = np.arange(r.cached, r.seq_len)
        o1, l1 = oracle.attend(q, k_pool[row], v_pool[row], pos, wl.sm_scale)
        o2, l2 = oracle.attend(q, k_own, v_own, pos, wl.sm_scale)
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)

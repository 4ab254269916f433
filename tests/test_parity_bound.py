"""CPU control of the per-request bf16 parity check used on the mixed batch.

The check must be able to fail where it matters: on the longest contexts of the mixed
batch (about 32k keys), whose outputs are small.  Here the oracle's own input is damaged
on purpose (one aligned 32-key tile of the context removed) and the check must reject the
result; a correct bf16 computation of the same request (fp32 scores, weights rounded to
bf16 against the first tile's maximum or against no reference point, fp32 sums, output
rounded to bf16) must pass it.
Both a decode request (its one query) and an extend request (query rows at the end of its
512-token chunk) are tried.
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import bf16_request_errors, bf16_request_ok, BF16_MAX_ABS


def _bf(x):
    return synth._round_bf16(np.asarray(x, np.float32)).astype(np.float64)


def _bf16_attention(q, K, V, pos, sm, ref):
    """What a correct bf16 kernel computes, on the CPU: weights exp(s - m) rounded to bf16,
    with m each row's maximum over the first 32 keys (ref="tile0") or m = 0 (ref="none")."""
    n, Hq, D = q.shape
    G = Hq // K.shape[1]
    out = np.empty((n, Hq, D))
    hidden = np.arange(K.shape[0])[None, :] > np.asarray(pos)[:, None]
    for h in range(Hq):
        s = sm * (q[:, h, :].astype(np.float64) @ K[:, h // G, :].T.astype(np.float64))
        s[hidden] = -np.inf
        m = s[:, :32].max(1, keepdims=True) if ref == "tile0" else 0.0
        p = _bf(np.exp(s - m))
        out[:, h, :] = _bf((p @ V[:, h // G, :]) / p.sum(1, keepdims=True))
    return out


@pytest.fixture(scope="module")
def mixed():
    wl = synth.make(5)
    return wl, synth.Values(wl)


@pytest.mark.parametrize("kind", ["decode", "extend"])
@pytest.mark.parametrize("weight_ref", ["tile0", "none"])
def test_check_rejects_one_dropped_tile_at_32k(mixed, kind, weight_ref):
    wl, vals = mixed
    reqs = wl.decode_requests() if kind == "decode" else wl.extend_requests()
    r = max(reqs, key=lambda r: r.seq_len)
    assert r.seq_len > 30000
    k, v = vals.kv_rows(r.tokens, 0, r.seq_len)
    if kind == "decode":
        rows = np.array([r.seq_len - 1])
    else:
        rows = r.cached + np.array([0, 255, r.new - 1])
    q = vals.q_rows(r.tokens, 0, r.seq_len)[rows]
    ref, _ = oracle.attend(q, k, v, rows, wl.sm_scale)
    # a correct bf16 result passes
    good = _bf16_attention(q, k, v, rows, wl.sm_scale, weight_ref)
    assert bf16_request_ok(good, ref), bf16_request_errors(good, ref)
    # one 32-key tile in the middle of the context left out: rejected, although its
    # max-abs error alone is well inside the stated 2e-2
    j = (r.cached // 2) // 32 * 32
    keep = np.r_[0:j, j + 32:r.seq_len]
    bad, _ = oracle.attend(q, k[keep], v[keep], rows - 32, wl.sm_scale)
    mx, rel = bf16_request_errors(bad, ref)
    assert mx < BF16_MAX_ABS
    assert not bf16_request_ok(bad, ref), (mx, rel)

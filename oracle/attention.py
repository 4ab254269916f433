"""Oracle attention in float64: the plain definition, one request at a time.

TEST INFRASTRUCTURE ONLY.  Nothing in the product imports this module.

What it computes.  "How does SGLang work" (modernaiengineering.com), section
"A quick recap of how an LLM generates text": each token's keys and values
depend only on it and the tokens before it, decode attends over the cache
and appends its own keys and values; section "What happens when a request
arrives": the unmatched suffix is prefilled while attending to the reused
entries exactly as if they had just been computed.  The pages never write
the arithmetic out, so the reading is standard causal softmax attention:

    o[p, h] = sum_{j <= p} softmax_j(sm_scale * q[p, h] . K[j, h // G]) V[j, h // G]
    lse[p, h] = log sum_{j <= p} exp(sm_scale * q[p, h] . K[j, h // G])

with G = Hq / Hkv consecutive query heads per KV head, and the natural log.
K and V are the request's own full context, materialised (no sharing).
A decode step is the same formula at the single position p = L - 1.
"""
from __future__ import annotations

import numpy as np


def attend(q, K, V, positions, sm_scale):
    """q [n, Hq, D]; K, V [L, Hkv, D]; positions [n]: query i sees keys 0..positions[i].

    Returns (out [n, Hq, D], lse [n, Hq]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    pos = np.asarray(positions, dtype=np.int64)
    n, Hq, D = q.shape
    L, Hkv, _ = K.shape
    assert Hq % Hkv == 0 and V.shape == K.shape and len(pos) == n
    assert n == 0 or (pos.min() >= 0 and pos.max() < L)
    G = Hq // Hkv
    out = np.empty((n, Hq, D), dtype=np.float64)
    lse = np.empty((n, Hq), dtype=np.float64)
    hidden = np.arange(L)[None, :] > pos[:, None]           # key j not visible to query i
    for h in range(Hq):
        kv = h // G
        s = sm_scale * (q[:, h, :] @ K[:, kv, :].T)          # [n, L]
        s[hidden] = -np.inf
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        out[:, h, :] = (e @ V[:, kv, :]) / z
        lse[:, h] = (m + np.log(z))[:, 0]
    return out, lse


def merge_states(o_a, lse_a, o_b, lse_b):
    """Combine two attention results over disjoint key sets into the result over their union.

    With lse = log sum exp, the union's lse is log(exp(lse_a) + exp(lse_b)) and
    its output is the exp(lse_x - lse)-weighted sum of the two outputs.
    """
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    wa = np.exp(lse_a - m)
    wb = np.exp(lse_b - m)
    lse = m + np.log(wa + wb)
    o = (np.asarray(o_a, np.float64) * (wa / (wa + wb))[..., None]
         + np.asarray(o_b, np.float64) * (wb / (wa + wb))[..., None])
    return o, lse

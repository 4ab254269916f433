"""Pins of the verify-attention oracle against things other than itself.

"SGLang: the tree, and the language nobody remembers" (ai.thesatyajit.com), section
"Speculative decoding puts a tree inside the tree": every verify token attends to the
whole prompt and to its own ancestors (itself included), never to a sibling branch.
The expected results here come from torch's scaled_dot_product_attention in float64 on
the CPU, given a visibility mask typed in by hand for each tree shape:

* a chain (each token's parent is the token before it) is ordinary causal attention
  over prompt + chain, the bottom-right causal mask;
* a star (every token's parent is the root) lets token i see the prompt, the root and
  itself only;
* the page's own example tree, depths [0, 1, 1, 2] (parents -1, 0, 0, 1): token 1 sees
  {0, 1}, token 2 sees {0, 2}, token 3 sees {0, 1, 3}.

A mistake in the oracle's ancestor walk (descendants instead of ancestors, self left
out, siblings let in, the prompt dropped) changes at least one of these.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _data(rng, prefix, n, Hq=8, Hkv=2, D=32):
    q = rng.standard_normal((n, Hq, D))
    kc, vc = rng.standard_normal((prefix, Hkv, D)), rng.standard_normal((prefix, Hkv, D))
    kd, vd = rng.standard_normal((n, Hkv, D)), rng.standard_normal((n, Hkv, D))
    return q, kc, vc, kd, vd


def _sdpa(q, kc, vc, kd, vd, visible_draft, sm):
    """SDPA over keys prompt ++ draft with mask[i, prompt + j] = visible_draft[i][j]."""
    prefix, n = len(kc), len(kd)
    mask = np.zeros((n, prefix + n), bool)
    mask[:, :prefix] = True
    for i, vis in enumerate(visible_draft):
        for j in vis:
            mask[i, prefix + j] = True
    K, V = np.concatenate([kc, kd]), np.concatenate([vc, vd])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).double().permute(1, 0, 2)[None]
    out = F.scaled_dot_product_attention(t(q), t(K), t(V), attn_mask=torch.from_numpy(mask)[None, None],
                                         scale=sm, enable_gqa=True)
    return out[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("prefix,n", [(0, 1), (5, 7), (40, 16), (3, 64)])
def test_chain_tree_is_causal_attention(prefix, n):
    rng = np.random.default_rng(prefix * 100 + n)
    q, kc, vc, kd, vd = _data(rng, prefix, n)
    sm = 0.3
    parents = np.array([-1] + list(range(n - 1)), np.int32)
    got = oracle.speculative.verify_attention(q, kc, vc, kd, vd, parents, sm)
    # the bottom-right causal mask: token i sees draft tokens 0..i
    want = _sdpa(q, kc, vc, kd, vd, [range(i + 1) for i in range(n)], sm)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # and, independently of the mask construction, torch's own causal attention over
    # prompt + chain (its last n rows) when there is no prompt
    if prefix == 0:
        t = lambda a: torch.from_numpy(a).double().permute(1, 0, 2)[None]
        causal = F.scaled_dot_product_attention(t(q), t(kd), t(vd), is_causal=True, scale=sm,
                                                enable_gqa=True)[0].permute(1, 0, 2).numpy()
        np.testing.assert_allclose(got, causal, rtol=0, atol=1e-12)


@pytest.mark.parametrize("prefix,n", [(6, 2), (17, 9), (1, 64)])
def test_star_tree_sees_prompt_root_and_self(prefix, n):
    rng = np.random.default_rng(7 + n)
    q, kc, vc, kd, vd = _data(rng, prefix, n)
    sm = 0.25
    parents = np.array([-1] + [0] * (n - 1), np.int32)
    got = oracle.speculative.verify_attention(q, kc, vc, kd, vd, parents, sm)
    want = _sdpa(q, kc, vc, kd, vd, [[0]] + [[0, i] for i in range(1, n)], sm)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_page_example_tree():
    rng = np.random.default_rng(11)
    q, kc, vc, kd, vd = _data(rng, 7, 4, Hq=4, Hkv=4, D=16)
    sm = 0.5
    got = oracle.speculative.verify_attention(q, kc, vc, kd, vd, np.array([-1, 0, 0, 1], np.int32), sm)
    want = _sdpa(q, kc, vc, kd, vd, [[0], [0, 1], [0, 2], [0, 1, 3]], sm)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_sibling_value_does_not_leak():
    """Closed form: with every score equal (zero keys), token i's output is the mean of the
    values it sees.  In the star tree token 1 sees prompt, root and itself: changing the value
    of its sibling, token 2, leaves it unchanged."""
    prefix, n, Hkv, D = 3, 3, 1, 4
    q = np.ones((n, 2, D))
    kc, kd = np.zeros((prefix, Hkv, D)), np.zeros((n, Hkv, D))
    vc = np.arange(prefix * D, dtype=float).reshape(prefix, Hkv, D)
    vd = 100.0 + np.arange(n * D, dtype=float).reshape(n, Hkv, D)
    parents = np.array([-1, 0, 0], np.int32)
    got = oracle.speculative.verify_attention(q, kc, vc, kd, vd, parents, 1.0)
    want1 = (vc[:, 0].sum(0) + vd[0, 0] + vd[1, 0]) / (prefix + 2)
    np.testing.assert_allclose(got[1, 0], want1, rtol=0, atol=1e-12)
    vd2 = vd.copy()
    vd2[2] += 1000.0
    got2 = oracle.speculative.verify_attention(q, kc, vc, kd, vd2, parents, 1.0)
    np.testing.assert_array_equal(got2[1], got[1])
    np.testing.assert_allclose(got2[2, 0], (vc[:, 0].sum(0) + vd2[0, 0] + vd2[2, 0]) / (prefix + 2), atol=1e-12)

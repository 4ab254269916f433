"""Host-side behaviour of the C ABI that needs no GPU: argument validation (which
returns before any device work), the extend work order and workspace sizing."""
import ctypes as C

import numpy as np
import pytest

import radix_tree_prefix_amd as rs
from radix_tree_prefix_amd import _lib

FAKE = C.c_void_p(0x1000)      # never dereferenced: every call below fails validation first


def test_extend_rejects_unsupported_shapes_before_touching_memory():
    for Hq, Hkv, D in ((8, 8, 96), (8, 3, 128), (256, 1, 128), (0, 1, 64)):
        rc = _lib.lib.rs_extend_attention(FAKE, FAKE, FAKE, FAKE, 8, FAKE, FAKE, FAKE, 1, 4, Hq, Hkv, D,
                                          0.1, _lib.DTYPE_BF16, None, FAKE, None)
        assert rc == _lib.RS_E_UNSUPPORTED, (Hq, Hkv, D)
    rc = _lib.lib.rs_extend_attention(FAKE, FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, 1, 4, 8, 8, 128, 0.1,
                                      _lib.DTYPE_BF16, None, FAKE, None)
    assert rc == _lib.RS_E_INVAL
    # nothing to do is success and touches nothing
    assert _lib.lib.rs_extend_attention(None, None, None, FAKE, 8, None, None, None, 0, 0, 8, 8, 128, 0.1,
                                        _lib.DTYPE_BF16, None, None, None) == _lib.RS_OK


def test_decode_rejects_bad_arguments_before_touching_memory():
    rc = _lib.lib.rs_decode_attention(FAKE, FAKE, FAKE, FAKE, 8, FAKE, 2, 8, 12, 5, 128, 0.1, _lib.DTYPE_BF16,
                                      None, None, FAKE, 1 << 20, FAKE, None, None)
    assert rc == _lib.RS_E_UNSUPPORTED
    # a plan without its device image (or the reverse) is refused
    t = rs.Tree(64)
    _r, n, _m = t.admit(np.arange(5, dtype=np.int32), 5, 1)
    p = rs.Plan(t, [n], [5], [6], 8, 8, 128)
    rc = _lib.lib.rs_decode_attention(FAKE, FAKE, FAKE, FAKE, 8, FAKE, 1, 8, 8, 8, 128, 0.1, _lib.DTYPE_BF16,
                                      p.handle, None, FAKE, 1 << 20, FAKE, None, None)
    assert rc == _lib.RS_E_INVAL
    # a plan built for other heads is refused
    rc = _lib.lib.rs_decode_attention(FAKE, FAKE, FAKE, FAKE, 8, FAKE, 1, 8, 16, 8, 128, 0.1, _lib.DTYPE_BF16,
                                      p.handle, FAKE, FAKE, 1 << 20, FAKE, None, None)
    assert rc == _lib.RS_E_INVAL
    # a workspace smaller than asked for is refused
    need = rs.decode_workspace_bytes(p, 1, 6, 8, 8, 128)
    rc = _lib.lib.rs_decode_attention(FAKE, FAKE, FAKE, FAKE, 8, FAKE, 1, 8, 8, 8, 128, 0.1, _lib.DTYPE_BF16,
                                      p.handle, FAKE, FAKE, need - 1, FAKE, None, None)
    assert rc == _lib.RS_E_INVAL
    assert b"workspace" in _lib.lib.rs_last_error()


def test_store_and_merge_validation():
    assert _lib.lib.rs_store_kv(None, None, None, None, None, 0, 8, 128, _lib.DTYPE_BF16, None) == _lib.RS_OK
    assert _lib.lib.rs_store_kv(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, 7, None) == _lib.RS_E_UNSUPPORTED
    assert _lib.lib.rs_store_kv(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1, 4, _lib.DTYPE_BF16, None) == _lib.RS_E_UNSUPPORTED
    unaligned = C.c_void_p(0x1004)
    assert _lib.lib.rs_store_kv(unaligned, FAKE, FAKE, FAKE, FAKE, 4, 8, 128, _lib.DTYPE_BF16, None) == _lib.RS_E_INVAL
    assert _lib.lib.rs_merge_states(FAKE, FAKE, FAKE, FAKE, 4, 128, 9, FAKE, None, None) == _lib.RS_E_UNSUPPORTED
    assert _lib.lib.rs_merge_states(None, None, None, None, 0, 128, 0, None, None, None) == _lib.RS_OK


def test_extend_order_is_longest_work_first_permutation():
    rng = np.random.default_rng(3)
    pre = rng.integers(0, 30000, 97).astype(np.int32)
    ext = rng.integers(0, 600, 97).astype(np.int32)
    order = rs.extend_order(pre, ext)
    assert sorted(order.tolist()) == list(range(97))
    work = ext.astype(np.int64) * (pre + (ext + 1) // 2)
    w = work[order]
    assert (w[:-1] >= w[1:]).all()
    # ties keep index order
    order2 = rs.extend_order(np.zeros(5, np.int32), np.ones(5, np.int32))
    assert order2.tolist() == [0, 1, 2, 3, 4]


def test_workspace_sizes():
    # flat mode: B x ceil(L / 256) partials per KV head per query head of the group
    b = rs.decode_workspace_bytes(None, 4, 1000, 32, 8, 128)
    P = 4 * 4
    assert b >= 8 * P * 4 * 128 * 4 + 8 * P * 4 * 4
    with pytest.raises(rs.RsError):
        rs.decode_workspace_bytes(None, 4, 1000, 32, 7, 128)

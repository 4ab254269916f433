"""RadixAttention's data-parallel hot path on one MI355X.

A host radix tree (C++) indexes one token-granular KV pool; hand-written HIP
kernels for gfx950 run extend and prefix-aware decode attention through the
tree's index tables.  Everything crosses the C ABI in include/rs.h; this
package only marshals torch tensors and numpy arrays into those calls.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib
from ._lib import (Tree, Plan, RsError, NoSpaceError, StaleError, DTYPE_F32, DTYPE_BF16,  # noqa: F401
                   decode_workspace_bytes, extend_order, draft_tree_build, LIB_PATH)

__all__ = ["Tree", "Plan", "RsError", "NoSpaceError", "StaleError", "store_kv", "extend_attention",
           "decode_attention_noalloc",
           "decode_attention", "merge_states", "DecodeWorkspace", "draft_tree_build", "tree_verify_attention",
           "move_kv", "copy_kv", "host_pool", "LIB_PATH"]

_DT = {torch.float32: DTYPE_F32, torch.bfloat16: DTYPE_BF16}


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise RsError(_lib.RS_E_UNSUPPORTED, f"dtype {t.dtype} (float32 and bfloat16 are implemented)")
    return _DT[t.dtype]


def _stream(stream):
    return (stream if stream is not None else torch.cuda.current_stream()).cuda_stream


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda or not t.is_contiguous():
        raise RsError(_lib.RS_E_INVAL, f"{name} must be a contiguous device tensor")
    if dtype is not None and t.dtype != dtype:
        raise RsError(_lib.RS_E_INVAL, f"{name} must be {dtype}")
    return t.data_ptr()


def store_kv(k_pool, v_pool, k_new, v_new, slots, stream=None):
    """k_pool/v_pool [S, Hkv, D]; k_new/v_new [n, Hkv, D]; slots int32 [n] (device)."""
    S, Hkv, D = k_pool.shape
    _lib.store_kv(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype), _dev(k_new, "k_new", k_pool.dtype),
                  _dev(v_new, "v_new", k_pool.dtype), _dev(slots, "slots", torch.int32), slots.numel(), Hkv, D,
                  _dtype(k_pool), _stream(stream))


def extend_attention(q, k_pool, v_pool, req_to_token, qo_indptr, prefix_lens, extend_lens, max_extend_len,
                     sm_scale, out=None, order=None, stream=None):
    """q [sum(ext), Hq, D]; req_to_token int32 [B, ld]; qo_indptr [B+1], prefix_lens/extend_lens [B] (device);
    order: optional device int32 [B] start order (extend_order)."""
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    B, ld = req_to_token.shape
    out = torch.empty_like(q) if out is None else out
    _lib.extend_attention(_dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype),
                          _dev(req_to_token, "req_to_token", torch.int32), ld,
                          _dev(qo_indptr, "qo_indptr", torch.int32), _dev(prefix_lens, "prefix_lens", torch.int32),
                          _dev(extend_lens, "extend_lens", torch.int32), B, max_extend_len, Hq, Hkv, D, sm_scale,
                          _dtype(k_pool), _dev(out, "out", k_pool.dtype),
                          order=_dev(order, "order", torch.int32) if order is not None else None, stream=_stream(stream))
    return out


def tree_verify_attention(q, k_pool, v_pool, req_to_token, prefix_lens, tree_mask, sm_scale, out=None,
                          stream=None):
    """q [B*n, Hq, D]; req_to_token int32 [B, ld] (row b: prefix slots, then the n verify tokens' slots);
    prefix_lens int32 [B]; tree_mask uint64-as-int64 [B, n] (device, from draft_tree_build)."""
    T, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    B, ld = req_to_token.shape
    n = tree_mask.shape[1]
    assert T == B * n and tree_mask.shape[0] == B
    out = torch.empty_like(q) if out is None else out
    _lib.tree_verify_attention(_dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
                               _dev(v_pool, "v_pool", k_pool.dtype), _dev(req_to_token, "req_to_token", torch.int32),
                               ld, _dev(prefix_lens, "prefix_lens", torch.int32), _dev(tree_mask, "tree_mask",
                                                                                     torch.int64),
                               B, n, Hq, Hkv, D, sm_scale, _dtype(k_pool), _dev(out, "out", k_pool.dtype),
                               _stream(stream))
    return out


def move_kv(k_pool, v_pool, src_slots, dst_slots, stream=None):
    """Copy pool rows src_slots[r] -> dst_slots[r] (device int32 [n]) in both pools."""
    S, Hkv, D = k_pool.shape
    _lib.move_kv(_dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype),
                 _dev(src_slots, "src_slots", torch.int32), _dev(dst_slots, "dst_slots", torch.int32),
                 src_slots.numel(), Hkv, D, _dtype(k_pool), _stream(stream))


def host_pool(shape, dtype=torch.bfloat16):
    """A host-tier pool: a CPU tensor in pinned memory from rs_host_alloc, which rs_copy_kv
    may read and write (other host memory it refuses)."""
    n = 1
    for x in shape:
        n *= int(x)
    nbytes = max(n * torch.empty((), dtype=dtype).element_size(), 1)
    arr = np.frombuffer(_lib.host_alloc(nbytes), dtype=np.uint8)
    return torch.from_numpy(arr).view(dtype).view(*shape)


def _pool(t: torch.Tensor, name: str, dtype=None):
    """A device tensor, or a host pool (host_pool)."""
    if not t.is_contiguous():
        raise RsError(_lib.RS_E_INVAL, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise RsError(_lib.RS_E_INVAL, f"{name} must be {dtype}")
    return t.data_ptr()


def copy_kv(dst_k, dst_v, src_k, src_v, dst_slots, src_slots, stream=None):
    """dst pools[dst_slots[r]] = src pools[src_slots[r]] (slot arrays device int32 [n]); pools
    [rows, Hkv, D], on the device or pinned on the host (the host tier's copies)."""
    R, Hkv, D = dst_k.shape
    S = src_k.shape[0]
    if tuple(src_k.shape[1:]) != (Hkv, D) or dst_v.shape != dst_k.shape or src_v.shape != src_k.shape:
        raise RsError(_lib.RS_E_INVAL, "copy_kv: pool shapes differ")
    if dst_slots.numel() != src_slots.numel():
        raise RsError(_lib.RS_E_INVAL, "copy_kv: slot arrays differ in length")
    _lib.copy_kv(_pool(dst_k, "dst_k"), _pool(dst_v, "dst_v", dst_k.dtype), _pool(src_k, "src_k", dst_k.dtype),
                 _pool(src_v, "src_v", dst_k.dtype), _dev(dst_slots, "dst_slots", torch.int32),
                 _dev(src_slots, "src_slots", torch.int32), src_slots.numel(), R, S, Hkv, D, _dtype(dst_k),
                 _stream(stream))


class DecodeWorkspace:
    """Device workspace for rs_decode_attention (per-item partial outputs and lse)."""

    def __init__(self, plan, B, max_seq_len, Hq, Hkv, D, device="cuda", stream=None):
        self.nbytes = decode_workspace_bytes(plan, B, max_seq_len, Hq, Hkv, D)
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        _lib.decode_workspace_init(self.buf.data_ptr(), self.nbytes, _stream(stream))


def upload_plan(plan: Plan, device="cuda", stream=None):
    """Device image of a plan (uint8 tensor); the plan must outlive the copy."""
    dev = torch.empty(plan.nbytes, dtype=torch.uint8, device=device)
    plan.upload(dev.data_ptr(), _stream(stream))
    return dev


def decode_attention(q, k_pool, v_pool, req_to_token, seq_lens, max_seq_len, sm_scale, workspace, plan=None,
                     plan_dev=None, out=None, lse=None, stream=None):
    """q [B, Hq, D]; req_to_token int32 [B, ld]; seq_lens int32 [B] (device).  Returns out (and fills lse)."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    ld = req_to_token.shape[1]
    out = torch.empty_like(q) if out is None else out
    _lib.decode_attention(_dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"), _dev(v_pool, "v_pool", k_pool.dtype),
                          _dev(req_to_token, "req_to_token", torch.int32), ld, _dev(seq_lens, "seq_lens", torch.int32),
                          B, max_seq_len, Hq, Hkv, D, sm_scale, _dtype(k_pool), plan,
                          plan_dev.data_ptr() if plan_dev is not None else None,
                          workspace.buf.data_ptr(), workspace.nbytes, _dev(out, "out", k_pool.dtype),
                          _dev(lse, "lse", torch.float32) if lse is not None else None, _stream(stream))
    return out


def decode_attention_noalloc(q, k_pool, v_pool, req_to_token, seq_lens, max_seq_len, sm_scale, out, plan=None,
                             plan_dev=None, lse=None, stream=None):
    """decode_attention with the library's static workspace: allocates nothing (out is required)."""
    B, Hq, D = q.shape
    Hkv = k_pool.shape[1]
    ld = req_to_token.shape[1]
    _lib.decode_attention_noalloc(_dev(q, "q", k_pool.dtype), _dev(k_pool, "k_pool"),
                                  _dev(v_pool, "v_pool", k_pool.dtype), _dev(req_to_token, "req_to_token", torch.int32),
                                  ld, _dev(seq_lens, "seq_lens", torch.int32), B, max_seq_len, Hq, Hkv, D, sm_scale,
                                  _dtype(k_pool), plan, plan_dev.data_ptr() if plan_dev is not None else None,
                                  _dev(out, "out", k_pool.dtype),
                                  _dev(lse, "lse", torch.float32) if lse is not None else None, _stream(stream))
    return out


def merge_states(o_a, lse_a, o_b, lse_b, out=None, lse=None, stream=None):
    """o_* [rows, D] (float32 or bfloat16), lse_* float32 [rows]."""
    rows, D = o_a.shape
    out = torch.empty_like(o_a) if out is None else out
    _lib.merge_states(_dev(o_a, "o_a"), _dev(lse_a, "lse_a", torch.float32), _dev(o_b, "o_b", o_a.dtype),
                      _dev(lse_b, "lse_b", torch.float32), rows, D, _dtype(o_a), _dev(out, "out", o_a.dtype),
                      _dev(lse, "lse", torch.float32) if lse is not None else None, _stream(stream))
    return out

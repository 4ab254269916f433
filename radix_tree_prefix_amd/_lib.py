"""ctypes binding of librs (include/rs.h): argument marshalling only.

Every call forwards to the C ABI; host arrays are numpy, device arrays are torch
tensors (only their data pointers cross), streams are torch HIP streams.
Importing this module fails loudly if librs.so has not been built.
"""
from __future__ import annotations

import ctypes as C
import os
import weakref

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librs.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("librs.so is not built: run `python radix_tree_prefix_amd/build.py` "
                      "(or __graft_entry__.build()) first")

lib = C.CDLL(LIB_PATH)

RS_OK, RS_E_INVAL, RS_E_NOSPACE, RS_E_STALE, RS_E_HIP, RS_E_UNSUPPORTED = 0, -1, -2, -3, -4, -5
SCHED_POLICIES = {"fcfs": 0, "lpm": 1, "dfs-weight": 2}
DTYPE_F32, DTYPE_BF16 = 0, 1
_NAMES = {RS_E_INVAL: "RS_E_INVAL", RS_E_NOSPACE: "RS_E_NOSPACE", RS_E_STALE: "RS_E_STALE",
          RS_E_HIP: "RS_E_HIP", RS_E_UNSUPPORTED: "RS_E_UNSUPPORTED"}


class RsError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{_NAMES.get(code, code)}: {msg}")
        self.code = code


class NoSpaceError(RsError):
    pass


class StaleError(RsError):
    pass


def _check(rc):
    if rc < 0:
        msg = lib.rs_last_error().decode()
        cls = NoSpaceError if rc == RS_E_NOSPACE else StaleError if rc == RS_E_STALE else RsError
        raise cls(rc, msg)
    return rc


class Stats(C.Structure):
    _fields_ = [(n, C.c_int64) for n in (
        "pool_slots", "nodes", "tree_tokens", "evictable", "protected", "free_slots", "evicted_total",
        "clock", "matched_total", "match_calls", "insert_calls", "host_slots", "host_tokens", "host_free")] + \
        [("reserved", C.c_int64 * 2)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_ if n != "reserved"}


class PlanInfo(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("B", "Hq", "Hkv", "D", "n_items", "n_segments", "n_shared", "chunk")] + \
               [(n, C.c_int64) for n in ("n_partials", "unique_kv_tokens", "flat_kv_tokens", "bytes")] + \
               [("reserved", C.c_int64 * 4)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_ if n != "reserved"}


_P = C.c_void_p
_I32P = C.POINTER(C.c_int32)
_I64P = C.POINTER(C.c_int64)
_SIGS = {
    "rs_last_error": (C.c_char_p, []),
    "rs_version": (C.c_char_p, []),
    "rs_tree_create": (_P, [C.c_int64, C.c_int32]),
    "rs_tree_destroy": (None, [_P]),
    "rs_match_prefix": (C.c_int, [_P, _P, C.c_int64, _P, _I64P, _I64P]),
    "rs_inc_lock_ref": (C.c_int, [_P, C.c_int64]),
    "rs_dec_lock_ref": (C.c_int, [_P, C.c_int64]),
    "rs_alloc_slots": (C.c_int, [_P, C.c_int64, _P]),
    "rs_free_slots": (C.c_int, [_P, _P, C.c_int64]),
    "rs_insert": (C.c_int, [_P, _P, _P, C.c_int64, _I64P, _I64P]),
    "rs_evict": (C.c_int64, [_P, C.c_int64]),
    "rs_admit": (C.c_int, [_P, _P, C.c_int64, C.c_int64, _P, _I64P, _I64P]),
    "rs_stats": (C.c_int, [_P, C.POINTER(Stats)]),
    "rs_tree_dump": (C.c_int, [_P, C.c_char_p, C.c_int64, _I64P]),
    "rs_schedule": (C.c_int, [_P, _P, _P, C.c_int32, C.c_int32, _P, _P]),
    "rs_decode_plan_build": (C.c_int, [_P, _P, _P, _P, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                       C.POINTER(C.c_void_p)]),
    "rs_plan_info": (C.c_int, [_P, C.POINTER(PlanInfo)]),
    "rs_decode_plan_bytes": (C.c_int64, [_P]),
    "rs_decode_plan_upload": (C.c_int, [_P, _P, _P]),
    "rs_decode_plan_read": (C.c_int, [_P, _P, C.c_int64]),
    "rs_plan_destroy": (None, [_P]),
    "rs_decode_workspace_bytes": (C.c_int64, [_P, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32]),
    "rs_decode_workspace_init": (C.c_int, [_P, C.c_int64, _P]),
    "rs_store_kv": (C.c_int, [_P, _P, _P, _P, _P, C.c_int64, C.c_int32, C.c_int32, C.c_int32, _P]),
    "rs_extend_attention": (C.c_int, [_P, _P, _P, _P, C.c_int64, _P, _P, _P, C.c_int32, C.c_int32, C.c_int32,
                                      C.c_int32, C.c_int32, C.c_float, C.c_int32, _P, _P, _P]),
    "rs_extend_order": (C.c_int, [_P, _P, C.c_int32, _P]),
    "rs_draft_tree_build": (C.c_int, [_P, _P, C.c_int32, C.c_int32, _P, _P, _P, _P]),
    "rs_tree_verify_attention": (C.c_int, [_P, _P, _P, _P, C.c_int64, _P, _P, C.c_int32, C.c_int32, C.c_int32,
                                           C.c_int32, C.c_int32, C.c_float, C.c_int32, _P, _P]),
    "rs_move_kv": (C.c_int, [_P, _P, _P, _P, C.c_int64, C.c_int32, C.c_int32, C.c_int32, _P]),
    "rs_copy_kv": (C.c_int, [_P, _P, _P, _P, _P, _P, C.c_int64, C.c_int64, C.c_int64, C.c_int32, C.c_int32,
                             C.c_int32, _P]),
    "rs_host_alloc": (C.c_int, [C.c_int64, C.POINTER(C.c_void_p)]),
    "rs_host_free": (C.c_int, [_P]),
    "rs_host_tier_enable": (C.c_int, [_P, C.c_int64]),
    "rs_match_prefix2": (C.c_int, [_P, _P, C.c_int64, _P, _P, _I64P, _I64P, _I64P, _I64P]),
    "rs_write_through": (C.c_int, [_P, C.c_int64, C.c_int64, _P, _P, _I64P, _I64P]),
    "rs_load_back": (C.c_int, [_P, C.c_int64, C.c_int64, _P, _P, _I64P, _I64P]),
    "rs_commit": (C.c_int, [_P, C.c_int64, C.c_int32]),
    "rs_evict_host": (C.c_int64, [_P, C.c_int64]),
    "rs_decode_attention": (C.c_int, [_P, _P, _P, _P, C.c_int64, _P, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                      C.c_int32, C.c_float, C.c_int32, _P, _P, _P, C.c_int64, _P, _P, _P]),
    "rs_decode_attention_noalloc": (C.c_int, [_P, _P, _P, _P, C.c_int64, _P, C.c_int32, C.c_int32, C.c_int32,
                                              C.c_int32, C.c_int32, C.c_float, C.c_int32, _P, _P, _P, _P, _P]),
    "rs_merge_states": (C.c_int, [_P, _P, _P, _P, C.c_int64, C.c_int32, C.c_int32, _P, _P, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTS = tuple(_SIGS)


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(C.c_void_p)


def _i64(a):
    a = np.ascontiguousarray(a, dtype=np.int64)
    return a, a.ctypes.data_as(C.c_void_p)


def pack_queue(queue):
    """A list of token sequences as (int32 tokens, int64 offsets[n+1]) for rs_schedule."""
    offs = np.zeros(len(queue) + 1, np.int64)
    np.cumsum([len(q) for q in queue], out=offs[1:])
    tok = np.concatenate([np.asarray(q, np.int32) for q in queue]) if len(queue) else np.zeros(0, np.int32)
    return tok, offs


# ------------------------------------------------------------------ tree
class Tree:
    """Host radix tree over pool slots 0..pool_slots-1 (rs_tree_* calls)."""

    def __init__(self, pool_slots: int, page_size: int = 1):
        h = lib.rs_tree_create(int(pool_slots), int(page_size))
        if not h:
            raise RsError(RS_E_INVAL, lib.rs_last_error().decode())
        self._h = C.c_void_p(h)
        self.pool_slots = int(pool_slots)
        self.host_slots = 0

    def close(self):
        if self._h:
            lib.rs_tree_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self):
        return self._h

    def match_prefix(self, tokens, out=None):
        tok, tp = _i32(tokens)
        buf = np.empty(len(tok), np.int32) if out is None else out
        n, node = C.c_int64(), C.c_int64()
        _check(lib.rs_match_prefix(self._h, tp, len(tok), buf.ctypes.data_as(C.c_void_p), C.byref(n), C.byref(node)))
        return buf[:n.value], node.value

    def inc_lock_ref(self, node):
        _check(lib.rs_inc_lock_ref(self._h, int(node)))

    def dec_lock_ref(self, node):
        _check(lib.rs_dec_lock_ref(self._h, int(node)))

    def alloc(self, n):
        out = np.empty(int(n), np.int32)
        _check(lib.rs_alloc_slots(self._h, int(n), out.ctypes.data_as(C.c_void_p)))
        return out

    def free_slots(self, slots):
        s, sp = _i32(slots)
        _check(lib.rs_free_slots(self._h, sp, len(s)))

    def insert(self, tokens, slots):
        tok, tp = _i32(tokens)
        s = np.array(slots, dtype=np.int32, copy=True)
        assert len(s) == len(tok)
        pre, node = C.c_int64(), C.c_int64()
        _check(lib.rs_insert(self._h, tp, s.ctypes.data_as(C.c_void_p), len(tok), C.byref(pre), C.byref(node)))
        return pre.value, node.value, s

    def evict(self, num_tokens):
        return _check(lib.rs_evict(self._h, int(num_tokens)))

    def admit(self, tokens, cached, new, out_row=None):
        tok, tp = _i32(tokens)
        row = np.empty(int(cached) + int(new), np.int32) if out_row is None else out_row
        node, m = C.c_int64(), C.c_int64()
        _check(lib.rs_admit(self._h, tp, int(cached), int(new), row.ctypes.data_as(C.c_void_p),
                            C.byref(node), C.byref(m)))
        return row, node.value, m.value

    def schedule(self, queue, policy="lpm"):
        """Order of a waiting queue (list of token arrays): (order, matched) from rs_schedule."""
        return self.schedule_packed(*pack_queue(queue), policy)

    def schedule_packed(self, tokens, offsets, policy="lpm"):
        """rs_schedule on a queue already packed as (int32 tokens, int64 offsets[n+1])."""
        tok, tp = _i32(tokens)
        offs, op = _i64(offsets)
        n = len(offs) - 1
        order = np.empty(n, np.int32)
        matched = np.empty(n, np.int64)
        _check(lib.rs_schedule(self._h, tp, op, n, SCHED_POLICIES[policy], order.ctypes.data_as(C.c_void_p),
                               matched.ctypes.data_as(C.c_void_p)))
        return order, matched

    # -------------------------------------------------------------- host tier
    def enable_host(self, host_slots):
        _check(lib.rs_host_tier_enable(self._h, int(host_slots)))
        self.host_slots = int(host_slots)

    def match2(self, tokens):
        """(device slots, host slots, device length, total length, device node, last node)."""
        tok, tp = _i32(tokens)
        dev = np.empty(len(tok), np.int32)
        host = np.empty(len(tok), np.int32)
        dl, tl, dn, nd = C.c_int64(), C.c_int64(), C.c_int64(), C.c_int64()
        _check(lib.rs_match_prefix2(self._h, tp, len(tok), dev.ctypes.data_as(C.c_void_p),
                                    host.ctypes.data_as(C.c_void_p), C.byref(dl), C.byref(tl), C.byref(dn),
                                    C.byref(nd)))
        return dev[:dl.value], host[:tl.value - dl.value], dl.value, tl.value, dn.value, nd.value

    def _pairs(self, fn, node, cap):
        a = np.empty(cap, np.int32)
        b = np.empty(cap, np.int32)
        n, tk = C.c_int64(), C.c_int64()
        _check(fn(self._h, int(node), cap, a.ctypes.data_as(C.c_void_p), b.ctypes.data_as(C.c_void_p),
                  C.byref(n), C.byref(tk)))
        return a[:n.value], b[:n.value], tk.value

    def write_through(self, node):
        """(device slots, host slots, ticket): the rows to copy to the host tier."""
        return self._pairs(lib.rs_write_through, node, self.host_slots)

    def load_back(self, node):
        """(host slots, device slots, ticket): the rows to copy back to the device."""
        return self._pairs(lib.rs_load_back, node, self.pool_slots)

    def commit(self, ticket, success=True):
        _check(lib.rs_commit(self._h, int(ticket), 1 if success else 0))

    def evict_host(self, num_tokens):
        return _check(lib.rs_evict_host(self._h, int(num_tokens)))

    def stats(self):
        s = Stats()
        _check(lib.rs_stats(self._h, C.byref(s)))
        return s.as_dict()

    def dump(self):
        need = C.c_int64()
        _check(lib.rs_tree_dump(self._h, None, 0, C.byref(need)))
        buf = C.create_string_buffer(need.value + 1)
        _check(lib.rs_tree_dump(self._h, buf, need.value + 1, C.byref(need)))
        return buf.raw[:need.value].decode()


# ------------------------------------------------------------------ plan
class Plan:
    """Decode plan (rs_decode_plan_*): segments of a decode batch from the tree."""

    def __init__(self, tree: Tree, nodes, cached_lens, seq_lens, Hq, Hkv, D):
        nd, ndp = _i64(nodes)
        cl, clp = _i32(cached_lens)
        sl, slp = _i32(seq_lens)
        h = C.c_void_p()
        _check(lib.rs_decode_plan_build(tree.handle, ndp, clp, slp, len(nd), int(Hq), int(Hkv), int(D), C.byref(h)))
        self._h = h
        info = PlanInfo()
        _check(lib.rs_plan_info(self._h, C.byref(info)))
        self.info = info.as_dict()

    @property
    def handle(self):
        return self._h

    @property
    def nbytes(self):
        return _check(lib.rs_decode_plan_bytes(self._h))

    def image(self):
        """The device image as int32 words (host copy)."""
        buf = np.empty(self.nbytes // 4, np.int32)
        _check(lib.rs_decode_plan_read(self._h, buf.ctypes.data_as(C.c_void_p), buf.nbytes))
        return buf

    def upload(self, dev_ptr, stream=None):
        _check(lib.rs_decode_plan_upload(self._h, C.c_void_p(dev_ptr), C.c_void_p(stream or 0)))

    def close(self):
        if self._h:
            lib.rs_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def decode_workspace_bytes(plan, B, max_seq_len, Hq, Hkv, D):
    return _check(lib.rs_decode_workspace_bytes(plan.handle if plan is not None else None,
                                                int(B), int(max_seq_len), int(Hq), int(Hkv), int(D)))


# ------------------------------------------------------------------ device ops (raw pointers)
def decode_workspace_init(ws_ptr, nbytes, stream=0):
    _check(lib.rs_decode_workspace_init(C.c_void_p(ws_ptr), int(nbytes), C.c_void_p(stream)))


def store_kv(k_pool, v_pool, k_new, v_new, slots, n, Hkv, D, dtype, stream=0):
    _check(lib.rs_store_kv(k_pool, v_pool, k_new, v_new, slots, int(n), int(Hkv), int(D), int(dtype),
                           C.c_void_p(stream)))


def extend_attention(q, k_pool, v_pool, req_to_token, ld, qo_indptr, prefix_lens, extend_lens, B, max_extend_len,
                     Hq, Hkv, D, sm_scale, dtype, out, order=None, stream=0):
    _check(lib.rs_extend_attention(q, k_pool, v_pool, req_to_token, int(ld), qo_indptr, prefix_lens, extend_lens,
                                   int(B), int(max_extend_len), int(Hq), int(Hkv), int(D), float(sm_scale),
                                   int(dtype), order, out, C.c_void_p(stream)))


def draft_tree_build(parents, prefix_lens):
    """Host: (tree_mask uint64, positions, next_token, next_sibling), each [B, n], of draft trees
    given by parents (int32 [B, n], token 0 the root with parent -1)."""
    par = np.ascontiguousarray(parents, dtype=np.int32)
    B, n = par.shape
    pl, plp = _i32(prefix_lens)
    assert len(pl) == B
    mask = np.empty((B, n), np.uint64)
    pos, nt, ns = (np.empty((B, n), np.int32) for _ in range(3))
    _check(lib.rs_draft_tree_build(par.ctypes.data_as(C.c_void_p), plp, B, n, mask.ctypes.data_as(C.c_void_p),
                                   pos.ctypes.data_as(C.c_void_p), nt.ctypes.data_as(C.c_void_p),
                                   ns.ctypes.data_as(C.c_void_p)))
    return mask, pos, nt, ns


def tree_verify_attention(q, k_pool, v_pool, req_to_token, ld, prefix_lens, tree_mask, B, n, Hq, Hkv, D, sm_scale,
                          dtype, out, stream=0):
    _check(lib.rs_tree_verify_attention(q, k_pool, v_pool, req_to_token, int(ld), prefix_lens, tree_mask, int(B),
                                        int(n), int(Hq), int(Hkv), int(D), float(sm_scale), int(dtype), out,
                                        C.c_void_p(stream)))


def host_alloc(nbytes):
    """A pinned host block from rs_host_alloc as a ctypes byte array; rs_host_free runs when the
    array (and every view of it) is gone."""
    p = C.c_void_p()
    _check(lib.rs_host_alloc(int(nbytes), C.byref(p)))
    buf = (C.c_uint8 * int(nbytes)).from_address(p.value)
    weakref.finalize(buf, lib.rs_host_free, C.c_void_p(p.value))
    return buf


def copy_kv(dst_k, dst_v, src_k, src_v, dst_slots, src_slots, n, dst_rows, src_rows, Hkv, D, dtype, stream=0):
    _check(lib.rs_copy_kv(dst_k, dst_v, src_k, src_v, dst_slots, src_slots, int(n), int(dst_rows), int(src_rows),
                          int(Hkv), int(D), int(dtype), C.c_void_p(stream)))


def move_kv(k_pool, v_pool, src, dst, n, Hkv, D, dtype, stream=0):
    _check(lib.rs_move_kv(k_pool, v_pool, src, dst, int(n), int(Hkv), int(D), int(dtype), C.c_void_p(stream)))


def extend_order(prefix_lens, extend_lens):
    """Host: longest-work-first request order for extend_attention."""
    p, pp = _i32(prefix_lens)
    e, ep = _i32(extend_lens)
    out = np.empty(len(p), np.int32)
    _check(lib.rs_extend_order(pp, ep, len(p), out.ctypes.data_as(C.c_void_p)))
    return out


def decode_attention(q, k_pool, v_pool, req_to_token, ld, seq_lens, B, max_seq_len, Hq, Hkv, D, sm_scale, dtype,
                     plan, plan_dev, ws, ws_bytes, out, lse_out, stream=0):
    _check(lib.rs_decode_attention(q, k_pool, v_pool, req_to_token, int(ld), seq_lens, int(B), int(max_seq_len),
                                   int(Hq), int(Hkv), int(D), float(sm_scale), int(dtype),
                                   plan.handle if plan is not None else None, plan_dev, ws, int(ws_bytes), out,
                                   lse_out, C.c_void_p(stream)))


def decode_attention_noalloc(q, k_pool, v_pool, req_to_token, ld, seq_lens, B, max_seq_len, Hq, Hkv, D, sm_scale,
                             dtype, plan, plan_dev, out, lse_out, stream=0):
    _check(lib.rs_decode_attention_noalloc(q, k_pool, v_pool, req_to_token, int(ld), seq_lens, int(B),
                                           int(max_seq_len), int(Hq), int(Hkv), int(D), float(sm_scale), int(dtype),
                                           plan.handle if plan is not None else None, plan_dev, out, lse_out,
                                           C.c_void_p(stream)))


def merge_states(o_a, lse_a, o_b, lse_b, rows, D, dtype, o, lse, stream=0):
    _check(lib.rs_merge_states(o_a, lse_a, o_b, lse_b, int(rows), int(D), int(dtype), o, lse, C.c_void_p(stream)))

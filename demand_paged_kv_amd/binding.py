"""ctypes binding of libgrowpage (argument marshalling only).

Every function takes tensors (anything with ``data_ptr()``) or raw integer device
addresses, builds the C structs, calls the library on the current HIP stream and
raises ``GrowPageError`` on a non-OK status.  All compute happens in the HIP kernels;
there is no fallback: a missing library raises at import of the first call.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgrowpage.so")

GP_OK, GP_ERR_INVALID, GP_ERR_HIP, GP_ERR_SCRATCH, GP_ERR_UNSUPPORTED = 0, 1, 2, 3, 4
GP_F32, GP_BF16 = 0, 1
GP_REQ_GROW_DENIED, GP_REQ_DEFERRED, GP_REQ_NOT_AT_BOUNDARY, GP_REQ_OVERFLOW = 1, 2, 4, 8
GP_DECISION_COMPACT, GP_DECISION_GROW, GP_DECISION_SHRINK = 0, 1, 2
COUNTER_NAMES = ("grows", "compacts", "grow_denied", "deferred", "cow_pages", "freed_pages",
                 "moved_rows", "copied_rows", "shrinks")
GP_NUM_COUNTERS = len(COUNTER_NAMES)

EXPORTED = ("gp_abi_version", "gp_status_string", "gp_last_hip_error_string", "gp_update_summaries",
            "gp_scratch_bytes",
            "gp_boundary_scan", "gp_decide", "gp_decide_policy", "gp_compact", "gp_compact_prepare",
            "gp_compact_move", "gp_append_kv", "gp_decode_attention", "gp_contiguous_malloc",
            "gp_contiguous_free", "gp_scan_logits", "gp_boundary_step_static")
GP_STATIC_SCRATCH_BYTES = 64 << 20
# decision policies (gp_decide_policy)
POLICIES = {"growpage": 0, "random": 1, "inverse": 2, "always_compact": 3, "shrink": 4}


class GrowPageError(RuntimeError):
    pass


class Params(ctypes.Structure):
    _fields_ = [("beta_s", ctypes.c_float), ("beta_l", ctypes.c_float), ("top_p", ctypes.c_float),
                ("tau", ctypes.c_int32), ("n_local", ctypes.c_int32), ("shrink", ctypes.c_int32)]


class KV(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("d", ctypes.c_int32), ("P", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("stride_layer", ctypes.c_int64), ("stride_page", ctypes.c_int64),
                ("stride_head", ctypes.c_int64), ("stride_tok", ctypes.c_int64)]


class Pages(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("max_req", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("n_alloc", ctypes.c_void_p),
                ("fill", ctypes.c_void_p), ("refcount", ctypes.c_void_p),
                ("free_stack", ctypes.c_void_p), ("free_top", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgrowpage.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise GrowPageError(f"{path} not found: build it with `python -m demand_paged_kv_amd.build`")
    # torch ships its own HIP runtime; load it first so that the library binds to the same
    # runtime (one HIP runtime per process), otherwise torch's streams and pointers would
    # be foreign to the runtime the library launches on.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.gp_abi_version.restype = i32
    lib.gp_status_string.restype = ctypes.c_char_p
    lib.gp_status_string.argtypes = [i32]
    lib.gp_last_hip_error_string.restype = ctypes.c_char_p
    lib.gp_update_summaries.restype = i32
    lib.gp_update_summaries.argtypes = [P, i32, i64, i64, i64, P, i32, i32, i32, i32, P, P,
                                        ctypes.POINTER(Params), P]
    lib.gp_scratch_bytes.restype = sz
    lib.gp_scratch_bytes.argtypes = [ctypes.POINTER(KV), i32, i64]
    lib.gp_boundary_scan.restype = i32
    lib.gp_boundary_scan.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Pages), P, i32, P, P, P, P,
                                     i32, P, ctypes.POINTER(Params), P, P, P, sz, i64, P]
    lib.gp_boundary_step_static.restype = i32
    lib.gp_boundary_step_static.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Pages), P, i32, P, P, P, P, i32,
                                            P, ctypes.POINTER(Params), i64, P, P, P, P, P, P, P, P]
    lib.gp_scan_logits.restype = i32
    lib.gp_scan_logits.argtypes = [ctypes.POINTER(KV), i32, i64, P, sz, i32, i32, P, P]
    lib.gp_decide.restype = i32
    lib.gp_decide.argtypes = [P, P, i32, i32, i32, i32, ctypes.POINTER(Params),
                              ctypes.POINTER(Pages), P, P, P, P, P]
    lib.gp_decide_policy.restype = i32
    lib.gp_decide_policy.argtypes = [P, P, i32, i32, i32, i32, ctypes.POINTER(Params), i32, P,
                                     ctypes.c_float, ctypes.POINTER(Pages), P, P, P, P, P]
    lib.gp_compact.restype = i32
    lib.gp_compact.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Pages), P, P, i32,
                               ctypes.POINTER(Params), P, P, P, P, sz, i64, P]
    lib.gp_compact_prepare.restype = i32
    lib.gp_compact_prepare.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Pages), P, P, i32,
                                       ctypes.POINTER(Params), P, P, P, sz, i64, P]
    lib.gp_compact_move.restype = i32
    lib.gp_compact_move.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Pages), P, i32, P, P, sz,
                                    i64, P]
    lib.gp_decode_attention.restype = i32
    lib.gp_decode_attention.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Pages), P, i32, i64, i64, i64, P,
                                        i32, P, P, i32, P, P, P]
    lib.gp_append_kv.restype = i32
    lib.gp_append_kv.argtypes = [ctypes.POINTER(KV), ctypes.POINTER(Pages), P, P, P, i32, P, P]
    lib.gp_contiguous_malloc.restype = P
    lib.gp_contiguous_malloc.argtypes = [i64, i32, P]
    lib.gp_contiguous_free.restype = None
    lib.gp_contiguous_free.argtypes = [P, i64, i32, P]
    _lib = lib
    return lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream) or None
    if isinstance(stream, int):
        return stream or None
    return int(stream.cuda_stream) or None


def _check(status: int, what: str):
    if status != GP_OK:
        lib = load()
        msg = lib.gp_status_string(status).decode()
        if status == GP_ERR_HIP:
            msg += f" ({lib.gp_last_hip_error_string().decode()})"
        raise GrowPageError(f"{what}: {msg}")


def params(beta_s=0.9, beta_l=0.999, top_p=0.9, tau=0, n_local=64, shrink=0) -> Params:
    return Params(float(beta_s), float(beta_l), float(top_p), int(tau), int(n_local), int(shrink))


def params_from(d: dict) -> Params:
    return params(d["beta_s"], d["beta_l"], d["top_p"], d["tau"], d["n_local"],
                  1 if d.get("policy") == "shrink" else 0)


def make_kv(k, v, L, Hq, Hkv, d, P, num_pages, dtype, strides=None) -> KV:
    """K/V pools; default layout [L][num_pages][Hkv][P][d] contiguous."""
    if strides is None:
        strides = (num_pages * Hkv * P * d, Hkv * P * d, P * d, d)
    return KV(L, Hq, Hkv, d, P, num_pages, dtype, _ptr(k), _ptr(v), *[int(s) for s in strides])


def make_pages(page_table, n_alloc, fill, refcount, free_stack, free_top) -> Pages:
    max_req, max_pages = page_table.shape
    return Pages(_ptr(page_table), int(max_req), int(max_pages), _ptr(n_alloc), _ptr(fill),
                 _ptr(refcount), _ptr(free_stack), _ptr(free_top))


# ----------------------------------------------------------------------------- entry points
def update_summaries(q, q_dtype, q_strides, req_ids, n_req, L, Hq, d, sum_s, sum_l, prm: Params,
                     stream=None):
    st = load().gp_update_summaries(_ptr(q), q_dtype, *[int(s) for s in q_strides], _ptr(req_ids),
                                    int(n_req), L, Hq, d, _ptr(sum_s), _ptr(sum_l),
                                    ctypes.byref(prm), _stream(stream))
    _check(st, "gp_update_summaries")


def scratch_bytes(kv: KV, n_req: int, max_total_tokens: int) -> int:
    return int(load().gp_scratch_bytes(ctypes.byref(kv), int(n_req), int(max_total_tokens)))


def boundary_scan(kv: KV, pages: Pages, req_ids, n_req, sum_s, sum_l, rope_cos, rope_sin,
                  rope_max_pos, pos, prm: Params, ws_out, stats_out, scratch, scratch_nbytes,
                  max_total_tokens, stream=None):
    st = load().gp_boundary_scan(ctypes.byref(kv), ctypes.byref(pages), _ptr(req_ids), int(n_req),
                                 _ptr(sum_s), _ptr(sum_l), _ptr(rope_cos), _ptr(rope_sin),
                                 int(rope_max_pos), _ptr(pos), ctypes.byref(prm), _ptr(ws_out),
                                 _ptr(stats_out), _ptr(scratch), int(scratch_nbytes),
                                 int(max_total_tokens), _stream(stream))
    _check(st, "gp_boundary_scan")


def boundary_step_static(kv: KV, pages: Pages, req_ids, n_req, sum_s, sum_l, rope_cos, rope_sin, rope_max_pos,
                         pos, prm: Params, max_total_tokens, ws_out, stats_out, decision_out, delta_out,
                         status_out, evicted_out=None, counters_out=None, stream=None):
    st = load().gp_boundary_step_static(ctypes.byref(kv), ctypes.byref(pages), _ptr(req_ids), int(n_req),
                                        _ptr(sum_s), _ptr(sum_l), _ptr(rope_cos), _ptr(rope_sin),
                                        int(rope_max_pos), _ptr(pos), ctypes.byref(prm), int(max_total_tokens),
                                        _ptr(ws_out), _ptr(stats_out), _ptr(decision_out), _ptr(delta_out),
                                        _ptr(status_out), _ptr(evicted_out), _ptr(counters_out),
                                        _stream(stream))
    _check(st, "gp_boundary_step_static")


def scan_logits(kv: KV, n_req, max_total_tokens, scratch, scratch_nbytes, entry, n, logits_out, stream=None):
    st = load().gp_scan_logits(ctypes.byref(kv), int(n_req), int(max_total_tokens), _ptr(scratch),
                               int(scratch_nbytes), int(entry), int(n), _ptr(logits_out), _stream(stream))
    _check(st, "gp_scan_logits")


def decide(ws, req_ids, n_req, L, Hq, P, prm: Params, pages: Pages, decision_out, delta_out,
           status_out, counters_out=None, stream=None):
    st = load().gp_decide(_ptr(ws), _ptr(req_ids), int(n_req), int(L), int(Hq), int(P),
                          ctypes.byref(prm), ctypes.byref(pages), _ptr(decision_out),
                          _ptr(delta_out), _ptr(status_out), _ptr(counters_out), _stream(stream))
    _check(st, "gp_decide")


def decide_policy(ws, req_ids, n_req, L, Hq, P, prm: Params, policy: str, rand_u, grow_prob,
                  pages: Pages, decision_out, delta_out, status_out, counters_out=None, stream=None):
    st = load().gp_decide_policy(_ptr(ws), _ptr(req_ids), int(n_req), int(L), int(Hq), int(P),
                                 ctypes.byref(prm), POLICIES[policy], _ptr(rand_u), float(grow_prob),
                                 ctypes.byref(pages), _ptr(decision_out), _ptr(delta_out),
                                 _ptr(status_out), _ptr(counters_out), _stream(stream))
    _check(st, "gp_decide_policy")


def compact(kv: KV, pages: Pages, req_ids, decision, n_req, prm: Params, evicted_out, status_out,
            counters_out, scratch, scratch_nbytes, max_total_tokens, stream=None):
    st = load().gp_compact(ctypes.byref(kv), ctypes.byref(pages), _ptr(req_ids), _ptr(decision),
                           int(n_req), ctypes.byref(prm), _ptr(evicted_out), _ptr(status_out),
                           _ptr(counters_out), _ptr(scratch), int(scratch_nbytes),
                           int(max_total_tokens), _stream(stream))
    _check(st, "gp_compact")


def compact_prepare(kv: KV, pages: Pages, req_ids, decision, n_req, prm: Params, evicted_out,
                    status_out, scratch, scratch_nbytes, max_total_tokens, stream=None):
    st = load().gp_compact_prepare(ctypes.byref(kv), ctypes.byref(pages), _ptr(req_ids),
                                   _ptr(decision), int(n_req), ctypes.byref(prm), _ptr(evicted_out),
                                   _ptr(status_out), _ptr(scratch), int(scratch_nbytes),
                                   int(max_total_tokens), _stream(stream))
    _check(st, "gp_compact_prepare")


def compact_move(kv: KV, pages: Pages, req_ids, n_req, counters_out, scratch, scratch_nbytes,
                 max_total_tokens, stream=None):
    st = load().gp_compact_move(ctypes.byref(kv), ctypes.byref(pages), _ptr(req_ids), int(n_req),
                                _ptr(counters_out), _ptr(scratch), int(scratch_nbytes),
                                int(max_total_tokens), _stream(stream))
    _check(st, "gp_compact_move")


def append_kv(kv: KV, pages: Pages, k_new, v_new, req_ids, n_req, status_out=None, stream=None):
    st = load().gp_append_kv(ctypes.byref(kv), ctypes.byref(pages), _ptr(k_new), _ptr(v_new),
                             _ptr(req_ids), int(n_req), _ptr(status_out), _stream(stream))
    _check(st, "gp_append_kv")


def decode_attention(kv: KV, pages: Pages, q, q_dtype, q_strides, req_ids, n_req, rope_cos, rope_sin,
                     rope_max_pos, pos, out, stream=None):
    st = load().gp_decode_attention(ctypes.byref(kv), ctypes.byref(pages), _ptr(q), int(q_dtype),
                                    *[int(x) for x in q_strides], _ptr(req_ids), int(n_req), _ptr(rope_cos),
                                    _ptr(rope_sin), int(rope_max_pos), _ptr(pos), _ptr(out), _stream(stream))
    _check(st, "gp_decode_attention")

"""Oracle: plain, slow CPU reference of the MoE decode layer (ctypes wrapper).

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
CPU-baseline leg of bench.py, never by the product path. It shares no code
with the HIP library. The arithmetic lives in moe_oracle.c (built by
oracle/build.py); this wrapper only moves numpy arrays in and out.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")

_lib = None


class OCfg(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_routed", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32), ("gate_temp", ctypes.c_float),
                ("route_scale", ctypes.c_float), ("swiglu_limit", ctypes.c_float), ("score_mode", ctypes.c_int32)]


def cfg_of(shape) -> OCfg:
    return OCfg(shape.dim, shape.inter, shape.n_routed, shape.topk, int(shape.norm_topk_prob),
                shape.gate_temp, shape.route_scale, shape.swiglu_limit, int(shape.score_mode))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = ctypes.CDLL(LIB_PATH)
        _lib.oracle_score.restype = ctypes.c_float
        _lib.oracle_score.argtypes = [ctypes.c_float, ctypes.c_float]
        _lib.oracle_exp_cr.restype = ctypes.c_float
        _lib.oracle_exp_cr.argtypes = [ctypes.c_float]
        _lib.oracle_log1p_cr.restype = ctypes.c_float
        _lib.oracle_log1p_cr.argtypes = [ctypes.c_float]
        _lib.oracle_swiglu.restype = ctypes.c_float
        _lib.oracle_swiglu.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_float]
        _lib.oracle_f32_to_fp16.restype = ctypes.c_uint16
        _lib.oracle_f32_to_fp16.argtypes = [ctypes.c_float]
        _lib.oracle_num_threads.restype = ctypes.c_int
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "arrays passed to the oracle must be contiguous"
    return ctypes.c_void_p(a.ctypes.data)


def _i64(n: int):
    return ctypes.c_int64(int(n))


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- formats
def bf16_to_f32(b) -> np.ndarray:
    b = _c(b, np.uint16)
    out = np.empty(b.shape, np.float32)
    lib().oracle_bf16_to_f32_n(_p(b), _i64(b.size), _p(out))
    return out


def f32_to_bf16(a) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_f32_to_bf16_n(_p(a), _i64(a.size), _p(out))
    return out


def f32_to_fp16(a) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.uint16)
    lib().oracle_f32_to_fp16_n(_p(a), _i64(a.size), _p(out))
    return out


def fp16_to_f64(h) -> np.ndarray:
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float64)
    lib().oracle_fp16_to_f64_n(_p(h), _i64(h.size), _p(out))
    return out


# ------------------------------------------------------- elementary maths
def exp_cr(a) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.float32)
    lib().oracle_exp_cr_n(_p(a), _i64(a.size), _p(out))
    return out


def log1p_cr(a) -> np.ndarray:
    a = _c(a, np.float32)
    out = np.empty(a.shape, np.float32)
    lib().oracle_log1p_cr_n(_p(a), _i64(a.size), _p(out))
    return out


def scores(logits, temp: float) -> np.ndarray:
    a = _c(logits, np.float32)
    out = np.empty(a.shape, np.float32)
    lib().oracle_scores_par(_p(a), _i64(a.size), ctypes.c_float(temp), _p(out))
    return out


def scores_glibc(logits, temp: float) -> np.ndarray:
    """The glibc mode's scores: the host C library's f32 expf / log1pf / sqrtf chain."""
    a = _c(logits, np.float32)
    out = np.empty(a.shape, np.float32)
    lib().oracle_scores_glibc(_p(a), _i64(a.size), ctypes.c_float(temp), _p(out))
    return out


def swiglu(g, u, limit: float) -> np.ndarray:
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    assert g.shape == u.shape
    out = np.empty(g.shape, np.float32)
    lib().oracle_swiglu_n(_p(g), _p(u), _i64(g.size), ctypes.c_float(limit), _p(out))
    return out


# ------------------------------------------------------------- K-quants
def q2k_dequant(blocks) -> np.ndarray:
    b = _c(blocks, np.uint8).reshape(-1)
    assert b.size % 84 == 0
    out = np.empty(b.size // 84 * 256, np.float64)
    lib().oracle_q2k_dequant(_p(b), _i64(b.size // 84), _p(out))
    return out


def q3k_dequant(blocks) -> np.ndarray:
    b = _c(blocks, np.uint8).reshape(-1)
    assert b.size % 110 == 0
    out = np.empty(b.size // 110 * 256, np.float64)
    lib().oracle_q3k_dequant(_p(b), _i64(b.size // 110), _p(out))
    return out


def q8_1(x):
    """q8_1 of a float32 vector (length a multiple of 32): (int8 codes, fp16 scale bits)."""
    x = _c(x, np.float32).reshape(-1)
    q = np.empty(x.size, np.int8)
    d = np.empty(x.size // 32, np.uint16)
    lib().oracle_q8_1(_p(x), _i64(x.size), _p(q), _p(d))
    return q, d


def q2k_gemv(w, rows: int, cols: int, act, d16):
    w = _c(w, np.uint8)
    act = _c(act, np.int8)
    d16 = _c(d16, np.uint16)
    assert w.size == rows * (cols // 256) * 84 and act.size == cols and d16.size == cols // 32
    y = np.empty(rows, np.float32)
    near = np.empty(rows, np.uint8)
    lib().oracle_q2k_gemv(_p(w), _i64(rows), _i64(cols), _p(act), _p(d16), _p(y), _p(near))
    return y, near


def q3k_gemv(w, rows: int, cols: int, act, d16):
    w = _c(w, np.uint8)
    act = _c(act, np.int8)
    d16 = _c(d16, np.uint16)
    assert w.size == rows * (cols // 256) * 110 and act.size == cols and d16.size == cols // 32
    y = np.empty(rows, np.float32)
    near = np.empty(rows, np.uint8)
    lib().oracle_q3k_gemv(_p(w), _i64(rows), _i64(cols), _p(act), _p(d16), _p(y), _p(near))
    return y, near


# --------------------------------------------------------------- routing
def router_logits(x_bf16, gate_w_bf16) -> np.ndarray:
    x = _c(x_bf16, np.uint16)
    w = _c(gate_w_bf16, np.uint16)
    m, dim = x.shape
    n = w.shape[0]
    assert w.shape[1] == dim
    out = np.empty((m, n), np.float32)
    lib().oracle_router_logits(_p(x), _i64(m), _p(w), _i64(n), _i64(dim), _p(out))
    return out


def select(shape, logits, bias):
    """Header words [m, 1+3*topk] and the scores [m, n_routed]."""
    lg = _c(logits, np.float32)
    b = _c(bias, np.float32)
    m = lg.shape[0]
    c = cfg_of(shape)
    hdr = np.empty((m, 1 + 3 * shape.topk), np.int32)
    sc = np.empty(lg.shape, np.float32)
    lib().oracle_select(ctypes.byref(c), _p(lg), _i64(m), _p(b), _p(hdr), _p(sc))
    return hdr, sc


def header_fields(hdr: np.ndarray, topk: int):
    """(status, picks, weight floats, plan ids) out of header rows."""
    hdr = np.asarray(hdr, np.int32).reshape(-1, 1 + 3 * topk)
    status = hdr[:, 0]
    picks = hdr[:, 1:1 + topk]
    wts = np.ascontiguousarray(hdr[:, 1 + topk:1 + 2 * topk]).view(np.float32)
    plan = hdr[:, 1 + 2 * topk:1 + 3 * topk]
    return status, picks, wts, plan


# ---------------------------------------------------------------- experts
def expert(shape, xq, xd16, gate_blocks, up_blocks, down_blocks) -> dict:
    c = cfg_of(shape)
    dim, inter = shape.dim, shape.inter
    out = {k: np.empty(inter, np.float32) for k in ("g", "u", "h")}
    out["hq"] = np.empty(inter, np.int8)
    out["hd16"] = np.empty(inter // 32, np.uint16)
    out["y"] = np.empty(dim, np.float32)
    for k, n in (("near_g", inter), ("near_u", inter), ("near_y", dim)):
        out[k] = np.empty(n, np.uint8)
    xq = _c(xq, np.int8)
    xd16 = _c(xd16, np.uint16)
    gb, ub, db = (_c(a, np.uint8) for a in (gate_blocks, up_blocks, down_blocks))
    assert gb.size == shape.gate_bytes and ub.size == shape.gate_bytes and db.size == shape.down_bytes
    lib().oracle_expert(ctypes.byref(c), _p(xq), _p(xd16), _p(gb), _p(ub), _p(db), _p(out["g"]), _p(out["u"]),
                        _p(out["h"]), _p(out["hq"]), _p(out["hd16"]), _p(out["y"]), _p(out["near_g"]),
                        _p(out["near_u"]), _p(out["near_y"]))
    return out


def shared(shape, x_bf16, w1, w3, w2) -> dict:
    c = cfg_of(shape)
    x = _c(x_bf16, np.uint16).reshape(-1)
    w1, w3, w2 = (_c(a, np.uint16) for a in (w1, w3, w2))
    out = {"sg": np.empty(shape.inter, np.float32), "su": np.empty(shape.inter, np.float32),
           "sh": np.empty(shape.inter, np.uint16), "sd": np.empty(shape.dim, np.float32)}
    lib().oracle_shared(ctypes.byref(c), _p(x), _p(w1), _p(w3), _p(w2), _p(out["sg"]), _p(out["su"]),
                        _p(out["sh"]), _p(out["sd"]))
    return out


def combine(ys, w, sd=None):
    ys = _c(ys, np.float32)
    w = _c(w, np.float32)
    k, dim = ys.shape
    out = np.empty(dim, np.float32)
    ob = np.empty(dim, np.uint16)
    sdp = None
    if sd is not None:
        sd = _c(sd, np.float32)
        sdp = _p(sd)
    lib().oracle_combine(_i64(dim), _i64(k), _p(ys), _p(w), sdp, _p(out), _p(ob))
    return out, ob


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(ctypes.c_int(int(n)))


# ------------------------------------------- the entry points, on host memory
class OExperts(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("stride", ctypes.c_uint64), ("gate_off", ctypes.c_uint64),
                ("up_off", ctypes.c_uint64), ("down_off", ctypes.c_uint64)]


class OLayer(ctypes.Structure):
    _fields_ = [("gate_w", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("experts", OExperts),
                ("sh_w1", ctypes.c_void_p), ("sh_w3", ctypes.c_void_p), ("sh_w2", ctypes.c_void_p),
                ("shared_kind", ctypes.c_int32), ("shared_q", OExperts)]


def _rc(code: int, name: str):
    if code != 0:
        raise ValueError(f"{name}: invalid arguments ({code})")


def ref_route_select(shape, x, gate_w, bias):
    """moe_ref_route_select: (logits [m, n_routed], header [m, 1+3k])."""
    x = _c(x, np.uint16)
    m = x.shape[0]
    logits = np.empty((m, shape.n_routed), np.float32)
    hdr = np.empty((m, 1 + 3 * shape.topk), np.int32)
    c = cfg_of(shape)
    _rc(lib().moe_ref_route_select(ctypes.byref(c), _p(x), ctypes.c_int32(m), _p(_c(gate_w, np.uint16)),
                                   _p(_c(bias, np.float32)), _p(logits), _p(hdr)), "moe_ref_route_select")
    return logits, hdr


def ref_experts(shape, x, header, arena, stride, gate_off, up_off, down_off, prefill=False):
    """moe_ref_experts_decode / _prefill on a host arena (uint8, expert e at e * stride)."""
    x = _c(x, np.uint16)
    m = x.shape[0]
    hdr = _c(header, np.int32)
    arena = _c(arena, np.uint8)
    ex = OExperts(arena.ctypes.data, stride, gate_off, up_off, down_off)
    y = np.empty((m, shape.dim), np.float32)
    c = cfg_of(shape)
    f = lib().moe_ref_experts_prefill if prefill else lib().moe_ref_experts_decode
    _rc(f(ctypes.byref(c), _p(x), ctypes.c_int32(m), _p(hdr), ctypes.byref(ex), _p(y)), "moe_ref_experts")
    return y


def ref_layer_forward(shape, x, gate_w, bias, arena, stride, gate_off, up_off, down_off, shared_bf16=None,
                      shared_q=None):
    """moe_ref_layer_forward: (out_bf16, out_f32, header). shared_bf16 = (w1, w3, w2), or shared_q = one
    expert's raw blocks (gate | up | down at the arena's offsets)."""
    x = _c(x, np.uint16)
    m = x.shape[0]
    keep = [_c(gate_w, np.uint16), _c(bias, np.float32), _c(arena, np.uint8)]
    ex = OExperts(keep[2].ctypes.data, stride, gate_off, up_off, down_off)
    if shared_q is not None:
        sq = _c(shared_q, np.uint8)
        keep.append(sq)
        layer = OLayer(keep[0].ctypes.data, keep[1].ctypes.data, ex, None, None, None, 1,
                       OExperts(sq.ctypes.data, 0, gate_off, up_off, down_off))
    else:
        w = [_c(a, np.uint16) for a in shared_bf16]
        keep += w
        layer = OLayer(keep[0].ctypes.data, keep[1].ctypes.data, ex, w[0].ctypes.data, w[1].ctypes.data,
                       w[2].ctypes.data, 0, OExperts())
    ob = np.empty((m, shape.dim), np.uint16)
    of = np.empty((m, shape.dim), np.float32)
    hdr = np.empty((m, 1 + 3 * shape.topk), np.int32)
    c = cfg_of(shape)
    _rc(lib().moe_ref_layer_forward(ctypes.byref(c), ctypes.byref(layer), _p(x), ctypes.c_int32(m), _p(ob), _p(of),
                                    _p(hdr)), "moe_ref_layer_forward")
    return ob, of, hdr

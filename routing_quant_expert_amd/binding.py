"""ctypes binding of libmoe.so (include/moe.h). Argument marshalling only:
device tensors are passed as raw pointers with the caller's current HIP
stream; every computation runs in the library's kernels. There is no
fallback: if the library is missing the import of a call fails loudly."""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_STATUS_MISS = 1
MOE_STATUS_NAN_KEY = 2
MOE_STATUS_BAD_PICK = 4
MOE_K_GATEUP, MOE_K_DOWN, MOE_K_ROUTER, MOE_K_SHARED_GU, MOE_K_SHARED_DOWN, MOE_K_GATEUP2, MOE_K_DOWN2 = (
    1, 2, 3, 4, 5, 6, 7)
MOE_K_READ_PROBE = 8


class MoeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libmoe error {code}: {msg}")
        self.code = code


class Cfg(ctypes.Structure):
    _fields_ = [("dim", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_routed", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("norm_topk_prob", ctypes.c_int32), ("gate_temp", ctypes.c_float),
                ("route_scale", ctypes.c_float), ("swiglu_limit", ctypes.c_float), ("score_mode", ctypes.c_int32)]


class Experts(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("stride", ctypes.c_uint64), ("gate_off", ctypes.c_uint64),
                ("up_off", ctypes.c_uint64), ("down_off", ctypes.c_uint64)]


class Layer(ctypes.Structure):
    _fields_ = [("gate_w", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("experts", Experts),
                ("sh_w1", ctypes.c_void_p), ("sh_w3", ctypes.c_void_p), ("sh_w2", ctypes.c_void_p),
                ("shared_kind", ctypes.c_int32), ("shared_q", Experts)]


MOE_SHARED_BF16, MOE_SHARED_KQUANT = 0, 1


class CacheStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("hits", "misses", "prefetched", "prefetch_used", "bytes_copied",
                                               "reads_back")]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("total", "xq", "xd", "xs", "logits", "scores", "plan", "g", "u",
                                                 "h", "hq", "hd", "hs", "y", "sg", "su", "sh", "sd", "yr",
                                                 "status", "ctl", "grp", "xd64", "hd64")] + [("max_pairs", ctypes.c_int32),
                                                               ("plan_words", ctypes.c_int32)]


_lib = None
_VP = ctypes.c_void_p


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build() (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_header_words.restype = ctypes.c_int32
        L.moe_header_words.argtypes = [ctypes.POINTER(Cfg)]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_workspace_bytes.argtypes = [ctypes.POINTER(Cfg), ctypes.c_int32]
        L.moe_workspace_layout.argtypes = [ctypes.POINTER(Cfg), ctypes.c_int32, ctypes.POINTER(WsLayout)]
        L.moe_workspace_init.argtypes = [ctypes.POINTER(Cfg), ctypes.c_int32, _VP, ctypes.c_size_t, _VP]
        L.moe_route_select.argtypes = [ctypes.POINTER(Cfg), _VP, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP,
                                       ctypes.c_size_t, _VP]
        L.moe_experts_decode.argtypes = [ctypes.POINTER(Cfg), _VP, ctypes.c_int32, _VP, ctypes.POINTER(Experts),
                                         _VP, _VP, ctypes.c_size_t, _VP]
        L.moe_experts_prefill.argtypes = [ctypes.POINTER(Cfg), _VP, ctypes.c_int32, _VP, ctypes.POINTER(Experts),
                                          _VP, _VP, ctypes.c_size_t, _VP]
        L.moe_layer_forward.argtypes = [ctypes.POINTER(Cfg), ctypes.POINTER(Layer), _VP, ctypes.c_int32, _VP, _VP,
                                        _VP, _VP, ctypes.c_size_t, _VP]
        L.moe_layer_forward_noalloc.argtypes = [ctypes.POINTER(Cfg), ctypes.POINTER(Layer), _VP, ctypes.c_int32,
                                                _VP, _VP, _VP, _VP]
        L.moe_stack_forward.argtypes = [ctypes.POINTER(Cfg), ctypes.POINTER(Layer), ctypes.c_int32, _VP,
                                         ctypes.c_int32, _VP, _VP, _VP, ctypes.c_size_t, _VP]
        L.moe_scores.argtypes = [_VP, ctypes.c_int64, ctypes.c_float, _VP, ctypes.c_int32, _VP]
        L.moe_scores_host.argtypes = [_VP, ctypes.c_int64, ctypes.c_float, _VP, ctypes.c_int32]
        L.moe_swiglu_host.argtypes = [_VP, _VP, ctypes.c_int64, ctypes.c_float, _VP]
        L.moe_time_next_launch.argtypes = [ctypes.c_int32, _VP, _VP]
        L.moe_read_probe.argtypes = [_VP, ctypes.c_uint64, _VP, ctypes.c_int32, _VP]
        L.moe_glibc_score_table.argtypes = [_VP, _VP, _VP, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
        L.moe_set_score_table.argtypes = [_VP, _VP, _VP, ctypes.c_int64]
        L.moe_cache_create.argtypes = [ctypes.POINTER(Cfg), ctypes.c_int32, ctypes.POINTER(_VP), ctypes.c_uint64,
                                       ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.POINTER(_VP)]
        L.moe_cache_destroy.argtypes = [_VP]
        L.moe_cache_forward.argtypes = [_VP, ctypes.POINTER(Cfg), ctypes.POINTER(Layer), ctypes.c_int32, ctypes.c_int32,
                                        _VP, ctypes.c_int32, _VP, _VP, ctypes.c_int32, _VP, ctypes.c_size_t, _VP]
        L.moe_cache_prefetch.argtypes = [_VP, ctypes.c_int32, _VP, ctypes.c_int32, _VP]
        L.moe_cache_get_stats.argtypes = [_VP, ctypes.POINTER(CacheStats)]
        L.moe_cache_resident.argtypes = [_VP, ctypes.c_int32, _VP]
        L.moe_lru_simulate.argtypes = [ctypes.c_int32, ctypes.c_int64, _VP, _VP, ctypes.c_int32, _VP, _VP]
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(code: int):
    if code != 0:
        raise MoeError(code, lib().moe_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)


def cfg_from_shape(shape) -> Cfg:
    return Cfg(shape.dim, shape.inter, shape.n_routed, shape.topk, int(shape.norm_topk_prob), shape.gate_temp,
               shape.route_scale, shape.swiglu_limit, int(shape.score_mode))


def header_words(cfg: Cfg) -> int:
    return int(lib().moe_header_words(ctypes.byref(cfg)))


def workspace_bytes(cfg: Cfg, max_m: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(cfg), max_m))


def workspace_layout(cfg: Cfg, max_m: int) -> dict:
    L = WsLayout()
    _check(lib().moe_workspace_layout(ctypes.byref(cfg), max_m, ctypes.byref(L)))
    return {n: getattr(L, n) for n, _ in WsLayout._fields_}


def workspace_init(cfg: Cfg, max_m: int, ws, stream=None):
    _check(lib().moe_workspace_init(ctypes.byref(cfg), max_m, _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))


def route_select(cfg: Cfg, x, gate_w, bias, header, ws, logits=None, stream=None):
    m = x.shape[0]
    _check(lib().moe_route_select(ctypes.byref(cfg), _ptr(x), m, _ptr(gate_w), _ptr(bias), _ptr(logits),
                                  _ptr(header), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def experts_decode(cfg: Cfg, x, header, experts: Experts, y_routed, ws, stream=None):
    m = x.shape[0]
    _check(lib().moe_experts_decode(ctypes.byref(cfg), _ptr(x), m, _ptr(header), ctypes.byref(experts),
                                    _ptr(y_routed), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def experts_prefill(cfg: Cfg, x, header, experts: Experts, y_routed, ws, stream=None):
    m = x.shape[0]
    _check(lib().moe_experts_prefill(ctypes.byref(cfg), _ptr(x), m, _ptr(header), ctypes.byref(experts),
                                     _ptr(y_routed), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def layer_forward(cfg: Cfg, layer: Layer, x, out_bf16, ws, out_f32=None, header=None, stream=None):
    m = x.shape[0]
    _check(lib().moe_layer_forward(ctypes.byref(cfg), ctypes.byref(layer), _ptr(x), m, _ptr(out_bf16),
                                   _ptr(out_f32), _ptr(header), _ptr(ws), ws.numel() * ws.element_size(),
                                   _stream(stream)))


def layer_forward_noalloc(cfg: Cfg, layer: Layer, x, out_bf16, out_f32=None, header=None, stream=None):
    """The layer for m <= 8 tokens on the library's fixed scratch (no workspace argument)."""
    m = x.shape[0]
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(cfg), ctypes.byref(layer), _ptr(x), m, _ptr(out_bf16),
                                           _ptr(out_f32), _ptr(header), _stream(stream)))


def stack_forward(cfg: Cfg, layers, xs, ws, out_f32=None, headers=None, stream=None):
    """xs: bf16 [n_layers+1, m, dim] (xs[0] the input); layers: a sequence of Layer."""
    n = len(layers)
    arr = (Layer * n)(*layers)
    m = xs.shape[1]
    _check(lib().moe_stack_forward(ctypes.byref(cfg), arr, n, _ptr(xs), m, _ptr(out_f32), _ptr(headers), _ptr(ws),
                                   ws.numel() * ws.element_size(), _stream(stream)))


def scores(logits, temp: float, out, flags: int = 0, stream=None):
    _check(lib().moe_scores(_ptr(logits), logits.numel(), ctypes.c_float(temp), _ptr(out), flags, _stream(stream)))


def scores_host(logits: np.ndarray, temp: float, flags: int = 0) -> np.ndarray:
    a = np.ascontiguousarray(logits, np.float32)
    out = np.empty_like(a)
    _check(lib().moe_scores_host(a.ctypes.data, a.size, ctypes.c_float(temp), out.ctypes.data, flags))
    return out


# flag bits of scores / scores_host
SCORES_EXTENDED = 1   # every exp/log1p through the extended-precision path
SCORES_GLIBC = 2      # the glibc mode's scores
SCORES_EXP_ONLY = 4   # the chain's exp step alone

MOE_SCORE_CR = 0
MOE_SCORE_GLIBC = 1
SCORE_INDEX_LEN = (1 << 24) + 1


def glibc_score_table():
    """(keys, vals, index) of the glibc score mode, as uint32 numpy arrays."""
    n = ctypes.c_int64(0)
    _check(lib().moe_glibc_score_table(None, None, None, 0, ctypes.byref(n)))
    keys = np.empty(n.value, np.uint32)
    vals = np.empty(n.value, np.uint32)
    index = np.empty(SCORE_INDEX_LEN, np.uint32)
    _check(lib().moe_glibc_score_table(keys.ctypes.data, vals.ctypes.data, index.ctypes.data, n.value,
                                       ctypes.byref(n)))
    return keys, vals, index


_score_tables = {}


def enable_glibc_scores(device=None):
    """Uploads the glibc score table to `device` (default: the current one) and
    registers it there; the tensors stay referenced here for the process."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else device)
    if dev.index in _score_tables:
        return
    keys, vals, index = glibc_score_table()
    with torch.cuda.device(dev):
        # (a host whose libm agrees everywhere still registers a non-NULL, empty table)
        t = [torch.from_numpy(a.view(np.int32) if a.size else np.zeros(1, np.int32)).to(dev)
             for a in (keys, vals, index)]
        torch.cuda.synchronize(dev)
        _check(lib().moe_set_score_table(t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), keys.size))
    _score_tables[dev.index] = t


def swiglu_host(g: np.ndarray, u: np.ndarray, limit: float) -> np.ndarray:
    g = np.ascontiguousarray(g, np.float32)
    u = np.ascontiguousarray(u, np.float32)
    out = np.empty_like(g)
    _check(lib().moe_swiglu_host(g.ctypes.data, u.ctypes.data, g.size, ctypes.c_float(limit), out.ctypes.data))
    return out


def time_next_launch(which: int, ev_begin, ev_end):
    """Bracket the next launch of kernel `which` with two torch.cuda.Event objects."""
    b = None if ev_begin is None else ctypes.c_void_p(ev_begin.cuda_event)
    e = None if ev_end is None else ctypes.c_void_p(ev_end.cuda_event)
    _check(lib().moe_time_next_launch(which, b, e))


def read_probe(buf, nbytes: int, sink, blocks: int, stream=None):
    """Stream `nbytes` of the device tensor `buf` through the library's read-only probe kernel."""
    _check(lib().moe_read_probe(_ptr(buf), nbytes, _ptr(sink), blocks, _stream(stream)))


class ExpertCache:
    """An expert cache (moe_cache_*): n_slots device slots over the host-resident
    experts of len(host_arenas) layers (host tensors or addresses)."""

    def __init__(self, cfg: Cfg, host_arenas, stride: int, gate_off: int, up_off: int, down_off: int, n_slots: int,
                 max_m: int):
        ptrs = [a if isinstance(a, int) else a.data_ptr() for a in host_arenas]
        arr = (_VP * len(ptrs))(*ptrs)
        h = _VP()
        _check(lib().moe_cache_create(ctypes.byref(cfg), len(ptrs), arr, stride, gate_off, up_off, down_off, n_slots,
                                      max_m, ctypes.byref(h)))
        self.h, self.cfg = h, cfg

    def forward(self, layers, xs, ws, first_layer: int = 0, out_f32=None, headers=None, prefetch_k: int = 0,
                stream=None):
        """xs: bf16 [n_layers+1, m, dim] (xs[0] the input); layers: the cache's layers first_layer.. (Layer)."""
        n = len(layers)
        arr = (Layer * n)(*layers)
        _check(lib().moe_cache_forward(self.h, ctypes.byref(self.cfg), arr, first_layer, n, _ptr(xs), xs.shape[1],
                                       _ptr(out_f32), _ptr(headers), prefetch_k, _ptr(ws),
                                       ws.numel() * ws.element_size(), _stream(stream)))

    def prefetch(self, layer: int, experts, stream=None):
        a = np.ascontiguousarray(experts, np.int32)
        _check(lib().moe_cache_prefetch(self.h, layer, a.ctypes.data, a.size, _stream(stream)))

    def stats(self) -> dict:
        st = CacheStats()
        _check(lib().moe_cache_get_stats(self.h, ctypes.byref(st)))
        return {n: getattr(st, n) for n, _ in CacheStats._fields_}

    def resident(self, layer: int) -> np.ndarray:
        out = np.empty(self.cfg.n_routed, np.int32)
        _check(lib().moe_cache_resident(self.h, layer, out.ctypes.data))
        return out

    def close(self):
        if self.h:
            lib().moe_cache_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def lru_simulate(n_slots: int, n_keys: int, batches):
    """The cache's slot assignment on the host: each batch a list of keys; returns (slots, misses) per request."""
    keys = np.ascontiguousarray(np.concatenate([np.asarray(b, np.int64) for b in batches]) if batches else
                                np.zeros(0, np.int64))
    lens = np.ascontiguousarray([len(b) for b in batches], np.int32)
    slots = np.empty(keys.size, np.int32)
    miss = np.empty(keys.size, np.int32)
    _check(lib().moe_lru_simulate(n_slots, n_keys, keys.ctypes.data, lens.ctypes.data, len(batches),
                                  slots.ctypes.data, miss.ctypes.data))
    return slots, miss

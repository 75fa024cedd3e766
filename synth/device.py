"""Device-side generation of the synthetic inputs into torch tensors, with
libsynth.so (the HIP twin of the numpy recipes in synth/__init__.py)."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import (K_EXP_DOWN, K_EXP_GATE, K_EXP_UP, K_GATE_W, K_SH_W1, K_SH_W2, K_SH_W3, K_X, Q2K_BYTES, Q3K_BYTES,
               SIGMA_W, SIGMA_X, LayerSpec, bias, gate_w, make_tag, shared_w, tokens)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsynth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        vp, u64 = ctypes.c_void_p, ctypes.c_uint64
        L.synth_q2k_blocks.argtypes = [vp, u64, u64, u64, u64, vp]
        L.synth_q3k_blocks.argtypes = [vp, u64, u64, u64, u64, vp]
        L.synth_normal_bf16.argtypes = [vp, u64, u64, u64, u64, ctypes.c_double, vp]
        L.synth_uniform_f32.argtypes = [vp, u64, u64, u64, u64, ctypes.c_double, ctypes.c_double, vp]
        _lib = L
    return _lib


def _stream():
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ok(rc: int):
    if rc != 0:
        raise RuntimeError(f"libsynth call failed with {rc}")


def fill_arena(spec: LayerSpec, arena, experts=None):
    """Fill a uint8 device tensor of n_routed*stride bytes with every expert's
    blocks (or only the listed experts)."""
    s = spec.shape
    assert arena.numel() >= s.n_routed * s.expert_stride and arena.data_ptr() % 16 == 0
    base = arena.data_ptr()
    st = _stream()
    nq2 = s.inter * s.nsb_gate
    nq3 = s.dim * s.nsb_down
    for e in (range(s.n_routed) if experts is None else experts):
        p = base + e * s.expert_stride
        _ok(lib().synth_q2k_blocks(p + s.gate_off, spec.seed, spec.tag(K_EXP_GATE, e), 0, nq2, st))
        _ok(lib().synth_q2k_blocks(p + s.up_off, spec.seed, spec.tag(K_EXP_UP, e), 0, nq2, st))
        _ok(lib().synth_q3k_blocks(p + s.down_off, spec.seed, spec.tag(K_EXP_DOWN, e), 0, nq3, st))


def normal_bf16_into(t, seed: int, tag: int, sigma: float, i0: int = 0):
    _ok(lib().synth_normal_bf16(t.data_ptr(), seed, tag, i0, t.numel(), sigma, _stream()))


def tokens_into(spec: LayerSpec, x, t0: int = 0):
    """Input rows t0.. of the token recipe into the device tensor x [m, dim]
    (the same bits as synth.tokens, one seeded stream per row)."""
    for i in range(x.shape[0]):
        normal_bf16_into(x[i], spec.seed, make_tag(K_X, spec.layer, t0 + i), SIGMA_X)


def fill_expert(spec: LayerSpec, buf, e: int):
    """Expert index e's blocks (gate | up | down, one stride) into a uint8
    device tensor; e = n_routed gives the K-quant shared expert."""
    s = spec.shape
    assert buf.numel() >= s.expert_stride and buf.data_ptr() % 16 == 0
    p, st = buf.data_ptr(), _stream()
    _ok(lib().synth_q2k_blocks(p + s.gate_off, spec.seed, spec.tag(K_EXP_GATE, e), 0, s.inter * s.nsb_gate, st))
    _ok(lib().synth_q2k_blocks(p + s.up_off, spec.seed, spec.tag(K_EXP_UP, e), 0, s.inter * s.nsb_gate, st))
    _ok(lib().synth_q3k_blocks(p + s.down_off, spec.seed, spec.tag(K_EXP_DOWN, e), 0, s.dim * s.nsb_down, st))


class DeviceLayer:
    """One synthetic layer resident on the GPU: router, bias, expert arena and
    shared expert (bf16, or K-quant blocks when spec.shared_quant), plus the
    binding structs that point at them."""

    def __init__(self, spec: LayerSpec, device="cuda", arena=None, experts_on_device=True):
        import torch
        from routing_quant_expert_amd import MOE_SHARED_KQUANT, Experts, Layer, cfg_from_shape
        s = spec.shape
        self.spec = spec
        self.cfg = cfg_from_shape(s)
        self.gate_w = torch.empty((s.n_routed, s.dim), dtype=torch.uint16, device=device)
        normal_bf16_into(self.gate_w, spec.seed, spec.tag(K_GATE_W), SIGMA_W)
        self.bias = torch.from_numpy(bias(spec)).to(device)
        if experts_on_device:
            self.arena = arena if arena is not None else torch.empty(s.n_routed * s.expert_stride, dtype=torch.uint8,
                                                                      device=device)
            fill_arena(spec, self.arena)
        else:   # the routed experts live elsewhere (an expert cache): a placeholder arena of one expert
            self.arena = torch.zeros(s.expert_stride, dtype=torch.uint8, device=device)
        self.experts = Experts(self.arena.data_ptr(), s.expert_stride, s.gate_off, s.up_off, s.down_off)
        if spec.shared_quant:
            self.sh_w1 = self.sh_w3 = self.sh_w2 = None
            self.shared_q = torch.empty(s.expert_stride, dtype=torch.uint8, device=device)
            fill_expert(spec, self.shared_q, s.n_routed)
            sq = Experts(self.shared_q.data_ptr(), 0, s.gate_off, s.up_off, s.down_off)
            self.layer = Layer(self.gate_w.data_ptr(), self.bias.data_ptr(), self.experts, None, None, None,
                               MOE_SHARED_KQUANT, sq)
            return
        self.sh_w1 = torch.empty((s.inter, s.dim), dtype=torch.uint16, device=device)
        self.sh_w3 = torch.empty((s.inter, s.dim), dtype=torch.uint16, device=device)
        self.sh_w2 = torch.empty((s.dim, s.inter), dtype=torch.uint16, device=device)
        normal_bf16_into(self.sh_w1, spec.seed, spec.tag(K_SH_W1), SIGMA_W)
        normal_bf16_into(self.sh_w3, spec.seed, spec.tag(K_SH_W3), SIGMA_W)
        normal_bf16_into(self.sh_w2, spec.seed, spec.tag(K_SH_W2), SIGMA_W)
        self.layer = Layer(self.gate_w.data_ptr(), self.bias.data_ptr(), self.experts, self.sh_w1.data_ptr(),
                           self.sh_w3.data_ptr(), self.sh_w2.data_ptr())

    def tokens(self, t0: int, m: int, device="cuda"):
        import torch
        return torch.from_numpy(tokens(self.spec, t0, m)).to(device)


def host_arena(spec: LayerSpec, scratch=None):
    """Every routed expert's raw blocks of the layer in pinned host memory
    (generated on the device into `scratch`, a uint8 device tensor of at least
    n_routed * stride bytes, then copied down)."""
    import torch
    s = spec.shape
    nbytes = s.n_routed * s.expert_stride
    if scratch is None:
        scratch = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    fill_arena(spec, scratch)
    out = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    out.copy_(scratch[:nbytes])
    torch.cuda.synchronize()
    return out

"""CPU checks of the oracle's mirror of the four entry points (moe_ref_*,
host memory): each equals the oracle's own per-token composition bit for bit
(the wiring of the mirror: header, plan-order weights, the shared expert of
either kind, the rejected-pick rule), and rejects NULL arguments."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from oracle import layer as olayer

SH = synth.SHAPE_TINY


def _arena(spec):
    s = spec.shape
    return np.concatenate([synth.expert_bytes(spec, e) for e in range(s.n_routed)])


@pytest.mark.parametrize("shared_quant", [False, True])
def test_ref_layer_forward_equals_composition(shared_quant):
    spec = synth.LayerSpec(SH, seed=71, shared_quant=shared_quant)
    x = synth.tokens(spec, 0, 3)
    arena = _arena(spec)
    kw = dict(shared_q=synth.expert_bytes(spec, SH.n_routed)) if shared_quant else dict(
        shared_bf16=tuple(synth.shared_w(spec, w) for w in ("w1", "w3", "w2")))
    ob, of, hdr = oracle.ref_layer_forward(SH, x, synth.gate_w(spec), synth.bias(spec), arena, SH.expert_stride,
                                           SH.gate_off, SH.up_off, SH.down_off, **kw)
    ref = olayer.layer_forward(spec, x)
    assert np.array_equal(hdr, ref["header"])
    assert np.array_equal(of.view(np.uint32), ref["out_f32"].view(np.uint32))
    assert np.array_equal(ob, ref["out_bf16"])


def test_ref_route_select_and_experts_equal_composition():
    spec = synth.LayerSpec(SH, seed=72)
    x = synth.tokens(spec, 9, 4)
    lg, hdr = oracle.ref_route_select(SH, x, synth.gate_w(spec), synth.bias(spec))
    r = olayer.route(spec, x)
    assert np.array_equal(lg.view(np.uint32), r["logits"].view(np.uint32)) and np.array_equal(hdr, r["header"])
    arena = _arena(spec)
    ref = olayer.layer_forward(spec, x, with_shared=False)
    for prefill in (False, True):
        y = oracle.ref_experts(SH, x, hdr, arena, SH.expert_stride, SH.gate_off, SH.up_off, SH.down_off, prefill)
        assert np.array_equal(y.view(np.uint32), ref["y_routed"].view(np.uint32))
    bad = hdr.copy()
    bad[1, 2] = SH.n_routed     # out of range
    bad[2, 3] = bad[2, 1]       # repeated
    y = oracle.ref_experts(SH, x, bad, arena, SH.expert_stride, SH.gate_off, SH.up_off, SH.down_off)
    assert np.all(y[1] == 0) and np.all(y[2] == 0)
    assert np.array_equal(y[[0, 3]].view(np.uint32), ref["y_routed"][[0, 3]].view(np.uint32))


def test_ref_entry_points_reject_null_arguments():
    c = oracle.cfg_of(SH)
    L = oracle.lib()
    assert L.moe_ref_route_select(ctypes.byref(c), None, 1, None, None, None, None) == -1
    assert L.moe_ref_experts_decode(ctypes.byref(c), None, 1, None, None, None) == -1
    assert L.moe_ref_layer_forward(ctypes.byref(c), None, None, 1, None, None, None) == -1

"""One suite, two implementations: every entry point of the library (device
buffers, through the C ABI) and its mirror in the oracle (moe_ref_*, host
memory) are driven through the same interface with the same inputs, and
their results compared at the parity bar: logits and headers bit for bit,
routed and layer outputs within rel-L2 1e-3 and max-abs 1e-2 [device_route.rs,
fn device_route_check: two implementations of the selection checked on the
same logits]."""
import numpy as np
import pytest
import torch

import oracle
import routing_quant_expert_amd as R
import synth
from synth.device import DeviceLayer
from tests.gpu_helpers import rel_l2, say, to_np_u16, workspace

pytestmark = pytest.mark.gpu


class Device:
    """The library's entry points on device copies of host inputs."""
    name = "device"

    def route_select(self, shape, x, gate_w, bias):
        c = R.cfg_from_shape(shape)
        m = x.shape[0]
        xd = torch.from_numpy(x).cuda()
        lg = torch.empty((m, shape.n_routed), dtype=torch.float32, device="cuda")
        hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
        R.route_select(c, xd, torch.from_numpy(gate_w.view(np.int16)).cuda(), torch.from_numpy(bias).cuda(), hdr,
                       workspace(c, m), logits=lg)
        torch.cuda.synchronize()
        return lg.cpu().numpy(), hdr.cpu().numpy()

    def experts(self, shape, x, header, dl, prefill):
        c = R.cfg_from_shape(shape)
        m = x.shape[0]
        y = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
        f = R.experts_prefill if prefill else R.experts_decode
        f(c, torch.from_numpy(x).cuda(), torch.from_numpy(header).cuda(), dl.experts, y, workspace(c, m))
        torch.cuda.synchronize()
        return y.cpu().numpy()

    def layer_forward(self, shape, x, dl):
        c = R.cfg_from_shape(shape)
        m = x.shape[0]
        ob = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
        of = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
        hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
        R.layer_forward(c, dl.layer, torch.from_numpy(x).cuda(), ob, workspace(c, m), out_f32=of, header=hdr)
        torch.cuda.synchronize()
        return to_np_u16(ob), of.cpu().numpy(), hdr.cpu().numpy()


class Ref:
    """The oracle's mirror of the same entry points on host memory."""
    name = "oracle"

    def route_select(self, shape, x, gate_w, bias):
        return oracle.ref_route_select(shape, x, gate_w, bias)

    def experts(self, shape, x, header, dl, prefill):
        s = shape
        return oracle.ref_experts(s, x, header, dl.host_arena, s.expert_stride, s.gate_off, s.up_off, s.down_off,
                                  prefill)

    def layer_forward(self, shape, x, dl):
        s, spec = shape, dl.spec
        kw = (dict(shared_q=dl.shared_q.cpu().numpy()) if spec.shared_quant else
              dict(shared_bf16=tuple(to_np_u16(t) for t in (dl.sh_w1, dl.sh_w3, dl.sh_w2))))
        return oracle.ref_layer_forward(s, x, to_np_u16(dl.gate_w), dl.bias.cpu().numpy(), dl.host_arena,
                                        s.expert_stride, s.gate_off, s.up_off, s.down_off, **kw)


_DL = {}


def layer(shape, shared_quant=False):
    key = (shape, shared_quant)
    if key not in _DL:
        if shape == synth.SHAPE_DS41:
            for k in [k for k in _DL if k[0] == synth.SHAPE_DS41]:
                del _DL[k]
            torch.cuda.empty_cache()
        say(f"generating layer dim {shape.dim} shared_quant={shared_quant}")
        dl = DeviceLayer(synth.LayerSpec(shape, seed=17, shared_quant=shared_quant))
        dl.host_arena = dl.arena.cpu().numpy()       # the same blocks for the host mirror
        _DL[key] = dl
    return _DL[key]


def _close(a, b):
    for t in range(a.shape[0]):
        assert rel_l2(a[t], b[t]) <= 1e-3 and np.abs(a[t] - b[t]).max() <= 1e-2, t


CASES = [(synth.SHAPE_TINY, 1, False), (synth.SHAPE_TINY, 5, False), (synth.SHAPE_TINY, 40, False),
         (synth.SHAPE_TINY, 3, True), (synth.SHAPE_TINY, 24, True), (synth.SHAPE_DS41, 1, False),
         (synth.SHAPE_DS41, 12, True)]


@pytest.mark.parametrize("shape,m,shared_quant", CASES,
                         ids=lambda v: f"dim{v.dim}" if hasattr(v, "dim") else str(v))
def test_entry_points_through_one_interface(shape, m, shared_quant):
    dl = layer(shape, shared_quant)
    x = synth.tokens(dl.spec, 40 * m, m)
    impls = (Device(), Ref())
    say(f"dim {shape.dim} m={m} shared_quant={shared_quant}: route_select")
    rs = [im.route_select(shape, x, to_np_u16(dl.gate_w), dl.bias.cpu().numpy()) for im in impls]
    assert np.array_equal(rs[0][0].view(np.uint32), rs[1][0].view(np.uint32))
    assert np.array_equal(rs[0][1], rs[1][1])
    header = rs[1][1]
    for prefill in ((False, True) if m <= 8 else (True,)):
        say(f"  experts_{'prefill' if prefill else 'decode'}")
        ys = [im.experts(shape, x, header, dl, prefill) for im in impls]
        _close(ys[0], ys[1])
    say("  layer_forward")
    lf = [im.layer_forward(shape, x, dl) for im in impls]
    assert np.array_equal(lf[0][2], lf[1][2])
    _close(lf[0][1], lf[1][1])
    assert np.array_equal(lf[0][0], oracle.f32_to_bf16(lf[0][1]))

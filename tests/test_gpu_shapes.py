"""GPU parity on the other supported widths: dim and inter from 256 to 4096
(the kernels are instantiated per dim/256 and inter/256), through the
decode path (m = 1 and m = 3) and the prefill path (m = 40), every token
checked against the oracle (headers bit-exact, layer output within rel-L2
1e-3 and max-abs 1e-2, the routed GEMV values bit-exact up to the flagged
near-midpoint neighbours)."""
import numpy as np
import pytest
import torch

import oracle
import routing_quant_expert_amd as R
import synth
from oracle import layer as olayer
from synth.device import DeviceLayer
from tests.gpu_helpers import f32_accept, plan_tables, rel_l2, say, workspace, ws_array

pytestmark = pytest.mark.gpu

SHAPES = [synth.Shape(dim=256, inter=256), synth.Shape(dim=1024, inter=512), synth.Shape(dim=2048, inter=1024),
          synth.Shape(dim=512, inter=4096)]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s.dim}x{s.inter}")
def test_layer_forward_other_widths(shape):
    spec = synth.LayerSpec(shape, seed=4, zipf_bias=True)
    say(f"generating layer {shape.dim}x{shape.inter}")
    dl = DeviceLayer(spec)
    c = dl.cfg
    try:
        for m in (1, 3, 40):
            x_np = synth.tokens(spec, 50 * m, m)
            x = torch.from_numpy(x_np).cuda()
            ws = workspace(c, m)
            out = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
            out32 = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
            hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
            say(f"  layer_forward m={m}")
            R.layer_forward(c, dl.layer, x, out, ws, out_f32=out32, header=hdr)
            torch.cuda.synchronize()
            ref = olayer.layer_forward(spec, x_np)
            assert np.array_equal(hdr.cpu().numpy(), ref["header"])
            o = out32.cpu().numpy()
            for t in range(m):
                err = np.abs(o[t] - ref["out_f32"][t])
                assert rel_l2(o[t], ref["out_f32"][t]) <= 1e-3 and err.max() <= 1e-2, (m, t)
            L = R.workspace_layout(c, m)
            tab = plan_tables(ws, L, m, shape.topk)
            P = L["max_pairs"]
            y = ws_array(ws, L, "y", np.float32, P * shape.dim).reshape(P, shape.dim)
            g = ws_array(ws, L, "g", np.float32, P * shape.inter).reshape(P, shape.inter)
            for t in range(m):
                for k, e in enumerate(ref["tok"][t]["ids"]):
                    p = int(tab["tok_pairs"][t][k])
                    ex = ref["tok"][t]["experts"][k]
                    f32_accept(g[p], ex["g"], ex["near_g"], f"g m={m} tok {t} e {e}")
                    f32_accept(y[p], ex["y"], ex["near_y"], f"y m={m} tok {t} e {e}")
    finally:
        del dl
        torch.cuda.empty_cache()


ROUTING = [dict(n_routed=100, topk=1, norm_topk_prob=False), dict(n_routed=100, topk=8, norm_topk_prob=True),
           dict(n_routed=1024, topk=8, norm_topk_prob=False), dict(n_routed=1024, topk=5, norm_topk_prob=True),
           dict(n_routed=64, topk=2, norm_topk_prob=True)]
# the K-quant shared expert at the ends of the topk range: topk 8 gives 9 plan entries per token
ROUTING_KQ = [dict(n_routed=100, topk=8, norm_topk_prob=True), dict(n_routed=1024, topk=1, norm_topk_prob=False)]


@pytest.mark.parametrize("routing,shared_quant", [(r, False) for r in ROUTING] + [(r, True) for r in ROUTING_KQ],
                         ids=lambda v: (f"e{v['n_routed']}_k{v['topk']}_n{int(v['norm_topk_prob'])}"
                                        if isinstance(v, dict) else ("kquant" if v else "bf16")))
def test_layer_forward_other_routing_configs(routing, shared_quant):
    """The rest of the supported routing set at dim 512: n_routed not a
    multiple of 64 and up to 1024 (the 16-key-per-lane selection), topk 1
    and 8 (topk above 6 takes the multi-token kernels at m = 1, with 64 pairs
    at m = 8), unnormalised weights, and the K-quant shared expert at topk 8
    and 1; m = 1, 8 and 40, every token against the oracle."""
    import dataclasses
    shape = dataclasses.replace(synth.SHAPE_TINY, **routing)
    spec = synth.LayerSpec(shape, seed=8, shared_quant=shared_quant)
    say(f"generating layer e{shape.n_routed} k{shape.topk} norm {shape.norm_topk_prob} shared_quant {shared_quant}")
    dl = DeviceLayer(spec)
    c = dl.cfg
    try:
        for m in (1, 8, 40):
            x_np = synth.tokens(spec, 10 * m, m)
            x = torch.from_numpy(x_np).cuda()
            ws = workspace(c, m)
            out = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
            out32 = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
            hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
            say(f"  layer_forward m={m}")
            R.layer_forward(c, dl.layer, x, out, ws, out_f32=out32, header=hdr)
            torch.cuda.synchronize()
            ref = olayer.layer_forward(spec, x_np)
            assert np.array_equal(hdr.cpu().numpy(), ref["header"]), m
            o = out32.cpu().numpy()
            for t in range(m):
                err = np.abs(o[t] - ref["out_f32"][t])
                assert rel_l2(o[t], ref["out_f32"][t]) <= 1e-3 and err.max() <= 1e-2, (m, t)
            L = R.workspace_layout(c, m)
            tab = plan_tables(ws, L, m, shape.topk)
            P = L["max_pairs"]
            y = ws_array(ws, L, "y", np.float32, P * shape.dim).reshape(P, shape.dim)
            for t in range(m):
                for k, e in enumerate(ref["tok"][t]["ids"]):
                    ex = ref["tok"][t]["experts"][k]
                    f32_accept(y[int(tab["tok_pairs"][t][k])], ex["y"], ex["near_y"], f"y m={m} tok {t} e {e}")
            # the routing call alone gives the same headers
            hdr2 = torch.empty_like(hdr)
            R.route_select(c, x, dl.gate_w, dl.bias, hdr2, ws)
            torch.cuda.synchronize()
            assert np.array_equal(hdr2.cpu().numpy(), ref["header"]), m
    finally:
        del dl
        torch.cuda.empty_cache()


def test_route_select_random_configs():
    """The routing call over seeded random configurations (n_routed 6..1024,
    topk 1..8, normalised or not, gate_temp and route_scale away from 1 and
    2.5, dim 256..4096, m 1..80): logits and headers bit for bit against the
    oracle's mirror of the same call."""
    import dataclasses
    rng = np.random.default_rng(2024)
    for case in range(24):
        topk = int(rng.integers(1, 9))
        n_routed = int(rng.integers(max(topk, 6), 1025))
        dim = int(256 * 2 ** rng.integers(0, 5))
        shape = dataclasses.replace(synth.SHAPE_TINY, dim=dim, n_routed=n_routed, topk=topk,
                                    norm_topk_prob=bool(rng.integers(0, 2)),
                                    gate_temp=float(np.float32(rng.uniform(0.3, 3.0))),
                                    route_scale=float(np.float32(rng.uniform(0.5, 4.0))))
        m = int(rng.choice([1, 2, 5, 8, 9, 33, 80]))
        x = oracle.f32_to_bf16(rng.normal(0, 1, (m, dim)).astype(np.float32))
        gw = oracle.f32_to_bf16(rng.normal(0, 0.05, (n_routed, dim)).astype(np.float32))
        bias = rng.uniform(-0.2, 0.2, n_routed).astype(np.float32)
        say(f"case {case}: e{n_routed} k{topk} dim {dim} m {m} temp {shape.gate_temp:.3f}")
        c = R.cfg_from_shape(shape)
        lg = torch.empty((m, n_routed), dtype=torch.float32, device="cuda")
        hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
        R.route_select(c, torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(gw.view(np.int16)).cuda(),
                       torch.from_numpy(bias).cuda(), hdr, workspace(c, m), logits=lg)
        torch.cuda.synchronize()
        rl, rh = oracle.ref_route_select(shape, x, gw, bias)
        assert np.array_equal(lg.cpu().numpy().view(np.uint32), rl.view(np.uint32)), case
        assert np.array_equal(hdr.cpu().numpy(), rh), case


def test_layer_forward_random_configs():
    """Whole layers over seeded random configurations (experts, topk,
    normalisation, temperature, route scale, SwiGLU limit, shared expert kind,
    dim 512 or 1024) at m = 1, 4 and 20 (the single-token, union and prefill
    paths): headers bit for bit and outputs within rel-L2 1e-3 and max-abs
    1e-2 against the oracle."""
    import dataclasses
    rng = np.random.default_rng(77)
    for case in range(6):
        topk = int(rng.integers(1, 9))
        dim, inter = ((512, 256), (1024, 512))[int(rng.integers(0, 2))]
        shape = dataclasses.replace(synth.SHAPE_TINY, dim=dim, inter=inter,
                                    n_routed=int(rng.integers(max(topk, 8), 600)), topk=topk,
                                    norm_topk_prob=bool(rng.integers(0, 2)),
                                    gate_temp=float(np.float32(rng.uniform(0.5, 2.0))),
                                    route_scale=float(np.float32(rng.uniform(0.5, 4.0))),
                                    swiglu_limit=float(np.float32(rng.uniform(0.5, 10.0))))
        shared_quant = bool(rng.integers(0, 2))
        spec = synth.LayerSpec(shape, seed=100 + case, shared_quant=shared_quant)
        say(f"case {case}: {shape} shared_quant={shared_quant}")
        dl = DeviceLayer(spec)
        c = dl.cfg
        try:
            for m in (1, 4, 20):
                x_np = synth.tokens(spec, 7 * m, m)
                ws = workspace(c, m)
                out = torch.empty((m, dim), dtype=torch.uint16, device="cuda")
                out32 = torch.empty((m, dim), dtype=torch.float32, device="cuda")
                hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
                R.layer_forward(c, dl.layer, torch.from_numpy(x_np).cuda(), out, ws, out_f32=out32, header=hdr)
                torch.cuda.synchronize()
                ref = olayer.layer_forward(spec, x_np)
                assert np.array_equal(hdr.cpu().numpy(), ref["header"]), (case, m)
                o = out32.cpu().numpy()
                for t in range(m):
                    err = np.abs(o[t] - ref["out_f32"][t])
                    assert rel_l2(o[t], ref["out_f32"][t]) <= 1e-3 and err.max() <= 1e-2, (case, m, t)
        finally:
            del dl
            torch.cuda.empty_cache()

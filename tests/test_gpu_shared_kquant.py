"""GPU parity of layers whose shared expert is K-quant blocks (Q2_K gate/up,
Q3_K down) [moe_v41.rs, struct MoeV41LayerWeights: the shared matrices as
bf16 or the GGUF's Q2_K (w1, w3) / Q3_K (w2) blocks on the routed experts'
kernels]. The shared expert runs as plan expert n_routed of every token with
weight 1, so every one of its values (g, u, h, q8_1 of h, y) is checked like
a routed pair's, and since no f32 GEMV of unstated order remains, the layer
output is the oracle's bit for bit (up to the flagged near-midpoint GEMV
neighbours). Single-token, multi-token and prefill paths, a layer stack and
the no-allocation entry point."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import routing_quant_expert_amd as R
import synth
from oracle import layer as olayer
from synth.device import DeviceLayer
from tests.gpu_helpers import check_combine_bits, plan_tables, rel_l2, say, to_np_u16, workspace, ws_array
from tests.test_gpu_parity import _check_layer
from tests.test_gpu_prefill import _check_tokens, _ws_views

pytestmark = pytest.mark.gpu

TINY, DS41 = synth.SHAPE_TINY, synth.SHAPE_DS41
_DL = {}


def kq_layer(shape, seed=2, zipf=False):
    key = (shape, seed, zipf)
    if key not in _DL:
        if shape == DS41:
            for k in [k for k in _DL if k[0] == DS41]:
                del _DL[k]
            torch.cuda.empty_cache()
        say(f"generating layer {shape.dim}x{shape.inter} seed {seed} with a K-quant shared expert")
        _DL[key] = DeviceLayer(synth.LayerSpec(shape, seed=seed, zipf_bias=zipf, shared_quant=True))
        torch.cuda.synchronize()
    return _DL[key]


def _run(dl, x_np, noalloc=False):
    c, dim = dl.cfg, dl.spec.shape.dim
    m = x_np.shape[0]
    x = torch.from_numpy(x_np).cuda()
    out = torch.empty((m, dim), dtype=torch.uint16, device="cuda")
    out32 = torch.empty((m, dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
    ws = None
    if noalloc:
        R.layer_forward_noalloc(c, dl.layer, x, out, out_f32=out32, header=hdr)
    else:
        ws = workspace(c, m)
        R.layer_forward(c, dl.layer, x, out, ws, out_f32=out32, header=hdr)
    torch.cuda.synchronize()
    return ws, out32.cpu().numpy(), to_np_u16(out), hdr.cpu().numpy()


@pytest.mark.parametrize("shape,m", [(TINY, 1), (TINY, 2), (TINY, 8), (DS41, 1), (DS41, 3)],
                         ids=lambda v: str(v.dim) if hasattr(v, "dim") else str(v))
def test_kquant_shared_layer_matches_oracle(shape, m):
    dl = kq_layer(shape)
    x_np = synth.tokens(dl.spec, 60, m)
    say(f"K-quant shared layer dim={shape.dim} m={m}")
    ws, o, ob, h = _run(dl, x_np)
    _check_layer(dl, x_np, m, o, ob, h, ws)


def test_kquant_shared_correlated_m8_full_size():
    dl = kq_layer(DS41)
    x_np = synth.correlated_tokens(dl.spec, 8, group=3)
    say("K-quant shared layer dim=4096 correlated m=8")
    ws, o, ob, h = _run(dl, x_np)
    _check_layer(dl, x_np, 8, o, ob, h, ws)


@pytest.mark.parametrize("shape", [TINY, DS41], ids=lambda s: f"dim{s.dim}")
def test_kquant_shared_single_and_multi_token_paths_agree(shape):
    """The same token alone (single-token kernels), twice in an m = 2 call
    (union kernels) and 9 times with 31 others in an m = 40 call (prefill
    kernels): the same header every time; the same output bits from the
    single-token and union kernels (the same float64 summation of the exact
    block sums), and from the prefill kernels (another float64 split of the
    same exact sums, which may round the other way next to an f32 midpoint)
    the output within the tolerance."""
    dl = kq_layer(shape)
    x1 = synth.tokens(dl.spec, 70, 1)
    rest = synth.tokens(dl.spec, 71, 31)
    runs = {1: x1, 2: np.concatenate([x1, x1]), 40: np.concatenate([np.repeat(x1, 9, axis=0), rest])}
    got = {}
    for m, x_np in runs.items():
        say(f"  dim={shape.dim} m={m}")
        _, o, _, h = _run(dl, x_np)
        got[m] = (o, h)
    o1, h1 = got[1]
    for m in (2, 40):
        om, hm = got[m]
        n = 2 if m == 2 else 9
        for t in range(n):
            assert np.array_equal(hm[t], h1[0]), (m, t)
            if m == 2:
                assert np.array_equal(om[t].view(np.uint32), o1[0].view(np.uint32)), (m, t)
            else:
                assert rel_l2(om[t], o1[0]) <= 1e-3 and np.abs(om[t] - o1[0]).max() <= 1e-2, (m, t)


@pytest.mark.parametrize("shape,m,check", [(TINY, 40, None), (DS41, 512, 64)],
                         ids=lambda v: str(v.dim) if hasattr(v, "dim") else str(v))
def test_kquant_shared_prefill(shape, m, check):
    """The prefill path: the K-quant shared expert is one more expert group
    holding every token (after all routed groups); every pair of the checked
    tokens against the oracle, the combine of every token bit for bit."""
    dl = kq_layer(shape, zipf=True)
    spec, c = dl.spec, dl.cfg
    x_np = synth.tokens(spec, 2000, m)
    say(f"K-quant shared prefill dim={shape.dim} m={m}")
    ws, o, ob, h = _run(dl, x_np)
    v = _ws_views(ws, c, m, shape)
    tab = v["tab"]
    assert tab["n_pairs"] == m * (shape.topk + 1)
    nu = tab["n_u"]
    nsh = (m + 15) // 16   # the shared group's plan entries: 16 tokens each (one MFMA pass), after the routed ones
    assert np.all(tab["u_expert"][nu - nsh:nu] == shape.n_routed) and tab["u_expert"][nu - nsh - 1] < shape.n_routed
    assert np.array_equal(tab["u_first"][nu - nsh:nu], m * shape.topk + 16 * np.arange(nsh))
    assert np.array_equal(tab["u_npairs"][nu - nsh:nu], np.minimum(16, m - 16 * np.arange(nsh)))
    assert np.array_equal(tab["pair_tok"][m * shape.topk:m * (shape.topk + 1)], np.arange(m))
    toks = range(m) if check is None else sorted(set(np.linspace(0, m - 1, check).astype(int)))
    _check_tokens(spec, x_np, toks, v, o, "out_f32", h)
    check_combine_bits(ws, v["L"], tab, m, shape.topk, o, False)
    assert np.array_equal(ob, oracle.f32_to_bf16(o))


def test_kquant_shared_stack_and_noalloc():
    """Three small K-quant-shared layers at m = 1 and m = 3 through the
    layer stack (teacher-forced against the oracle), and the no-allocation
    entry point equal to the workspace one on the same layer."""
    n = 3
    specs = [synth.LayerSpec(TINY, seed=12, layer=l, shared_quant=True) for l in range(n)]
    dls = [DeviceLayer(sp) for sp in specs]
    c = dls[0].cfg
    for m in (1, 3):
        say(f"K-quant shared stack of {n} layers m={m}")
        x0 = synth.tokens(specs[0], 5, m)
        xs = torch.empty((n + 1, m, TINY.dim), dtype=torch.uint16, device="cuda")
        xs[0] = torch.from_numpy(x0).cuda()
        out = torch.empty((n, m, TINY.dim), dtype=torch.float32, device="cuda")
        hdr = torch.empty((n, m, R.header_words(c)), dtype=torch.int32, device="cuda")
        R.stack_forward(c, [d.layer for d in dls], xs, workspace(c, m), out_f32=out, headers=hdr)
        torch.cuda.synchronize()
        xs_np, out_np, hdr_np = to_np_u16(xs), out.cpu().numpy(), hdr.cpu().numpy()
        for l in range(n):
            ref = olayer.layer_forward(specs[l], xs_np[l], keep_experts=False)
            assert np.array_equal(hdr_np[l], ref["header"]), l
            for t in range(m):
                assert rel_l2(out_np[l, t], ref["out_f32"][t]) <= 1e-3, (l, t)
                assert np.abs(out_np[l, t] - ref["out_f32"][t]).max() <= 1e-2, (l, t)
            assert np.array_equal(xs_np[l + 1], olayer.residual(xs_np[l], out_np[l])), l
    for m in (8, 2):
        x_np = synth.tokens(specs[0], 30, m)
        _, o_w, b_w, h_w = _run(dls[0], x_np)
        _, o_n, b_n, h_n = _run(dls[0], x_np, noalloc=True)
        assert np.array_equal(h_n, h_w) and np.array_equal(o_n.view(np.uint32), o_w.view(np.uint32)), m
    del dls
    torch.cuda.empty_cache()

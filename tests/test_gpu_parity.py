"""GPU parity: the HIP path (through the C ABI) against the oracle on the
same seeded inputs. Bit-exact: q8_1 codes and scales, router logits, scores,
headers (picks, weight bits, plan). GEMV outputs: the correctly rounded
exact value, or its neighbour where the oracle flags the exact value as lying
near an f32 midpoint. Layer output: rel-L2 <= 1e-3 and max-abs <= 1e-2."""
import numpy as np
import pytest
import torch

import oracle
import routing_quant_expert_amd as R
import synth
from oracle import layer as olayer
from synth.device import DeviceLayer, fill_arena, lib as synth_lib
from tests.gpu_helpers import (check_combine_bits, f32_accept, host_spec, oracle_header, plan_tables, rel_l2, say, to_np_u16,
                               workspace, ws_array)

pytestmark = pytest.mark.gpu

TINY, DS41 = synth.SHAPE_TINY, synth.SHAPE_DS41
_LAYERS = {}


def device_layer(shape, seed=1):
    key = (shape, seed)
    if key not in _LAYERS:
        if shape == DS41:                       # keep one 3.5 GB arena resident at a time
            for k in [k for k in _LAYERS if k[0] == DS41]:
                del _LAYERS[k]
            torch.cuda.empty_cache()
        say(f"generating layer {shape.dim}x{shape.inter} seed {seed} on the device")
        _LAYERS[key] = DeviceLayer(host_spec(shape, seed))
        torch.cuda.synchronize()
    return _LAYERS[key]


# ------------------------------------------------------------ generators
def test_device_generator_matches_host():
    for shape in (TINY, DS41):
        spec = host_spec(shape, seed=3)
        s = shape
        buf = torch.zeros(s.expert_stride + 64, dtype=torch.uint8, device="cuda")
        base = buf.data_ptr()
        for e in (0, 7, 383):
            st = torch.cuda.current_stream().cuda_stream
            L = synth_lib()
            assert L.synth_q2k_blocks(base + s.gate_off, spec.seed, spec.tag(synth.K_EXP_GATE, e), 0,
                                      s.inter * s.nsb_gate, st) == 0
            assert L.synth_q2k_blocks(base + s.up_off, spec.seed, spec.tag(synth.K_EXP_UP, e), 0,
                                      s.inter * s.nsb_gate, st) == 0
            assert L.synth_q3k_blocks(base + s.down_off, spec.seed, spec.tag(synth.K_EXP_DOWN, e), 0,
                                      s.dim * s.nsb_down, st) == 0
            got = buf[:s.expert_stride].cpu().numpy()
            assert np.array_equal(got, synth.expert_bytes(spec, e)), (shape, e)
    dl = device_layer(TINY)
    assert np.array_equal(to_np_u16(dl.gate_w), synth.gate_w(dl.spec))
    assert np.array_equal(to_np_u16(dl.sh_w2), synth.shared_w(dl.spec, "w2"))
    assert np.array_equal(dl.bias.cpu().numpy(), synth.bias(dl.spec))


# ---------------------------------------------------------------- scores
def test_scores_bit_exact_against_oracle():
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.normal(0, 1.28, 2_000_000), rng.uniform(-110, 25, 1_000_000),
                        np.ldexp(rng.uniform(-1, 1, 500_000), rng.integers(-140, 6, 500_000)),
                        np.array([0.0, -0.0, 20.0, 20.000002, 19.999998, -104.0, -103.99, 88.0, np.inf,
                                  -np.inf])]).astype(np.float32)
    want = oracle.scores(x, 1.0)
    xd = torch.from_numpy(x).cuda()
    out = torch.empty_like(xd)
    for flags in (0, 1):
        R.scores(xd, 1.0, out, flags)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
        assert bad.size == 0, (flags, x[bad[:5]], got[bad[:5]], want[bad[:5]])
        say(f"scores flags={flags}: {x.size} values bit-exact")


def _near_f32_midpoint(y64, rel):
    """Where a float64 value lies within rel * |y| of the midpoint between its
    f32 rounding and that rounding's neighbour toward it (torch, device)."""
    f = y64.float()
    fd = f.double()
    nb = torch.nextafter(f, torch.where(y64 > fd, torch.full_like(f, float("inf")), torch.full_like(f, float("-inf"))))
    mid = 0.5 * (fd + nb.double())
    return (fd != y64) & ((y64 - mid).abs() <= rel * y64.abs())


def test_score_chain_on_every_f32_input():
    """All 2^32 f32 inputs (temp 1): the device's fast score path (double
    exp/log1p with Ziv's rounding test) equals its extended-precision path on
    every input, so the test's bound holds everywhere; and on every finite
    input of [-104, 20] whose exp or log1p step lies within 2^-40 relative of
    an f32 midpoint (the hard cases of correct rounding, found with float64
    on the device) the device equals the oracle's correctly rounded chain."""
    n = 1 << 27
    hard = []
    for c in range(32):
        v = torch.arange(c * n, (c + 1) * n, dtype=torch.int64, device="cuda")
        x = (((v + (1 << 31)) % (1 << 32)) - (1 << 31)).to(torch.int32).view(torch.float32)
        a, b = torch.empty_like(x), torch.empty_like(x)
        R.scores(x, 1.0, a, 0)
        R.scores(x, 1.0, b, 1)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), c
        ok = torch.isfinite(x) & (x >= -104.0) & (x <= 20.0)
        xd = x.double()
        e64 = torch.exp(xd)
        l64 = torch.log1p(e64.float().double())
        h = ok & (_near_f32_midpoint(e64, 2.0 ** -40) | _near_f32_midpoint(l64, 2.0 ** -40))
        hard.append(x[h].cpu())
        del v, x, a, b, xd, e64, l64, h
    hx = torch.cat(hard).numpy()
    say(f"score chain: 2^32 inputs fast == extended; {hx.size} near-midpoint inputs against the oracle")
    assert hx.size > 1000
    want = oracle.scores(hx, 1.0)
    xd = torch.from_numpy(hx).cuda()
    out = torch.empty_like(xd)
    R.scores(xd, 1.0, out, 0)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, (hx[bad[:5]], got[bad[:5]], want[bad[:5]])
    torch.cuda.empty_cache()


def test_exp_step_on_every_f32_input():
    """Every f32 in [-104, 89] (the fast path's domain; the SwiGLU's exp
    reaches up to 89): the device's exp step (the straight-line float64
    estimate with Ziv's test) equals its extended-precision path on every
    input, and on the inputs whose float64 exp lies within 2^-40 of an f32
    midpoint (the hard cases) it equals the oracle's correctly rounded exp."""
    n = 1 << 27
    hard = []
    checked = 0
    for c in range(32):
        v = torch.arange(c * n, (c + 1) * n, dtype=torch.int64, device="cuda")
        x = (((v + (1 << 31)) % (1 << 32)) - (1 << 31)).to(torch.int32).view(torch.float32)
        x = x[torch.isfinite(x) & (x >= -104.0) & (x <= 89.0)]
        if x.numel() == 0:
            continue
        a, b = torch.empty_like(x), torch.empty_like(x)
        R.scores(x, 1.0, a, R.SCORES_EXP_ONLY)
        R.scores(x, 1.0, b, R.SCORES_EXP_ONLY | R.SCORES_EXTENDED)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32)), c
        checked += x.numel()
        h = _near_f32_midpoint(torch.exp(x.double()), 2.0 ** -40)
        hard.append(x[h].cpu())
        del v, x, a, b, h
    hx = torch.cat(hard).numpy()
    say(f"exp step: {checked} inputs fast == extended; {hx.size} near-midpoint inputs against the oracle")
    assert checked > 2_000_000_000 and hx.size > 100
    want = oracle.exp_cr(hx)
    xd = torch.from_numpy(hx).cuda()
    out = torch.empty_like(xd)
    R.scores(xd, 1.0, out, R.SCORES_EXP_ONLY)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, (hx[bad[:5]], got[bad[:5]], want[bad[:5]])
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- routing
@pytest.mark.parametrize("shape,m", [(TINY, 1), (TINY, 5), (TINY, 37), (DS41, 1), (DS41, 8)])
def test_route_select_bit_exact(shape, m):
    dl = device_layer(shape)
    spec = dl.spec
    c = dl.cfg
    x_np = synth.tokens(spec, 100, m)
    x = torch.from_numpy(x_np).cuda()
    ws = workspace(c, m)
    hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
    logits = torch.empty((m, shape.n_routed), dtype=torch.float32, device="cuda")
    say(f"route_select dim={shape.dim} m={m}")
    R.route_select(c, x, dl.gate_w, dl.bias, hdr, ws, logits=logits)
    torch.cuda.synchronize()
    lg, want_hdr, sc = oracle_header(spec, x_np)
    assert np.array_equal(logits.cpu().numpy().view(np.uint32), lg.view(np.uint32))
    assert np.array_equal(hdr.cpu().numpy(), want_hdr)
    L = R.workspace_layout(c, m)
    assert np.array_equal(ws_array(ws, L, "scores", np.float32, m * shape.n_routed).reshape(m, -1).view(np.uint32),
                          sc.view(np.uint32))
    xq = ws_array(ws, L, "xq", np.int8, m * shape.dim).reshape(m, -1)
    xd = ws_array(ws, L, "xd", np.uint16, m * shape.dim // 32).reshape(m, -1)
    xs = ws_array(ws, L, "xs", np.int32, m * shape.dim // 16).reshape(m, -1)
    for t in range(m):
        q, d = oracle.q8_1(oracle.bf16_to_f32(x_np[t]))
        assert np.array_equal(xq[t], q) and np.array_equal(xd[t], d)
        assert np.array_equal(xs[t], q.reshape(-1, 16).astype(np.int32).sum(axis=1))
    # a token's logits do not depend on the batch
    if m > 1:
        ws1 = workspace(c, 1)
        lg1 = torch.empty((1, shape.n_routed), dtype=torch.float32, device="cuda")
        h1 = torch.empty((1, R.header_words(c)), dtype=torch.int32, device="cuda")
        R.route_select(c, x[m - 1:m].contiguous(), dl.gate_w, dl.bias, h1, ws1, logits=lg1)
        torch.cuda.synchronize()
        assert np.array_equal(lg1.cpu().numpy()[0].view(np.uint32), logits.cpu().numpy()[m - 1].view(np.uint32))


def test_route_ties_and_nan():
    dl = device_layer(TINY)
    c = dl.cfg
    m = 3
    x_np = synth.tokens(dl.spec, 0, m)
    x_np[0] = 0                      # all logits 0 -> all scores equal
    x_np[2, 5] = 0x7FC0              # a bf16 NaN -> NaN logits -> NaN keys
    x = torch.from_numpy(x_np).cuda()
    zero_bias = torch.zeros(c.n_routed, dtype=torch.float32, device="cuda")
    ws = workspace(c, m)
    hdr = torch.empty((m, 19), dtype=torch.int32, device="cuda")
    R.route_select(c, x, dl.gate_w, zero_bias, hdr, ws)
    torch.cuda.synchronize()
    h = hdr.cpu().numpy()
    _, want, _ = oracle_header(dl.spec, x_np, np.zeros(c.n_routed, np.float32))
    assert list(h[0, 1:7]) == [0, 1, 2, 3, 4, 5]
    assert np.array_equal(h[:2], want[:2])
    assert h[2, 0] == R.MOE_STATUS_NAN_KEY and want[2, 0] == R.MOE_STATUS_NAN_KEY
    assert np.array_equal(h[2, 1:7], want[2, 1:7]) and np.array_equal(h[2, 13:19], want[2, 13:19])
    L = R.workspace_layout(c, m)
    assert ws_array(ws, L, "status", np.int32, 1)[0] & R.MOE_STATUS_NAN_KEY


def test_router_order_pins_on_device():
    """The hand-built rows whose logits only the stated summation order gives
    (the oracle's order pins): the device router must give the same values
    on the decode front (m = 1, 8), the route-select call at m = 16, and the
    prefill router (layer forward at m = 16)."""
    from tests.test_oracle_route import _order_pin_inputs
    shape = synth.Shape(dim=1024, inter=512)
    dl = device_layer(shape, seed=3)
    c = dl.cfg
    x1, w4, want4 = _order_pin_inputs(shape.dim)
    gw = np.zeros((shape.n_routed, shape.dim), np.uint16)
    gw[:4] = w4
    want = np.zeros(shape.n_routed, np.float32)
    want[:4] = want4
    gw_dev = torch.from_numpy(gw.view(np.int16)).cuda()
    zb = torch.zeros(shape.n_routed, dtype=torch.float32, device="cuda")
    layer = R.Layer(gw_dev.data_ptr(), zb.data_ptr(), dl.experts, dl.sh_w1.data_ptr(), dl.sh_w3.data_ptr(),
                    dl.sh_w2.data_ptr())
    for m in (1, 8, 16):
        x = torch.from_numpy(np.repeat(x1, m, axis=0)).cuda()
        ws = workspace(c, m)
        hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
        lg = torch.empty((m, shape.n_routed), dtype=torch.float32, device="cuda")
        say(f"router order pins: route_select m={m}")
        R.route_select(c, x, gw_dev, zb, hdr, ws, logits=lg)
        torch.cuda.synchronize()
        got = lg.cpu().numpy()
        for t in range(m):
            assert np.array_equal(got[t].view(np.uint32), want.view(np.uint32)), (m, t, got[t][:4])
        say(f"router order pins: layer_forward m={m}")
        out = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
        R.layer_forward(c, layer, x, out, ws, header=hdr)
        torch.cuda.synchronize()
        L = R.workspace_layout(c, m)
        got = ws_array(ws, L, "logits", np.float32, m * shape.n_routed).reshape(m, -1)
        for t in range(m):
            assert np.array_equal(got[t].view(np.uint32), want.view(np.uint32)), (m, t, got[t][:4])


# ------------------------------------------------------------ full layer
def _check_layer(dl, x_np, m, out_f32, out_bf16, hdr, ws, with_shared=True):
    spec, c, shape = dl.spec, dl.cfg, dl.spec.shape
    say(f"oracle layer dim={shape.dim} m={m}")
    ref = olayer.layer_forward(spec, x_np, with_shared=with_shared)
    assert np.array_equal(hdr, ref["header"])
    L = R.workspace_layout(c, m)
    tab = plan_tables(ws, L, m, shape.topk)
    P = L["max_pairs"]
    inter, dim = shape.inter, shape.dim
    g = ws_array(ws, L, "g", np.float32, P * inter).reshape(P, inter)
    u = ws_array(ws, L, "u", np.float32, P * inter).reshape(P, inter)
    h = ws_array(ws, L, "h", np.float32, P * inter).reshape(P, inter)
    hq = ws_array(ws, L, "hq", np.int8, P * inter).reshape(P, inter)
    hd = ws_array(ws, L, "hd", np.uint16, P * inter // 32).reshape(P, -1)
    hs = ws_array(ws, L, "hs", np.int32, P * inter // 16).reshape(P, -1)
    y = ws_array(ws, L, "y", np.float32, P * dim).reshape(P, dim)
    shq = with_shared and spec.shared_quant   # the K-quant shared expert: plan expert n_routed, weight 1, last
    assert tab["n_pairs"] == m * (shape.topk + (1 if shq else 0))
    if not shq:
        assert np.all(tab["tok_pairs"][:, shape.topk] == -1)
    accepted = 0   # over all pairs, for the log line and the whole-output comparison
    for p in range(tab["n_pairs"]):
        t, e = int(tab["pair_tok"][p]), int(tab["pair_expert"][p])
        if e == shape.n_routed:
            assert shq and tab["pair_w"][p] == 1.0 and tab["tok_pairs"][t][shape.topk] == p
            ex = ref["shared"][t]
            down = synth.shared_q_blocks(spec, "down")
        else:
            ids = list(ref["tok"][t]["ids"])
            k = ids.index(e)
            ex = ref["tok"][t]["experts"][k]
            assert tab["pair_w"][p] == ref["tok"][t]["w_plan"][k]
            assert tab["tok_pairs"][t][k] == p
            down = synth.expert_blocks(spec, e, "down")
        # this pair's g/u: a neighbour accepted at a flagged near-midpoint makes its own h differ legitimately,
        # so only this pair's h checks are skipped then
        gu_acc = f32_accept(g[p], ex["g"], ex["near_g"], f"g pair {p}")
        gu_acc += f32_accept(u[p], ex["u"], ex["near_u"], f"u pair {p}")
        if gu_acc == 0:
            assert np.array_equal(h[p].view(np.uint32), ex["h"].view(np.uint32)), f"h pair {p}"
            assert np.array_equal(hq[p], ex["hq"]) and np.array_equal(hd[p], ex["hd16"]), f"h q8_1 pair {p}"
            assert np.array_equal(hs[p], ex["hq"].reshape(-1, 16).astype(np.int32).sum(axis=1))
            accepted += f32_accept(y[p], ex["y"], ex["near_y"], f"y pair {p}")
        else:   # the rest of this pair is checked exactly on the device's own g and u
            hh = oracle.swiglu(g[p], u[p], shape.swiglu_limit)
            assert np.array_equal(h[p].view(np.uint32), hh.view(np.uint32)), f"h pair {p} (own g/u)"
            q, d = oracle.q8_1(hh)
            assert np.array_equal(hq[p], q) and np.array_equal(hd[p], d), f"h q8_1 pair {p} (own g/u)"
            yy, near = oracle.q3k_gemv(down, dim, inter, q, d)
            accepted += f32_accept(y[p], yy, near, f"y pair {p} (own h)")
        accepted += gu_acc
    if accepted:
        say(f"  {accepted} GEMV outputs took the other correct rounding next to an f32 midpoint")
    want = ref["out_f32"] if with_shared else ref["y_routed"]
    err = np.abs(out_f32 - want)
    assert rel_l2(out_f32, want) <= 1e-3 and err.max() <= 1e-2, (rel_l2(out_f32, want), err.max())
    if accepted == 0 and (shq or not with_shared):   # no f32 GEMV of unstated order: the output is exact
        assert np.array_equal(out_f32.view(np.uint32), want.view(np.uint32))
    check_combine_bits(ws, L, tab, m, shape.topk, out_f32, with_shared and not shq)
    if out_bf16 is not None:
        assert np.array_equal(out_bf16, oracle.f32_to_bf16(out_f32))
    return ref


@pytest.mark.parametrize("shape,m", [(TINY, 1), (TINY, 2), (TINY, 8), (DS41, 1), (DS41, 3)])
def test_layer_forward_matches_oracle(shape, m):
    dl = device_layer(shape)
    c = dl.cfg
    x_np = synth.tokens(dl.spec, 7, m)
    x = torch.from_numpy(x_np).cuda()
    ws = workspace(c, m)
    out = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
    out32 = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((m, 19), dtype=torch.int32, device="cuda")
    say(f"layer_forward dim={shape.dim} m={m}")
    R.layer_forward(c, dl.layer, x, out, ws, out_f32=out32, header=hdr)
    torch.cuda.synchronize()
    ref = _check_layer(dl, x_np, m, out32.cpu().numpy(), to_np_u16(out), hdr.cpu().numpy(), ws)
    # shared expert intermediates (f32 accumulation in the device's own order)
    L = R.workspace_layout(c, m)
    sg = ws_array(ws, L, "sg", np.float32, m * shape.inter).reshape(m, -1)
    for t in range(m):
        assert rel_l2(sg[t], ref["shared"][t]["sg"]) < 1e-5


def test_layer_forward_single_token_16_tokens_full_size():
    """The metric's workload: dim 4096, one token per call, 16 different
    tokens through one workspace, every pair of every token checked."""
    dl = device_layer(DS41)
    c, shape = dl.cfg, DS41
    n = 16
    x_np = synth.tokens(dl.spec, 200, n)
    ws = workspace(c, 1)
    say(f"layer_forward dim=4096 m=1, {n} tokens")
    for t in range(n):
        x = torch.from_numpy(x_np[t:t + 1].copy()).cuda()
        out = torch.empty((1, shape.dim), dtype=torch.uint16, device="cuda")
        out32 = torch.empty((1, shape.dim), dtype=torch.float32, device="cuda")
        hdr = torch.empty((1, R.header_words(c)), dtype=torch.int32, device="cuda")
        R.layer_forward(c, dl.layer, x, out, ws, out_f32=out32, header=hdr)
        torch.cuda.synchronize()
        _check_layer(dl, x_np[t:t + 1], 1, out32.cpu().numpy(), to_np_u16(out), hdr.cpu().numpy(), ws)


@pytest.mark.parametrize("group", [0, 1])
def test_layer_forward_correlated_m8_full_size(group):
    """Eight correlated tokens (a shared component of weight 0.5) through one
    dim-4096 layer: the union path with partly overlapping picks, every pair
    and every output checked."""
    dl = device_layer(DS41)
    c, shape = dl.cfg, DS41
    m = 8
    x_np = synth.correlated_tokens(dl.spec, m, group=group)
    x = torch.from_numpy(x_np).cuda()
    ws = workspace(c, m)
    out = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
    out32 = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
    say(f"layer_forward dim=4096 correlated m=8 group {group}")
    R.layer_forward(c, dl.layer, x, out, ws, out_f32=out32, header=hdr)
    torch.cuda.synchronize()
    h = hdr.cpu().numpy()
    n_u = len(np.unique(h[:, 1:1 + shape.topk]))
    say(f"  {n_u} distinct experts for {m * shape.topk} picks")
    assert n_u < m * shape.topk     # the picks overlap
    _check_layer(dl, x_np, m, out32.cpu().numpy(), to_np_u16(out), h, ws)


@pytest.mark.parametrize("shape,rows", [(TINY, [0, 0, 0]), (TINY, [0, 0, 0, 0, 0, 1, 1, 2]),
                                        (DS41, [0, 0, 0, 0, 0, 1, 1, 2]), (DS41, [0] * 8)])
def test_layer_forward_repeated_tokens(shape, rows):
    """Union path with experts shared by many tokens: repeated rows give each
    expert np = 1..8 tokens (np = 3, 5, 6, 7 leave some of the power-of-two
    token slots of the union kernels' lane groups empty)."""
    dl = device_layer(shape)
    c = dl.cfg
    m = len(rows)
    base = synth.tokens(dl.spec, 23, max(rows) + 1)
    x_np = np.ascontiguousarray(base[rows])
    x = torch.from_numpy(x_np).cuda()
    ws = workspace(c, m)
    out = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
    out32 = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((m, 19), dtype=torch.int32, device="cuda")
    say(f"layer_forward dim={shape.dim} rows={rows}")
    R.layer_forward(c, dl.layer, x, out, ws, out_f32=out32, header=hdr)
    torch.cuda.synchronize()
    o = out32.cpu().numpy()
    _check_layer(dl, x_np, m, o, to_np_u16(out), hdr.cpu().numpy(), ws)
    for t in range(1, m):   # equal rows give equal outputs, bit for bit
        if rows[t] == rows[0]:
            assert np.array_equal(o[t].view(np.uint32), o[0].view(np.uint32))


@pytest.mark.parametrize("shape,m", [(TINY, 1), (TINY, 3), (DS41, 1), (DS41, 2)])
def test_experts_decode_matches_oracle(shape, m):
    dl = device_layer(shape)
    c = dl.cfg
    x_np = synth.tokens(dl.spec, 11, m)
    x = torch.from_numpy(x_np).cuda()
    _, hdr_np, _ = oracle_header(dl.spec, x_np)
    hdr = torch.from_numpy(hdr_np).cuda()
    ws = workspace(c, m)
    y = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
    R.experts_decode(c, x, hdr, dl.experts, y, ws)
    torch.cuda.synchronize()
    _check_layer(dl, x_np, m, y.cpu().numpy(), None, hdr_np, ws, with_shared=False)


def test_experts_decode_single_token_rejects_bad_picks():
    dl = device_layer(TINY)
    c = dl.cfg
    x_np = synth.tokens(dl.spec, 0, 1)
    _, hdr_np, _ = oracle_header(dl.spec, x_np)
    ws = workspace(c, 1)
    for bad in ((2, 384), (3, -1), (4, int(hdr_np[0, 1]))):
        h = hdr_np.copy()
        h[0, bad[0]] = bad[1]
        y = torch.full((1, c.dim), 7.0, dtype=torch.float32, device="cuda")
        R.experts_decode(c, torch.from_numpy(x_np).cuda(), torch.from_numpy(h).cuda(), dl.experts, y, ws)
        torch.cuda.synchronize()
        assert np.all(y.cpu().numpy() == 0), bad
        L = R.workspace_layout(c, 1)
        assert ws_array(ws, L, "status", np.int32, 1)[0] & R.MOE_STATUS_BAD_PICK
    # and a good header afterwards still works in the same workspace
    y = torch.empty((1, c.dim), dtype=torch.float32, device="cuda")
    R.experts_decode(c, torch.from_numpy(x_np).cuda(), torch.from_numpy(hdr_np).cuda(), dl.experts, y, ws)
    torch.cuda.synchronize()
    ref = olayer.layer_forward(dl.spec, x_np, with_shared=False)
    assert rel_l2(y.cpu().numpy()[0], ref["y_routed"][0]) < 1e-6


def test_experts_decode_rejects_bad_picks():
    dl = device_layer(TINY)
    c = dl.cfg
    m = 3
    x_np = synth.tokens(dl.spec, 0, m)
    _, hdr_np, _ = oracle_header(dl.spec, x_np)
    hdr_np = hdr_np.copy()
    hdr_np[1, 2] = 384               # out of range
    hdr_np[2, 3] = hdr_np[2, 1]      # repeated
    ws = workspace(c, m)
    y = torch.full((m, c.dim), 7.0, dtype=torch.float32, device="cuda")
    R.experts_decode(c, torch.from_numpy(x_np).cuda(), torch.from_numpy(hdr_np).cuda(), dl.experts, y, ws)
    torch.cuda.synchronize()
    yy = y.cpu().numpy()
    assert np.all(yy[1] == 0) and np.all(yy[2] == 0)
    ref = olayer.layer_forward(dl.spec, x_np[:1], with_shared=False)
    assert rel_l2(yy[0], ref["y_routed"][0]) < 1e-6
    L = R.workspace_layout(c, m)
    assert ws_array(ws, L, "status", np.int32, 1)[0] & R.MOE_STATUS_BAD_PICK


# ------------------------------------------------ the single-token launches
@pytest.mark.parametrize("shape,calls", [(TINY, 4), (DS41, 2)])
def test_single_token_kernel_reuses_its_workspace(shape, calls):
    """Back-to-back m = 1 layers on one workspace: the front launch's router
    counter is left at zero by every call, so each call is right on its own."""
    dl = device_layer(shape)
    c = dl.cfg
    ws = workspace(c, 1)
    x_np = synth.tokens(dl.spec, 40, calls)
    x = torch.from_numpy(x_np).cuda()
    outs = torch.empty((calls, shape.dim), dtype=torch.float32, device="cuda")
    ob = torch.empty((calls, shape.dim), dtype=torch.uint16, device="cuda")
    hdr = torch.empty((calls, R.header_words(c)), dtype=torch.int32, device="cuda")
    say(f"single-token kernel dim={shape.dim}: {calls} calls on one workspace")
    for t in range(calls):
        R.layer_forward(c, dl.layer, x[t:t + 1], ob[t:t + 1], ws, out_f32=outs[t:t + 1], header=hdr[t:t + 1])
    torch.cuda.synchronize()
    L = R.workspace_layout(c, 1)
    assert ws_array(ws, L, "status", np.int32, 1)[0] == 0
    assert not ws_array(ws, L, "ctl", np.uint32, 64).any()
    ref = olayer.layer_forward(dl.spec, x_np)
    assert np.array_equal(hdr.cpu().numpy(), ref["header"])
    got = outs.cpu().numpy()
    for t in range(calls):
        err = np.abs(got[t] - ref["out_f32"][t])
        assert rel_l2(got[t], ref["out_f32"][t]) <= 1e-3 and err.max() <= 1e-2, t


@pytest.mark.parametrize("shape", [TINY, DS41])
def test_single_token_kernel_equals_multi_token_path(shape):
    """The same token alone (the single-token kernels) and twice in an m = 2
    call (the multi-token kernels): identical header and routed sum, and layer
    outputs that differ only by the shared expert's f32 summation order."""
    dl = device_layer(shape)
    c = dl.cfg
    x_np = synth.tokens(dl.spec, 77, 1)
    x1 = torch.from_numpy(x_np).cuda()
    x2 = torch.from_numpy(np.concatenate([x_np, x_np])).cuda()
    say(f"single vs multi-token path dim={shape.dim}")
    res = {}
    for m, x in ((1, x1), (2, x2)):
        ws = workspace(c, m)
        out = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
        o32 = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
        hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
        R.layer_forward(c, dl.layer, x, out, ws, out_f32=o32, header=hdr)
        y = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
        R.experts_decode(c, x, hdr, dl.experts, y, ws)
        torch.cuda.synchronize()
        res[m] = (hdr.cpu().numpy(), o32.cpu().numpy(), y.cpu().numpy())
    h1, o1, y1 = res[1]
    h2, o2, y2 = res[2]
    assert np.array_equal(h1[0], h2[0]) and np.array_equal(h2[0], h2[1])
    assert np.array_equal(y1[0].view(np.uint32), y2[0].view(np.uint32))
    assert np.array_equal(y2[0].view(np.uint32), y2[1].view(np.uint32))
    assert rel_l2(o1[0], o2[0]) <= 1e-5 and np.abs(o1[0] - o2[0]).max() <= 1e-3


# ------------------------------------------------------------ layer stack
def _check_stack(specs, xs_np, out_np, hdr_np, layers_checked):
    """Teacher-forced: the oracle runs layer l on the device's own x_l."""
    for i, l in enumerate(layers_checked):
        if i % 8 == 7:
            say(f"  layer {l} checked")
        ref = olayer.layer_forward(specs[l], xs_np[l], keep_experts=False)
        assert np.array_equal(hdr_np[l], ref["header"]), l
        for t in range(xs_np.shape[1]):
            err = np.abs(out_np[l, t] - ref["out_f32"][t])
            assert rel_l2(out_np[l, t], ref["out_f32"][t]) <= 1e-3 and err.max() <= 1e-2, (l, t)
    for l in range(len(specs)):   # the residual stream is exact given the device's out_l
        assert np.array_equal(xs_np[l + 1], olayer.residual(xs_np[l], out_np[l])), l


def _run_stack(dls, x0, n_layers):
    c = dls[0].cfg
    m, dim = x0.shape
    xs = torch.empty((n_layers + 1, m, dim), dtype=torch.uint16, device="cuda")
    xs[0] = torch.from_numpy(x0).cuda()
    out = torch.empty((n_layers, m, dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((n_layers, m, R.header_words(c)), dtype=torch.int32, device="cuda")
    ws = workspace(c, m)
    R.stack_forward(c, [d.layer for d in dls], xs, ws, out_f32=out, headers=hdr)
    torch.cuda.synchronize()
    return to_np_u16(xs), out.cpu().numpy(), hdr.cpu().numpy()


@pytest.mark.parametrize("m", [1, 3])
def test_stack_forward_40_small_layers(m):
    n = 40
    specs = [synth.LayerSpec(TINY, seed=5, layer=l) for l in range(n)]
    say(f"stack of {n} layers dim={TINY.dim} m={m}: generating")
    dls = [DeviceLayer(sp) for sp in specs]
    x0 = synth.tokens(specs[0], 3, m)
    xs_np, out_np, hdr_np = _run_stack(dls, x0, n)
    _check_stack(specs, xs_np, out_np, hdr_np, range(n))
    del dls
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m", [1, 3])
def test_stack_graph_capture_replays_equal_eager(m):
    """The decode step through a stack, captured in a graph on a side stream:
    three replays, with eager work and synchronisation between them, each
    give the eager residual stream, outputs and headers bit for bit (the
    kernels reset their own counters, so nothing needs a memset node)."""
    n = 4
    specs = [synth.LayerSpec(TINY, seed=9, layer=l) for l in range(n)]
    say(f"graph of a {n}-layer stack dim={TINY.dim} m={m}")
    dls = [DeviceLayer(sp) for sp in specs]
    c = dls[0].cfg
    layers = [d.layer for d in dls]
    xs = torch.empty((n + 1, m, TINY.dim), dtype=torch.uint16, device="cuda")
    xs[0] = torch.from_numpy(synth.tokens(specs[0], 11, m)).cuda()
    out = torch.empty((n, m, TINY.dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((n, m, R.header_words(c)), dtype=torch.int32, device="cuda")
    ws = workspace(c, m)
    R.stack_forward(c, layers, xs, ws, out_f32=out, headers=hdr)
    torch.cuda.synchronize()
    ref_xs, ref_out, ref_hdr = xs.clone(), out.clone(), hdr.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            R.stack_forward(c, layers, xs, ws, out_f32=out, headers=hdr, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        xs[1:].fill_(0)
        out.fill_(0.0)
        hdr.fill_(0)
        R.stack_forward(c, layers[:1], xs[:2], ws)   # eager work between replays
        torch.cuda.synchronize()
        xs[1:].fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(xs, ref_xs), rep
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), rep
        assert torch.equal(hdr, ref_hdr), rep
    del dls


def test_stack_forward_40_full_size_layers():
    """Forty dim-4096 layers resident at once (~142 GB), one decode step per
    token for two tokens; the oracle checks every layer of both steps
    (teacher-forced on the device's own x_l), the residual stream too."""
    n = 40
    for k in [k for k in _LAYERS if k[0] == DS41]:
        del _LAYERS[k]
    torch.cuda.empty_cache()
    specs = [synth.LayerSpec(DS41, seed=5, layer=l) for l in range(n)]
    say(f"stack of {n} layers dim={DS41.dim}: generating ~{n * DS41.n_routed * DS41.expert_stride / 1e9:.0f} GB")
    dls = [DeviceLayer(sp) for sp in specs]
    torch.cuda.synchronize()
    runs = [_run_stack(dls, synth.tokens(specs[0], tok, 1), n) for tok in (3, 4)]   # two single-token steps
    xs_np, out_np, hdr_np = (np.concatenate([r[i] for r in runs], axis=1) for i in range(3))
    say(f"  oracle on all {n} layers of both steps")
    _check_stack(specs, xs_np, out_np, hdr_np, range(n))
    del dls
    torch.cuda.empty_cache()

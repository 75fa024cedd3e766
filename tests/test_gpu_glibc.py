"""The glibc score mode on the device: the scores equal the host glibc chain
(the oracle's) bit for bit on every input where it differs from the
correctly rounded chain and on random logits; selection headers and layer
outputs in the mode equal the oracle's in the same mode, on logits built to
land on those inputs (router rows with one non-zero column and one-hot
tokens make the logits exact) and on the full-size layer's own tokens
[device_route.rs, module doc: the device selection bit for bit with the host
reference's glibc-exact softplus]."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import routing_quant_expert_amd as R
import synth
from synth.device import DeviceLayer
from tests.gpu_helpers import rel_l2, say, to_np_u16, workspace

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(31)


def glibc(shape):
    return dataclasses.replace(shape, score_mode=1)


@pytest.fixture(scope="module")
def table():
    say("building and registering the glibc score table")
    R.enable_glibc_scores()
    return R.glibc_score_table()


def _dev_scores(z: np.ndarray, temp: float, flags: int) -> np.ndarray:
    zd = torch.from_numpy(z).cuda()
    out = torch.empty_like(zd)
    R.scores(zd, temp, out, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_scores_on_every_exception(table):
    keys, vals, _ = table
    z = keys.view(np.float32)
    say(f"{z.size} inputs where glibc's chain differs")
    got = _dev_scores(z, 1.0, 2)
    assert np.array_equal(got.view(np.uint32), vals)
    assert np.array_equal(vals, oracle.scores_glibc(z, 1.0).view(np.uint32))
    # the correctly rounded mode keeps its own values there
    cr = _dev_scores(z[:1_000_000], 1.0, 0)
    assert np.all(cr.view(np.uint32) != vals[:1_000_000])


def test_scores_random_and_every_bf16(table):
    bf = np.arange(1 << 16, dtype=np.uint32) << 16
    zb = bf.view(np.float32)
    lg = np.concatenate([RNG.normal(0, 4, 3_000_000).astype(np.float32),
                         RNG.uniform(-1, 0, 1_000_000).astype(np.float32), zb])
    for temp in (1.0, 0.75, 1.5):
        say(f"temp {temp}")
        got = _dev_scores(lg, temp, 2)
        assert np.array_equal(got.view(np.uint32), oracle.scores_glibc(lg, temp).view(np.uint32)), temp


def test_unregistered_device_refuses(table):
    c = R.cfg_from_shape(glibc(synth.SHAPE_TINY))
    L = R.lib()
    assert L.moe_set_score_table(None, None, None, 0) == 0
    try:
        with pytest.raises(R.MoeError, match="moe_set_score_table"):
            _dev_scores(np.zeros(8, np.float32), 1.0, 2)
        with pytest.raises(R.MoeError, match="moe_set_score_table"):
            x = torch.zeros((1, 512), dtype=torch.uint16, device="cuda")
            gw = torch.zeros((384, 512), dtype=torch.uint16, device="cuda")
            b = torch.zeros(384, dtype=torch.float32, device="cuda")
            h = torch.empty((1, R.header_words(c)), dtype=torch.int32, device="cuda")
            R.route_select(c, x, gw, b, h, workspace(c, 1))
    finally:
        t = R.binding._score_tables[torch.cuda.current_device()]
        assert L.moe_set_score_table(t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), table[0].size) == 0


def _crafted(table, shape, m):
    """Router rows that are zero except in column t for token t, and one-hot
    tokens: logit(t, e) = gate_w[e, t] exactly. Each token's eight largest
    logits are bf16 values where the chains differ; the rest are negative
    ones of the same kind or small normals."""
    keys = table[0]
    bfk = keys[(keys & 0xFFFF) == 0].view(np.float32)
    hi = bfk[(bfk > 0.4) & (bfk < 20)]
    lo = bfk[bfk < 0]
    n = shape.n_routed
    gw = np.zeros((n, shape.dim), np.float32)
    for t in range(m):
        col = RNG.choice(lo, n)
        small = RNG.random(n) < 0.3
        col[small] = RNG.normal(-3, 1, small.sum())
        picks = RNG.choice(n, 8, replace=False)
        col[picks] = RNG.choice(hi, 8, replace=False)
        gw[:, t] = col
    x = np.zeros((m, shape.dim), np.float32)
    x[np.arange(m), np.arange(m)] = 1.0
    return oracle.f32_to_bf16(x), oracle.f32_to_bf16(gw)


def _route(shape, x, gw, bias):
    c = R.cfg_from_shape(shape)
    m = x.shape[0]
    lg = torch.empty((m, shape.n_routed), dtype=torch.float32, device="cuda")
    hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
    R.route_select(c, torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(gw.view(np.int16)).cuda(),
                   torch.from_numpy(bias).cuda(), hdr, workspace(c, m), logits=lg)
    torch.cuda.synchronize()
    return lg.cpu().numpy(), hdr.cpu().numpy()


@pytest.mark.parametrize("m", [1, 7, 64, 300])
def test_route_select_crafted(table, m):
    sh = synth.SHAPE_TINY
    x, gw = _crafted(table, sh, m)
    bias = np.zeros(sh.n_routed, np.float32)
    lg, hdr = _route(glibc(sh), x, gw, bias)
    rl, rh = oracle.ref_route_select(glibc(sh), x, gw, bias)
    assert np.array_equal(lg.view(np.uint32), rl.view(np.uint32))
    assert np.array_equal(hdr, rh)
    _, h0 = oracle.ref_route_select(sh, x, gw, bias)
    differ = int((hdr != h0).any(axis=1).sum())
    say(f"m={m}: {differ} tokens whose header differs from the correctly rounded mode")
    assert differ >= (m + 1) // 2


_DL = {}


def _layer(shape):
    if shape not in _DL:
        _DL.clear()
        torch.cuda.empty_cache()
        say(f"generating layer dim {shape.dim}")
        dl = DeviceLayer(synth.LayerSpec(shape, seed=29))
        dl.host_arena = dl.arena.cpu().numpy()
        _DL[shape] = dl
    return _DL[shape]


def _layer_pair(shape, dl, x, gw, bias, noalloc=False):
    """The library's layer (gate_w and bias replaced) and the oracle's mirror."""
    c = R.cfg_from_shape(shape)
    m = x.shape[0]
    gwd = torch.from_numpy(gw.view(np.int16)).cuda()
    bd = torch.from_numpy(bias).cuda()
    L = R.Layer.from_buffer_copy(dl.layer)
    L.gate_w, L.bias = gwd.data_ptr(), bd.data_ptr()
    ob = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
    of = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    if noalloc:
        R.layer_forward_noalloc(c, L, xd, ob, out_f32=of, header=hdr)
    else:
        R.layer_forward(c, L, xd, ob, workspace(c, m), out_f32=of, header=hdr)
    torch.cuda.synchronize()
    s = shape
    rb, rf, rh = oracle.ref_layer_forward(s, x, gw, bias, dl.host_arena, s.expert_stride, s.gate_off, s.up_off,
                                          s.down_off,
                                          shared_bf16=tuple(to_np_u16(t) for t in (dl.sh_w1, dl.sh_w3, dl.sh_w2)))
    return (to_np_u16(ob), of.cpu().numpy(), hdr.cpu().numpy()), (rb, rf, rh)


@pytest.mark.parametrize("m,noalloc", [(1, False), (5, False), (40, False), (1, True), (6, True)])
def test_layer_forward_crafted(table, m, noalloc):
    sh = synth.SHAPE_TINY
    dl = _layer(sh)
    x, gw = _crafted(table, sh, m)
    bias = np.zeros(sh.n_routed, np.float32)
    say(f"layer m={m} noalloc={noalloc}")
    got, want = _layer_pair(glibc(sh), dl, x, gw, bias, noalloc)
    assert np.array_equal(got[2], want[2])
    for t in range(m):
        assert rel_l2(got[1][t], want[1][t]) <= 1e-3 and np.abs(got[1][t] - want[1][t]).max() <= 1e-2, t
    _, h0 = oracle.ref_route_select(sh, x, gw, bias)
    assert (got[2] != h0).any(axis=1).sum() >= (m + 1) // 2


@pytest.mark.parametrize("m", [1, 8, 64])
def test_full_size_tokens(table, m):
    """The full-size layer on its own tokens and router: headers equal the
    oracle's glibc-mode headers; how many differ from the correctly rounded
    mode is reported."""
    sh = synth.SHAPE_DS41
    dl = _layer(sh)
    x = synth.tokens(dl.spec, 7 * m, m)
    gw, bias = to_np_u16(dl.gate_w), dl.bias.cpu().numpy()
    lg, hdr = _route(glibc(sh), x, gw, bias)
    rl, rh = oracle.ref_route_select(glibc(sh), x, gw, bias)
    assert np.array_equal(lg.view(np.uint32), rl.view(np.uint32))
    assert np.array_equal(hdr, rh)
    _, h0 = oracle.ref_route_select(sh, x, gw, bias)
    say(f"m={m}: {int((hdr != h0).any(axis=1).sum())} headers differ from the correctly rounded mode")
    if m <= 8:
        got, want = _layer_pair(glibc(sh), dl, x, gw, bias)
        assert np.array_equal(got[2], want[2])
        for t in range(m):
            assert rel_l2(got[1][t], want[1][t]) <= 1e-3, t


def test_expert_cache_routes_in_glibc_mode(table):
    """The expert cache's routing (against the slot table) in the glibc
    mode: the first layer's picks and weights equal the oracle's glibc-mode
    selection on crafted exact logits (and differ from the correctly rounded
    mode's), and every layer's results equal the resident stack's in the
    same mode, bit for bit."""
    from tests.test_gpu_cache import Stack, _run, _same_as_resident
    sh = synth.SHAPE_TINY
    stk = Stack(2, seed=43)
    stk.cfg.score_mode = R.MOE_SCORE_GLIBC
    m = 1
    x, gw = _crafted(table, sh, m)
    bias = np.zeros(sh.n_routed, np.float32)
    # the first layer gets the crafted router and no bias (gwd and bd stay referenced until the end)
    gwd, bd = torch.from_numpy(gw.view(np.int16)).cuda(), torch.from_numpy(bias).cuda()
    L = R.Layer.from_buffer_copy(stk.layers[0])
    L.gate_w, L.bias = gwd.data_ptr(), bd.data_ptr()
    stk.layers[0] = L
    ref = _run(stk, x)
    cache = stk.cache(n_slots=16, max_m=m)
    try:
        got = _run(stk, x, cache=cache)
    finally:
        cache.close()
    _same_as_resident(ref, got, sh.topk)
    k = sh.topk
    _, rh = oracle.ref_route_select(glibc(sh), x, gw, bias)
    _, h0 = oracle.ref_route_select(sh, x, gw, bias)
    assert np.array_equal(got[2][0][:, 1:1 + 2 * k], rh[:, 1:1 + 2 * k])
    assert not np.array_equal(got[2][0][:, 1 + k:1 + 2 * k], h0[:, 1 + k:1 + 2 * k])

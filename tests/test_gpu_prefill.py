"""GPU parity of the prefill path (m > 8 tokens: grouping by expert, int8
MFMA expert GEMMs, bf16 MFMA shared expert) against the oracle, through the
C ABI. The bar is the decode path's: router logits, headers, q8_1 codes and
scales bit-exact; every GEMV value the correctly rounded exact dot product
(or its neighbour where the oracle flags a near-midpoint); the layer output
within rel-L2 1e-3 and max-abs 1e-2. Each token is defined exactly as at
m = 1, so the oracle checks sampled tokens of the large batches."""
import numpy as np
import pytest
import torch

import oracle
import routing_quant_expert_amd as R
import synth
from oracle import layer as olayer
from synth.device import DeviceLayer
from tests.gpu_helpers import check_combine_bits, f32_accept, host_spec, plan_tables, rel_l2, say, to_np_u16, workspace, ws_array

pytestmark = pytest.mark.gpu

TINY, DS41 = synth.SHAPE_TINY, synth.SHAPE_DS41
_DL = {}


def dev_layer(shape, seed=1, zipf=False):
    key = (shape, seed, zipf)
    if key not in _DL:
        if shape == DS41:
            for k in [k for k in _DL if k[0] == DS41]:
                del _DL[k]
            torch.cuda.empty_cache()
        say(f"generating layer {shape.dim}x{shape.inter} seed {seed} zipf={zipf} on the device")
        _DL[key] = DeviceLayer(host_spec(shape, seed, zipf=zipf))
        torch.cuda.synchronize()
    return _DL[key]


def _ws_views(ws, c, m, shape):
    L = R.workspace_layout(c, m)
    P, inter, dim = L["max_pairs"], shape.inter, shape.dim
    v = {"tab": plan_tables(ws, L, m, shape.topk)}
    for name, dt, n in (("g", np.float32, inter), ("u", np.float32, inter), ("h", np.float32, inter),
                        ("hq", np.int8, inter), ("hd", np.uint16, inter // 32), ("hs", np.int32, inter // 16),
                        ("y", np.float32, dim)):
        v[name] = ws_array(ws, L, name, dt, P * n).reshape(P, n)
    v["L"] = L
    return v


def _check_plan(tab, hdr, m, topk, n_routed):
    """Structure of the plan at any size: pairs sorted by (expert, token),
    every valid pick of every token present once, tok_pairs pointing back."""
    status, picks, wts, plan = oracle.header_fields(hdr, topk)
    n = tab["n_pairs"]
    assert n == m * topk
    pe, pt = tab["pair_expert"][:n], tab["pair_tok"][:n]
    key = pe.astype(np.int64) * (m + 1) + pt
    assert np.all(np.diff(key) > 0)
    assert tab["n_u"] == len(np.unique(pe))
    ue, uf, un = tab["u_expert"][:tab["n_u"]], tab["u_first"][:tab["n_u"]], tab["u_npairs"][:tab["n_u"]]
    assert np.array_equal(ue, np.unique(pe)) and np.array_equal(np.cumsum(un) - un, uf) and un.sum() == n
    for t in range(m):
        ids = plan[t]
        order = np.argsort(picks[t], kind="stable")
        for k in range(topk):
            p = tab["tok_pairs"][t][k]
            assert pe[p] == ids[k] and pt[p] == t
            assert tab["pair_w"][p] == wts[t][order][k]


def _check_tokens(spec, x_np, toks, v, out_f32, want_key, hdr_dev):
    """Oracle on the sampled tokens: every pair's GEMV values and q8_1, then the output."""
    accepted = 0
    tab = v["tab"]
    toks = list(toks)
    ref = olayer.layer_forward(spec, x_np[toks], with_shared=(want_key == "out_f32"))
    shq = spec.shared_quant and want_key == "out_f32"
    topk = spec.shape.topk
    for i, t in enumerate(toks):
        assert np.array_equal(hdr_dev[t], ref["header"][i]), t
        # the token's plan entries: its picks, then (K-quant shared expert) expert n_routed with weight 1
        entries = [(int(e), ref["tok"][i]["experts"][k], k) for k, e in enumerate(ref["tok"][i]["ids"])]
        if shq:
            entries.append((spec.shape.n_routed, ref["shared"][i], topk))
            assert tab["pair_w"][int(tab["tok_pairs"][t][topk])] == 1.0
        else:
            assert tab["tok_pairs"][t][topk] == -1
        for e, ex, k in entries:
            p = int(tab["tok_pairs"][t][k])
            assert tab["pair_expert"][p] == e and tab["pair_tok"][p] == t
            acc = f32_accept(v["g"][p], ex["g"], ex["near_g"], f"g tok {t} e {e}")
            acc += f32_accept(v["u"][p], ex["u"], ex["near_u"], f"u tok {t} e {e}")
            if acc == 0:
                assert np.array_equal(v["h"][p].view(np.uint32), ex["h"].view(np.uint32)), (t, e)
                assert np.array_equal(v["hq"][p], ex["hq"]) and np.array_equal(v["hd"][p], ex["hd16"]), (t, e)
                assert np.array_equal(v["hs"][p], ex["hq"].reshape(-1, 16).astype(np.int32).sum(axis=1))
                acc += f32_accept(v["y"][p], ex["y"], ex["near_y"], f"y tok {t} e {e}")
            else:   # a g/u neighbour: the rest of this pair exactly on the device's own g and u
                sh = spec.shape
                hh = oracle.swiglu(v["g"][p], v["u"][p], sh.swiglu_limit)
                assert np.array_equal(v["h"][p].view(np.uint32), hh.view(np.uint32)), (t, e)
                q, d = oracle.q8_1(hh)
                assert np.array_equal(v["hq"][p], q) and np.array_equal(v["hd"][p], d), (t, e)
                down = (synth.shared_q_blocks(spec, "down") if e == sh.n_routed else
                        synth.expert_blocks(spec, int(e), "down"))
                yy, near = oracle.q3k_gemv(down, sh.dim, sh.inter, q, d)
                acc += f32_accept(v["y"][p], yy, near, f"y tok {t} e {e} (own h)")
            accepted += acc
        want = ref[want_key][i]
        err = np.abs(out_f32[t] - want)
        assert rel_l2(out_f32[t], want) <= 1e-3 and err.max() <= 1e-2, (t, rel_l2(out_f32[t], want), err.max())
    if accepted:
        say(f"  {accepted} GEMV outputs took the other correct rounding next to an f32 midpoint")


def _run_layer(dl, x_np):
    c, shape = dl.cfg, dl.spec.shape
    m = x_np.shape[0]
    x = torch.from_numpy(x_np).cuda()
    ws = workspace(c, m)
    out = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
    out32 = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
    R.layer_forward(c, dl.layer, x, out, ws, out_f32=out32, header=hdr)
    torch.cuda.synchronize()
    return ws, out32.cpu().numpy(), to_np_u16(out), hdr.cpu().numpy()


@pytest.mark.parametrize("m", [9, 37, 512])
def test_prefill_layer_small_shape_every_token(m):
    """dim 512: the oracle checks every token and every pair."""
    dl = dev_layer(TINY, zipf=True)
    spec, c, shape = dl.spec, dl.cfg, dl.spec.shape
    x_np = synth.tokens(spec, 1000, m)
    say(f"prefill layer_forward dim={shape.dim} m={m}")
    ws, out32, outb, hdr = _run_layer(dl, x_np)
    lg = oracle.router_logits(x_np, synth.gate_w(spec))
    L = R.workspace_layout(c, m)
    got_lg = ws_array(ws, L, "logits", np.float32, m * shape.n_routed).reshape(m, -1)
    assert np.array_equal(got_lg.view(np.uint32), lg.view(np.uint32))
    want_hdr, _ = oracle.select(shape, lg, synth.bias(spec))
    assert np.array_equal(hdr, want_hdr)
    v = _ws_views(ws, c, m, shape)
    _check_plan(v["tab"], hdr, m, shape.topk, shape.n_routed)
    _check_tokens(spec, x_np, range(m), v, out32, "out_f32", hdr)
    assert np.array_equal(outb, oracle.f32_to_bf16(out32))
    xq = ws_array(ws, L, "xq", np.int8, m * shape.dim).reshape(m, -1)
    xd = ws_array(ws, L, "xd", np.uint16, m * shape.dim // 32).reshape(m, -1)
    for t in range(0, m, max(1, m // 16)):
        q, d = oracle.q8_1(oracle.bf16_to_f32(x_np[t]))
        assert np.array_equal(xq[t], q) and np.array_equal(xd[t], d)


def test_prefill_full_size_zipf_512():
    """The dim-4096 workload: 512 tokens, Zipf-skewed bias. Headers of all
    tokens bit-exact; the plan's structure checked whole; the oracle checks
    every token's GEMV values, q8_1 codes and output, and the combine bit for
    bit on the device's own expert and shared outputs."""
    dl = dev_layer(DS41, zipf=True)
    spec, c, shape = dl.spec, dl.cfg, dl.spec.shape
    m = 512
    x_np = synth.tokens(spec, 0, m)
    say("prefill layer_forward dim=4096 m=512")
    ws, out32, outb, hdr = _run_layer(dl, x_np)
    lg = oracle.router_logits(x_np, synth.gate_w(spec))
    want_hdr, _ = oracle.select(shape, lg, synth.bias(spec))
    assert np.array_equal(hdr, want_hdr)
    v = _ws_views(ws, c, m, shape)
    _check_plan(v["tab"], hdr, m, shape.topk, shape.n_routed)
    counts = v["tab"]["u_npairs"][:v["tab"]["n_u"]]
    say(f"  {v['tab']['n_u']} experts used, largest group {counts.max()} tokens")
    for t0 in range(0, m, 128):   # in slices, so that the oracle's per-pair results stay small
        say(f"  oracle on tokens {t0}..{t0 + 127}")
        _check_tokens(spec, x_np, range(t0, t0 + 128), v, out32, "out_f32", hdr)
    check_combine_bits(ws, v["L"], v["tab"], m, shape.topk, out32, True)
    assert np.array_equal(outb, oracle.f32_to_bf16(out32))
    assert np.all(np.isfinite(out32))


def test_prefill_equals_decode_path_per_token():
    """Tokens in a 512-token prefill give the decode kernels' values: headers
    and routed GEMV values bitwise, the layer output (shared expert summed
    in another order) within the tolerance."""
    dl = dev_layer(DS41, zipf=True)
    c, shape = dl.cfg, dl.spec.shape
    x_np = synth.tokens(dl.spec, 0, 512)
    ws, out32, _, hdr = _run_layer(dl, x_np)
    v = _ws_views(ws, c, 512, shape)
    for t0, m in ((0, 1), (100, 8)):
        ws_d, out_d, _, hdr_d = _run_layer(dl, x_np[t0:t0 + m].copy())
        assert np.array_equal(hdr_d, hdr[t0:t0 + m])
        vd = _ws_views(ws_d, c, m, shape)
        for t in range(m):
            for k in range(shape.topk):
                p, pd = int(v["tab"]["tok_pairs"][t0 + t][k]), int(vd["tab"]["tok_pairs"][t][k])
                for name in ("g", "u", "y"):
                    a, b = v[name][p], vd[name][pd]
                    d = a.view(np.uint32).astype(np.int64) - b.view(np.uint32).astype(np.int64)
                    assert np.abs(d).max() <= 1, (name, t0 + t, k)   # equal, or both sides of a midpoint
            err = np.abs(out32[t0 + t] - out_d[t])
            assert rel_l2(out32[t0 + t], out_d[t]) <= 1e-3 and err.max() <= 1e-2


def test_prefill_hot_expert_spans_many_chunks():
    """A bias that makes every token pick expert 7: its group holds all m
    tokens (several 16-token passes over its blocks)."""
    dl = dev_layer(TINY)
    spec, c, shape = dl.spec, dl.cfg, dl.spec.shape
    m = 70
    b = synth.bias(spec).copy()
    b[7] = 50.0
    bias_dev = torch.from_numpy(b).cuda()
    layer = R.Layer(dl.gate_w.data_ptr(), bias_dev.data_ptr(), dl.experts, dl.sh_w1.data_ptr(),
                    dl.sh_w3.data_ptr(), dl.sh_w2.data_ptr())
    x_np = synth.tokens(spec, 500, m)
    x = torch.from_numpy(x_np).cuda()
    ws = workspace(c, m)
    out = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
    out32 = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
    R.layer_forward(c, layer, x, out, ws, out_f32=out32, header=hdr)
    torch.cuda.synchronize()
    hdr_np, out_np = hdr.cpu().numpy(), out32.cpu().numpy()
    assert np.all(hdr_np[:, 1] == 7)
    v = _ws_views(ws, c, m, shape)
    tab = v["tab"]
    u7 = list(tab["u_expert"][:tab["n_u"]]).index(7)
    assert tab["u_npairs"][u7] == m
    ref = olayer.layer_forward(spec, x_np, bias=b)
    assert np.array_equal(hdr_np, ref["header"])
    for t in range(m):
        want = ref["out_f32"][t]
        assert rel_l2(out_np[t], want) <= 1e-3 and np.abs(out_np[t] - want).max() <= 1e-2, t
        k = list(ref["tok"][t]["ids"]).index(7)
        p = int(tab["tok_pairs"][t][k])
        ex = ref["tok"][t]["experts"][k]
        f32_accept(v["y"][p], ex["y"], ex["near_y"], f"y tok {t}")


@pytest.mark.parametrize("shape,m", [(TINY, 40), (DS41, 64)])
def test_experts_prefill_matches_oracle(shape, m):
    dl = dev_layer(shape, zipf=True)
    spec, c = dl.spec, dl.cfg
    x_np = synth.tokens(spec, 77, m)
    lg = oracle.router_logits(x_np, synth.gate_w(spec))
    hdr_np, _ = oracle.select(shape, lg, synth.bias(spec))
    ws = workspace(c, m)
    y = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
    say(f"experts_prefill dim={shape.dim} m={m}")
    R.experts_prefill(c, torch.from_numpy(x_np).cuda(), torch.from_numpy(hdr_np).cuda(), dl.experts, y, ws)
    torch.cuda.synchronize()
    v = _ws_views(ws, c, m, shape)
    _check_plan(v["tab"], hdr_np, m, shape.topk, shape.n_routed)
    toks = range(m) if shape == TINY else (0, 5, 31, 63)
    _check_tokens(spec, x_np, toks, v, y.cpu().numpy(), "y_routed", hdr_np)


def test_experts_prefill_rejects_bad_picks():
    dl = dev_layer(TINY)
    spec, c, shape = dl.spec, dl.cfg, dl.spec.shape
    m = 20
    x_np = synth.tokens(spec, 0, m)
    lg = oracle.router_logits(x_np, synth.gate_w(spec))
    hdr_np, _ = oracle.select(shape, lg, synth.bias(spec))
    hdr_np = hdr_np.copy()
    hdr_np[3, 2] = shape.n_routed    # out of range
    hdr_np[11, 4] = hdr_np[11, 1]    # repeated
    hdr_np[19, 1] = -5
    ws = workspace(c, m)
    y = torch.full((m, shape.dim), 7.0, dtype=torch.float32, device="cuda")
    R.experts_prefill(c, torch.from_numpy(x_np).cuda(), torch.from_numpy(hdr_np).cuda(), dl.experts, y, ws)
    torch.cuda.synchronize()
    yy = y.cpu().numpy()
    for t in (3, 11, 19):
        assert np.all(yy[t] == 0), t
    L = R.workspace_layout(c, m)
    assert ws_array(ws, L, "status", np.int32, 1)[0] & R.MOE_STATUS_BAD_PICK
    tab = plan_tables(ws, L, m, shape.topk)
    assert tab["n_pairs"] == (m - 3) * shape.topk
    ref = olayer.layer_forward(spec, x_np[[0, 12]], with_shared=False)
    for i, t in enumerate((0, 12)):
        assert rel_l2(yy[t], ref["y_routed"][i]) < 1e-6


@pytest.mark.parametrize("m", [24])
def test_stack_forward_prefill(m):
    """Three small layers at m = 24 through the prefill kernels, teacher-forced."""
    n = 3
    specs = [synth.LayerSpec(TINY, seed=9, layer=l) for l in range(n)]
    dls = [DeviceLayer(sp) for sp in specs]
    c = dls[0].cfg
    x0 = synth.tokens(specs[0], 3, m)
    xs = torch.empty((n + 1, m, TINY.dim), dtype=torch.uint16, device="cuda")
    xs[0] = torch.from_numpy(x0).cuda()
    out = torch.empty((n, m, TINY.dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((n, m, R.header_words(c)), dtype=torch.int32, device="cuda")
    ws = workspace(c, m)
    R.stack_forward(c, [d.layer for d in dls], xs, ws, out_f32=out, headers=hdr)
    torch.cuda.synchronize()
    xs_np, out_np, hdr_np = to_np_u16(xs), out.cpu().numpy(), hdr.cpu().numpy()
    for l in range(n):
        ref = olayer.layer_forward(specs[l], xs_np[l], keep_experts=False)
        assert np.array_equal(hdr_np[l], ref["header"]), l
        for t in range(m):
            assert rel_l2(out_np[l, t], ref["out_f32"][t]) <= 1e-3
            assert np.abs(out_np[l, t] - ref["out_f32"][t]).max() <= 1e-2
        assert np.array_equal(xs_np[l + 1], olayer.residual(xs_np[l], out_np[l])), l


@pytest.mark.parametrize("shape", [synth.Shape(dim=1024, inter=512), DS41], ids=lambda s: f"{s.dim}x{s.inter}")
def test_prefill_group_sizes_at_the_kernel_split(shape):
    """Experts with at most 8 pairs run in the small-group gate/up and down
    kernels, the others in the 16-token-pass kernels. Rows repeated 8, 9 and
    16 times (shuffled) give every expert of a row at least that many pairs:
    groups of exactly 8, 9 and 16 when the rows' picks are disjoint, and of
    17 or more (a 16-token pass and a remainder) where they overlap. Equal
    rows must give equal results; each distinct row is checked against the
    oracle (every pair's GEMV values and the layer output)."""
    dl = dev_layer(shape, seed=3)
    spec, c = dl.spec, dl.cfg
    rows = synth.tokens(spec, 900, 3)
    reps = np.repeat(np.arange(3), [8, 9, 16])
    perm = np.random.default_rng(5).permutation(len(reps))
    which = reps[perm]
    x_np = rows[which]
    m = len(which)
    say(f"prefill group sizes dim={shape.dim} m={m}")
    ws, out32, _, hdr = _run_layer(dl, x_np)
    v = _ws_views(ws, c, m, shape)
    tab = v["tab"]
    sizes = sorted(int(n) for n in tab["u_npairs"][:tab["n_u"]])
    say(f"  group sizes {sizes}")
    assert max(sizes) >= 16 and min(sizes) >= 8 and any(n <= 8 for n in sizes) and any(n > 8 for n in sizes)
    first = [int(np.flatnonzero(which == r)[0]) for r in range(3)]
    ref = olayer.layer_forward(spec, rows)
    for r, t0 in enumerate(first):
        assert np.array_equal(hdr[t0], ref["header"][r])
        for t in np.flatnonzero(which == r):
            assert np.array_equal(out32[t].view(np.uint32), out32[t0].view(np.uint32)), (r, t)
            assert np.array_equal(hdr[t], hdr[t0])
        for k, e in enumerate(ref["tok"][r]["ids"]):
            p = int(tab["tok_pairs"][t0][k])
            ex = ref["tok"][r]["experts"][k]
            f32_accept(v["g"][p], ex["g"], ex["near_g"], f"g row {r} e {e}")
            f32_accept(v["u"][p], ex["u"], ex["near_u"], f"u row {r} e {e}")
            f32_accept(v["y"][p], ex["y"], ex["near_y"], f"y row {r} e {e}")
        want = ref["out_f32"][r]
        assert rel_l2(out32[t0], want) <= 1e-3 and np.abs(out32[t0] - want).max() <= 1e-2, r


def test_prefill_graph_capture_replays_equal_eager():
    """Prefill forks work onto the library's second stream (the shared expert
    from the start, the experts with more than 8 pairs after the grouping) and
    joins before the combine. Captured in a graph on the caller's stream, the
    fork and join come along: three replays, with eager work and
    synchronisation between them, each give the eager output bit for bit."""
    shape = synth.Shape(dim=1024, inter=512)
    dl = dev_layer(shape, seed=3)
    c = dl.cfg
    m = 40
    x = torch.from_numpy(synth.tokens(dl.spec, 300, m)).cuda()
    ws = workspace(c, m)
    out = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
    out32 = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
    R.layer_forward(c, dl.layer, x, out, ws, out_f32=out32, header=hdr)
    torch.cuda.synchronize()
    ref32, refh = out32.clone(), hdr.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        R.layer_forward(c, dl.layer, x, out, ws, out_f32=out32, header=hdr, stream=s.cuda_stream)
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            R.layer_forward(c, dl.layer, x, out, ws, out_f32=out32, header=hdr, stream=s.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(3):
        out32.fill_(0.0)
        hdr.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out32.view(torch.int32), ref32.view(torch.int32)), rep
        assert torch.equal(hdr, refh), rep


def _device_tokens(spec, m):
    """Input rows 0..m-1 of the layer's token recipe, generated on the device."""
    from synth.device import tokens_into
    x = torch.empty((m, spec.shape.dim), dtype=torch.uint16, device="cuda")
    tokens_into(spec, x)
    torch.cuda.synchronize()
    return x


@pytest.mark.parametrize("shape,shared_quant", [(DS41, False), (TINY, True)],
                         ids=lambda v: f"dim{v.dim}" if hasattr(v, "dim") else f"kquant{int(v)}")
def test_prefill_maximum_token_count(shape, shared_quant):
    """The largest accepted batch, 65535 tokens (the combine's grid rows;
    at dim 4096 the prefill kernels' 32-bit offsets reach 1.9e9), through
    moe_layer_forward: every header valid (picks distinct and in range,
    ascending plan, weights summing to route_scale), every bf16 output the
    rounding of its f32 output, and sampled tokens across the batch (both
    ends included) bit-exact in the header and within tolerance in the output
    against the oracle."""
    m = 65535
    if shape == DS41:
        dl = dev_layer(DS41, zipf=True)
    else:
        dl = DeviceLayer(synth.LayerSpec(shape, seed=9, zipf_bias=True, shared_quant=shared_quant))
    spec, c = dl.spec, dl.cfg
    k = shape.topk
    say(f"prefill at the maximum token count: dim {shape.dim}, m={m}, shared_quant={shared_quant}")
    x = _device_tokens(spec, m)
    ws = workspace(c, m)
    out = torch.empty((m, shape.dim), dtype=torch.uint16, device="cuda")
    out32 = torch.empty((m, shape.dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
    R.layer_forward(c, dl.layer, x, out, ws, out_f32=out32, header=hdr)
    torch.cuda.synchronize()
    del ws
    h = hdr.cpu().numpy()
    st, picks, wts, plan = oracle.header_fields(h, k)
    assert np.all(st == 0)
    assert np.all((picks >= 0) & (picks < shape.n_routed))
    assert np.all(np.sort(picks, axis=1) == plan) and np.all(np.diff(plan, axis=1) > 0)
    assert np.all(np.abs(wts.astype(np.float64).sum(axis=1) - shape.route_scale) <= 1e-5)
    for t0 in range(0, m, 8192):   # the bf16 output is the rounding of the f32 output, every token
        o32 = out32[t0:t0 + 8192].cpu().numpy()
        assert np.all(np.isfinite(o32))
        assert np.array_equal(to_np_u16(out[t0:t0 + 8192]), oracle.f32_to_bf16(o32))
    toks = [0, 1, 4097, 32767, 65533, 65534]
    x_np = np.concatenate([synth.tokens(spec, t, 1) for t in toks])
    assert np.array_equal(to_np_u16(x.view(torch.int16)[toks]), x_np)
    ref = olayer.layer_forward(spec, x_np)
    o32 = out32[toks].cpu().numpy()
    for i, t in enumerate(toks):
        assert np.array_equal(h[t], ref["header"][i]), t
        assert rel_l2(o32[i], ref["out_f32"][i]) <= 1e-3 and np.abs(o32[i] - ref["out_f32"][i]).max() <= 1e-2, t

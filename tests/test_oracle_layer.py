"""Oracle pins: K-quant GEMV values, SwiGLU, combine and the whole layer.

The GEMV is pinned against exact rational arithmetic on densely generated
weights (packed by the independent packer), the layer against special
cases that reduce to a textbook dense MLP."""
from fractions import Fraction

import mpmath
import numpy as np

import oracle
import synth
from oracle import layer
from tests._exact import f16_bits, fp16_fraction, pack_q2k, pack_q3k, round_to_f32

RNG = np.random.default_rng(99)


def _rand_q2k_rows(rows, nsb):
    dense = []
    blocks = []
    for r in range(rows):
        row_b, row_w = [], []
        for b in range(nsb):
            codes = RNG.integers(0, 4, 256)
            sc, mn = RNG.integers(0, 16, 16), RNG.integers(0, 16, 16)
            d = f16_bits(float(RNG.uniform(1e-3, 1e-2)))
            dm = f16_bits(float(RNG.uniform(1e-3, 1e-2)))
            row_b.append(pack_q2k(codes, sc, mn, d, dm))
            fd, fm = fp16_fraction(d), fp16_fraction(dm)
            row_w += [fd * int(sc[i // 16]) * int(codes[i]) - fm * int(mn[i // 16]) for i in range(256)]
        blocks.append(np.concatenate(row_b))
        dense.append(row_w)
    return np.stack(blocks), dense


def _rand_q3k_rows(rows, nsb):
    dense, blocks = [], []
    for r in range(rows):
        row_b, row_w = [], []
        for b in range(nsb):
            vals = RNG.integers(-4, 4, 256)
            sc = RNG.integers(0, 64, 16)
            d = f16_bits(float(RNG.uniform(1e-3, 1e-2)))
            row_b.append(pack_q3k(vals, sc, d))
            fd = fp16_fraction(d)
            row_w += [fd * (int(sc[i // 16]) - 32) * int(vals[i]) for i in range(256)]
        blocks.append(np.concatenate(row_b))
        dense.append(row_w)
    return np.stack(blocks), dense


def _rand_act(cols):
    x = RNG.normal(0, 1, cols).astype(np.float32)
    q, d16 = oracle.q8_1(x)
    act = [fp16_fraction(int(d16[k // 32])) * int(q[k]) for k in range(cols)]
    return q, d16, act


def test_q2k_gemv_is_rounded_exact_dot():
    for nsb in (1, 2):
        blocks, dense = _rand_q2k_rows(6, nsb)
        q, d16, act = _rand_act(256 * nsb)
        y, near = oracle.q2k_gemv(blocks, 6, 256 * nsb, q, d16)
        for r in range(6):
            exact = sum(wv * av for wv, av in zip(dense[r], act))
            assert y[r] == round_to_f32(exact), (nsb, r)


def test_q3k_gemv_is_rounded_exact_dot():
    for nsb in (1, 2):
        blocks, dense = _rand_q3k_rows(6, nsb)
        q, d16, act = _rand_act(256 * nsb)
        y, near = oracle.q3k_gemv(blocks, 6, 256 * nsb, q, d16)
        for r in range(6):
            exact = sum(wv * av for wv, av in zip(dense[r], act))
            assert y[r] == round_to_f32(exact), (nsb, r)


def test_gemv_one_hot_activation_reads_one_column():
    """x = 127 at position k, zero elsewhere: d = 1 for k's block, 0 for the
    rest, so y = 127 * W[:, k] (exact, rounded once)."""
    blocks, dense = _rand_q2k_rows(4, 2)
    for k in (0, 17, 255, 256, 300, 511):
        x = np.zeros(512, np.float32)
        x[k] = 127.0
        q, d16 = oracle.q8_1(x)
        y, _ = oracle.q2k_gemv(blocks, 4, 512, q, d16)
        for r in range(4):
            assert y[r] == round_to_f32(127 * dense[r][k])


def test_gemv_f64_dense_agrees_with_exact():
    """An independent float64 dense matvec of the dequantised matrix agrees
    with the exact GEMV to float64 accuracy (catches a transposed operand)."""
    spec = synth.LayerSpec(synth.SHAPE_TINY, seed=3)
    gate = synth.expert_blocks(spec, 5, "gate")
    down = synth.expert_blocks(spec, 5, "down")
    x = oracle.bf16_to_f32(synth.tokens(spec, 0, 1)[0])
    q, d16 = oracle.q8_1(x)
    a = q.astype(np.float64) * np.repeat(oracle.fp16_to_f64(d16), 32)
    W = oracle.q2k_dequant(gate).reshape(256, 512)
    y, near = oracle.q2k_gemv(gate, 256, 512, q, d16)
    ref = W @ a
    assert np.all(np.abs(y - ref) <= np.abs(ref) * 2.0 ** -23 + 1e-12)
    assert near.sum() == 0
    h = RNG.normal(0, 3, 256).astype(np.float32)
    hq, hd = oracle.q8_1(h)
    ha = hq.astype(np.float64) * np.repeat(oracle.fp16_to_f64(hd), 32)
    W2 = oracle.q3k_dequant(down).reshape(512, 256)
    y2, _ = oracle.q3k_gemv(down, 512, 256, hq, hd)
    ref2 = W2 @ ha
    assert np.all(np.abs(y2 - ref2) <= np.abs(ref2) * 2.0 ** -23 + 1e-12)


def test_gemv_zero_scales_give_zero():
    codes = RNG.integers(0, 4, 256)
    blk = pack_q2k(codes, RNG.integers(0, 16, 16), RNG.integers(0, 16, 16), 0, 0)
    q, d16 = oracle.q8_1(RNG.normal(0, 1, 256).astype(np.float32))
    y, _ = oracle.q2k_gemv(blk, 1, 256, q, d16)
    assert y[0] == 0.0


# ----------------------------------------------------------------- SwiGLU
def _exp_cr(x):
    with mpmath.workprec(200):
        man, e = mpmath.exp(mpmath.mpf(float(x))).man_exp
        return round_to_f32(Fraction(int(man)) * Fraction(2) ** int(e))


def test_swiglu_special_cases():
    L = np.float32(7.0)
    silu_L = np.float32(L / np.float32(np.float32(1.0) + _exp_cr(-7.0)))
    u = RNG.normal(0, 4, 200).astype(np.float32)
    # gate at or above the limit: silu(L) * clamp(u)
    g = np.full(200, 9.0, np.float32)
    got = oracle.swiglu(g, u, 7.0)
    assert np.array_equal(got, (silu_L * np.clip(u, -L, L)).astype(np.float32))
    # zero gate -> 0
    assert np.all(oracle.swiglu(np.zeros(200, np.float32), u, 7.0) == 0.0)
    # up beyond the limit clamps to +-L
    g = RNG.normal(0, 2, 200).astype(np.float32)
    big = np.where(RNG.random(200) < 0.5, 50.0, -50.0).astype(np.float32)
    got = oracle.swiglu(g, big, 7.0)
    for gi, bi, h in zip(g, big, got):
        zg = min(gi, L)
        s = np.float32(zg / np.float32(np.float32(1.0) + _exp_cr(-zg)))
        assert h == np.float32(s * np.float32(np.sign(bi) * L))
    # very negative gate: exp overflows, silu -> -0
    assert oracle.swiglu(np.array([-200.0], np.float32), np.array([1.0], np.float32), 7.0)[0] == 0.0


# ----------------------------------------------------------------- layer
def test_layer_with_zero_experts_is_the_dense_shared_mlp():
    """Routed scales all zero -> y = 0, so out = shared MLP, which is checked
    against a float64 textbook MLP (W2 @ bf16(silu(W1 x) * W3 x))."""
    spec = synth.LayerSpec(synth.SHAPE_TINY, seed=11)
    s = spec.shape

    def zero_experts(e):
        g = synth.expert_blocks(spec, e, "gate").copy()
        u = synth.expert_blocks(spec, e, "up").copy()
        d = synth.expert_blocks(spec, e, "down").copy()
        for arr, nbytes, offs in ((g, 84, (80, 81, 82, 83)), (u, 84, (80, 81, 82, 83)), (d, 110, (108, 109))):
            v = arr.reshape(-1, nbytes)
            for o in offs:
                v[:, o] = 0
        return g, u, d

    x = synth.tokens(spec, 0, 2)
    out = layer.layer_forward(spec, x, experts=zero_experts)
    assert np.all(out["y_routed"] == 0.0)
    w1, w3, w2 = (oracle.bf16_to_f32(synth.shared_w(spec, w)).astype(np.float64) for w in ("w1", "w3", "w2"))
    for t in range(2):
        xf = oracle.bf16_to_f32(x[t]).astype(np.float64)
        g, u = w1 @ xf, w3 @ xf
        L = 7.0
        gz = np.minimum(g, L)
        h = gz / (1 + np.exp(-gz)) * np.clip(u, -L, L)
        h16 = oracle.bf16_to_f32(oracle.f32_to_bf16(h.astype(np.float32))).astype(np.float64)
        ref = w2 @ h16
        err = np.abs(out["out_f32"][t] - ref)
        assert np.sqrt((err ** 2).sum() / (ref ** 2).sum()) < 1e-3
        assert err.max() < 1e-2


def test_layer_with_identical_experts_sums_the_weights():
    spec = synth.LayerSpec(synth.SHAPE_TINY, seed=12)
    same = tuple(synth.expert_blocks(spec, 0, w) for w in ("gate", "up", "down"))
    x = synth.tokens(spec, 0, 1)
    out = layer.layer_forward(spec, x, experts=lambda e: same, with_shared=False)
    y = out["tok"][0]["experts"][0]["y"].astype(np.float64)
    wsum = out["tok"][0]["w_plan"].astype(np.float64).sum()
    assert abs(wsum - 2.5) < 1e-5
    assert np.allclose(out["y_routed"][0], wsum * y, rtol=1e-5, atol=1e-4)
    # bf16 output is the RNE rounding of the f32 output
    assert np.array_equal(out["out_bf16"][0], oracle.f32_to_bf16(out["out_f32"][0]))


def test_plan_weights_are_pick_weights_in_id_order():
    spec = synth.LayerSpec(synth.SHAPE_TINY, seed=13)
    x = synth.tokens(spec, 0, 3)
    r = layer.route(spec, x)
    _, picks, w, plan = oracle.header_fields(r["header"], 6)
    for t in range(3):
        m = dict(zip(picks[t], w[t]))
        assert list(plan[t]) == sorted(picks[t])
        assert [m[e] for e in plan[t]] == [m[e] for e in sorted(picks[t])]


# ----------------------------------------------------------------- stack
def _zeroed_experts(spec):
    def experts(e):
        g = synth.expert_blocks(spec, e, "gate").copy()
        u = synth.expert_blocks(spec, e, "up").copy()
        d = synth.expert_blocks(spec, e, "down").copy()
        for arr, nbytes, offs in ((g, 84, (80, 81, 82, 83)), (u, 84, (80, 81, 82, 83)), (d, 110, (108, 109))):
            v = arr.reshape(-1, nbytes)
            for o in offs:
                v[:, o] = 0
        return g, u, d
    return experts


def test_stack_of_zero_layers_is_the_identity():
    """Layers whose routed and shared weights are all zero add +0 to the
    residual stream: every x_l equals x_0 bit for bit (bf16(x + 0) = x)."""
    specs = [synth.LayerSpec(synth.SHAPE_TINY, seed=21, layer=l) for l in range(3)]
    s = specs[0].shape
    zero_sh = (np.zeros((s.inter, s.dim), np.uint16), np.zeros((s.inter, s.dim), np.uint16),
               np.zeros((s.dim, s.inter), np.uint16))
    kw = [{"experts": _zeroed_experts(sp), "shared_w": zero_sh} for sp in specs]
    x0 = synth.tokens(specs[0], 0, 2)
    r = layer.stack_forward(specs, x0, layer_kwargs=kw)
    assert np.all(r["out_f32"] == 0.0)
    for l in range(4):
        assert np.array_equal(r["xs"][l], x0)


def test_stack_residual_against_exact_sums():
    """x_{l+1} is the bf16 rounding of the exact sum x_l + out_l (an f32 add
    is exact before its rounding here: both are finite and the sum is
    rounded once to f32, then once to bf16), and layer l routes on x_l."""
    specs = [synth.LayerSpec(synth.SHAPE_TINY, seed=22, layer=l) for l in range(3)]
    x0 = synth.tokens(specs[0], 0, 1)
    r = layer.stack_forward(specs, x0)
    for l in range(3):
        xf = oracle.bf16_to_f32(r["xs"][l]).astype(np.float64)
        exact = xf + r["out_f32"][l].astype(np.float64)
        f32 = exact.astype(np.float32)          # one rounding of the exact sum
        assert np.array_equal(r["xs"][l + 1], oracle.f32_to_bf16(f32))
        hdr = layer.route(specs[l], r["xs"][l])["header"]
        assert np.array_equal(r["headers"][l], hdr)
    # the layers differ (their own seeds): the step is not one layer repeated
    assert not np.array_equal(r["headers"][0], r["headers"][1])


# ------------------------------------------------ K-quant shared expert
# The shared expert's matrices as K-quant blocks run exactly as one more
# routed expert of the token, added after the routed sum [moe_v41.rs, struct
# MoeV41LayerWeights: the shared matrices as bf16 or the GGUF's Q2_K (w1, w3)
# / Q3_K (w2) blocks on the routed experts' kernels; fn shared_side].
def _kq_spec(seed):
    return synth.LayerSpec(synth.SHAPE_TINY, seed=seed, shared_quant=True)


def _zero_scales(g, u, d):
    g, u, d = g.copy(), u.copy(), d.copy()
    for arr, nbytes, offs in ((g, 84, (80, 81, 82, 83)), (u, 84, (80, 81, 82, 83)), (d, 110, (108, 109))):
        v = arr.reshape(-1, nbytes)
        for o in offs:
            v[:, o] = 0
    return g, u, d


def test_kquant_shared_with_zero_scales_adds_nothing():
    """All-zero shared scales: its output is +0 everywhere, so the layer
    output is the routed sum bit for bit (acc + 0 = acc)."""
    spec = _kq_spec(31)
    zq = _zero_scales(*(synth.shared_q_blocks(spec, w) for w in ("gate", "up", "down")))
    x = synth.tokens(spec, 0, 3)
    out = layer.layer_forward(spec, x, shared_q=zq)
    assert np.array_equal(out["out_f32"].view(np.uint32), out["y_routed"].view(np.uint32))
    assert all(np.all(sh["y"] == 0.0) for sh in out["shared"])


def test_kquant_shared_equal_to_a_picked_expert_gives_its_output():
    """Shared blocks equal to the blocks of an expert the token picked: the
    shared output equals that expert's output bit for bit (same q8_1 of x,
    same GEMVs, same SwiGLU and q8_1 of h)."""
    spec = _kq_spec(32)
    x = synth.tokens(spec, 5, 1)
    e = int(layer.route(spec, x)["header"][0, 1])
    same = tuple(synth.expert_blocks(spec, e, w) for w in ("gate", "up", "down"))
    out = layer.layer_forward(spec, x, shared_q=same)
    k = list(out["tok"][0]["ids"]).index(e)
    ye = out["tok"][0]["experts"][k]["y"]
    assert np.array_equal(out["shared"][0]["y"].view(np.uint32), ye.view(np.uint32))


def test_kquant_shared_alone_is_the_dense_quantised_mlp():
    """Routed scales all zero: the layer output is the shared expert alone,
    checked against a float64 textbook MLP on the dequantised matrices and
    the dequantised q8_1 activations (W2 . deq(q8_1(silu(min(g,L)) clamp(u))),
    g, u = W1 . deq(q8_1(x)), W3 . deq(q8_1(x)))."""
    spec = _kq_spec(33)
    s = spec.shape

    def zero_experts(e):
        return _zero_scales(*(synth.expert_blocks(spec, e, w) for w in ("gate", "up", "down")))

    x = synth.tokens(spec, 0, 2)
    out = layer.layer_forward(spec, x, experts=zero_experts)
    assert np.all(out["y_routed"] == 0.0)
    W1 = oracle.q2k_dequant(synth.shared_q_blocks(spec, "gate")).reshape(s.inter, s.dim)
    W3 = oracle.q2k_dequant(synth.shared_q_blocks(spec, "up")).reshape(s.inter, s.dim)
    W2 = oracle.q3k_dequant(synth.shared_q_blocks(spec, "down")).reshape(s.dim, s.inter)
    L = 7.0
    for t in range(2):
        q, d = oracle.q8_1(oracle.bf16_to_f32(x[t]))
        a = q.astype(np.float64) * np.repeat(oracle.fp16_to_f64(d), 32)
        g, u = (W1 @ a).astype(np.float32), (W3 @ a).astype(np.float32)
        gz = np.minimum(g.astype(np.float64), L)
        h = (gz / (1 + np.exp(-gz)) * np.clip(u.astype(np.float64), -L, L)).astype(np.float32)
        hq, hd = oracle.q8_1(h)
        ha = hq.astype(np.float64) * np.repeat(oracle.fp16_to_f64(hd), 32)
        ref = W2 @ ha
        got = out["out_f32"][t].astype(np.float64)
        # (on these inputs the textbook h quantises to the same codes as the f32 chain's: only rounding differs)
        assert np.array_equal(hq, out["shared"][t]["hq"])
        assert np.sqrt(((got - ref) ** 2).sum() / (ref ** 2).sum()) < 1e-6
        assert np.abs(got - ref).max() < 1e-4

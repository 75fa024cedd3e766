"""Oracle pins: router logits, selection (ranking, weights, header, plan).

The selection is pinned against a brute-force rank-by-counting and closed
forms of the weights; the router against exact sums (integers, or float64 of
exact products with a rigorous f32 error bound)."""
import dataclasses

import numpy as np

import oracle
import synth

RNG = np.random.default_rng(7)
SH = synth.SHAPE_TINY


def _bf16(v):
    return oracle.f32_to_bf16(np.asarray(v, np.float32))


# ---------------------------------------------------------------- router
def test_router_exact_on_integer_data():
    """Small integers: every partial sum is exact in f32, so any order of
    summation gives the exact dot product; a dropped or doubled position
    would show."""
    for dim in (256, 512, 1024, 4096):
        x = RNG.integers(-8, 9, (3, dim)).astype(np.float32)
        w = RNG.integers(-8, 9, (10, dim)).astype(np.float32)
        got = oracle.router_logits(_bf16(x), _bf16(w))
        want = x.astype(np.int64) @ w.astype(np.int64).T
        assert np.array_equal(got, want.astype(np.float32)), dim


def test_router_error_bound_against_exact_sum():
    """f32 recursive summation error: |got - exact| <= gamma_n * sum|p| with
    n = the longest chain of additions (dim/64 sequential + 6 pairwise)."""
    dim = 4096
    x = _bf16(RNG.normal(0, 1, (4, dim)))
    w = _bf16(RNG.normal(0, 0.02, (384, dim)))
    got = oracle.router_logits(x, w).astype(np.float64)
    xf, wf = oracle.bf16_to_f32(x).astype(np.float64), oracle.bf16_to_f32(w).astype(np.float64)
    prod = xf[:, None, :] * wf[None, :, :]             # exact in float64
    exact = prod.sum(axis=2)                           # float64 error ~1e-16 relative, negligible here
    n = dim // 64 + 6
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    bound = gamma * np.abs(prod).sum(axis=2)
    assert np.all(np.abs(got - exact) <= bound + 1e-30)


def test_router_rows_independent_of_batch():
    dim = 512
    x = _bf16(RNG.normal(0, 1, (8, dim)))
    w = _bf16(RNG.normal(0, 0.02, (384, dim)))
    batch = oracle.router_logits(x, w)
    for t in range(8):
        assert np.array_equal(batch[t], oracle.router_logits(x[t:t + 1], w)[0])


# ------------------------------------------------------------- selection
def _brute_force_picks(key, k):
    """Rank by counting: rank(e) = #{keys strictly greater} + #{lower ids with an equal key}."""
    n = len(key)
    rank = np.empty(n, int)
    for e in range(n):
        rank[e] = np.sum(key > key[e]) + np.sum((key == key[e]) & (np.arange(n) < e))
    return [int(np.nonzero(rank == r)[0][0]) for r in range(k)]


def test_picks_match_brute_force_rank():
    for trial in range(40):
        logits = RNG.normal(0, 1.3, (1, 384)).astype(np.float32)
        bias = RNG.uniform(-0.1, 0.1, 384).astype(np.float32)
        if trial % 4 == 0:                     # forced ties
            logits[0, ::7] = logits[0, 3]
            bias[::7] = bias[3]
        hdr, sc = oracle.select(SH, logits, bias)
        status, picks, wts, plan = oracle.header_fields(hdr, 6)
        key = (sc[0] + bias).astype(np.float32)
        assert list(picks[0]) == _brute_force_picks(key, 6)
        assert list(plan[0]) == sorted(picks[0])
        assert status[0] == 0


def test_tied_keys_pick_ascending_ids():
    logits = np.zeros((1, 384), np.float32)
    bias = np.zeros(384, np.float32)
    hdr, _ = oracle.select(SH, logits, bias)
    assert list(oracle.header_fields(hdr, 6)[1][0]) == [0, 1, 2, 3, 4, 5]
    bias[[200, 100, 300]] = 0.5                # three winners, then the tie at ids 0..2
    hdr, _ = oracle.select(SH, logits, bias)
    assert list(oracle.header_fields(hdr, 6)[1][0]) == [100, 200, 300, 0, 1, 2]


def test_signed_zero_keys_compare_equal():
    logits = np.full((1, 384), -1000.0, np.float32)    # scores are +0
    bias = np.zeros(384, np.float32)
    bias[5] = -0.0
    bias[10:] = -1.0
    hdr, _ = oracle.select(SH, logits, bias)
    assert list(oracle.header_fields(hdr, 6)[1][0]) == [0, 1, 2, 3, 4, 5]


def test_weights_sum_to_route_scale():
    for _ in range(50):
        logits = RNG.normal(0, 1.3, (1, 384)).astype(np.float32)
        bias = RNG.uniform(-0.1, 0.1, 384).astype(np.float32)
        hdr, _ = oracle.select(SH, logits, bias)
        w = oracle.header_fields(hdr, 6)[2][0].astype(np.float64)
        assert abs(w.sum() - 2.5) <= 8 * np.spacing(np.float32(2.5))
        assert np.all(w > 0)


def test_weights_closed_form_equal_scores():
    logits = np.full((1, 384), 0.3, np.float32)
    bias = np.zeros(384, np.float32)
    hdr, sc = oracle.select(SH, logits, bias)
    s = sc[0, 0]
    six = np.float32(np.float32(np.float32(np.float32(np.float32(np.float32(s + s) + s) + s) + s) + s))
    tot = np.float32(six + np.float32(1e-20))
    want = np.float32(np.float32(s / tot) * np.float32(2.5))
    w = oracle.header_fields(hdr, 6)[2][0]
    assert np.all(w == want)


def test_weights_without_renormalisation():
    sh = dataclasses.replace(SH, norm_topk_prob=False)
    logits = RNG.normal(0, 1.3, (1, 384)).astype(np.float32)
    bias = RNG.uniform(-0.1, 0.1, 384).astype(np.float32)
    hdr, sc = oracle.select(sh, logits, bias)
    _, picks, w, _ = oracle.header_fields(hdr, 6)
    assert np.array_equal(w[0], (sc[0, picks[0]] * np.float32(2.5)).astype(np.float32))
    # topk = 1 never renormalises either
    sh1 = dataclasses.replace(SH, topk=1)
    hdr1, sc1 = oracle.select(sh1, logits, bias)
    _, p1, w1, _ = oracle.header_fields(hdr1, 1)
    assert w1[0, 0] == np.float32(sc1[0, p1[0, 0]] * np.float32(2.5))


def test_nan_key_sets_status_bit():
    logits = RNG.normal(0, 1.3, (2, 384)).astype(np.float32)
    logits[1, 17] = np.nan
    bias = RNG.uniform(-0.1, 0.1, 384).astype(np.float32)
    hdr, _ = oracle.select(SH, logits, bias)
    status, picks, _, _ = oracle.header_fields(hdr, 6)
    assert status[0] == 0 and status[1] == 2
    assert 17 not in picks[1]


def test_header_layout_words():
    logits = RNG.normal(0, 1.3, (3, 384)).astype(np.float32)
    bias = RNG.uniform(-0.1, 0.1, 384).astype(np.float32)
    hdr, _ = oracle.select(SH, logits, bias)
    assert hdr.shape == (3, 19)
    for t in range(3):
        picks = hdr[t, 1:7]
        assert len(set(picks)) == 6 and np.all((picks >= 0) & (picks < 384))
        assert np.array_equal(hdr[t, 13:19], np.sort(picks))


# ------------------------------------------------- router summation order
# The reading of the strict-order router [moe_v41.rs, Kernels: router_gemv]:
# lane l of a wave64 sums the products at k = 512*i + 8*l + j in f32, i-major
# then j-minor; the 64 partials then combine by p[l] += p[l ^ s] for
# s = 32, 16, 8, 4, 2, 1, and the logit is p[0]. Every bf16 x bf16 product is
# exact in f32, so only this order decides the rounding. The rows below put
# products of +-2^24 and 1 where only that order gives the value written next
# to them (2^24 + 1 rounds to 2^24: a tie, to even). The exact sum of every
# row is 1, so a plain sum, or any of the orders that the mutants below
# implement, gives something else.
def _order_pin_inputs(dim=1024):
    P = 2.0 ** 12
    x = np.zeros((1, dim), np.float32)
    x[0, 0], x[0, 1], x[0, 8], x[0, 256], x[0, 512] = P, 1.0, 1.0, P, P
    w = np.zeros((4, dim), np.float32)
    # row 0: lane 0 holds 2^24, lane 1 holds 1, lane 32 holds -2^24. The s = 32 step first cancels lanes 0
    # and 32 (p0 = 0, p1 = 1), the s = 1 step then gives 1.
    w[0, 0], w[0, 8], w[0, 256] = P, 1.0, -P
    # row 1: k = 0 and k = 1 are both lane 0's (8 consecutive k per lane): 2^24 + 1 = 2^24 there; lane 1
    # holds -2^24 (k = 8 = 8*1 + 0): the tree gives 0.
    w[1, 0], w[1, 1], w[1, 8] = P, 1.0, -(2.0 ** 24)
    # row 2: lane 0 holds k = 0, 1 (i = 0) and k = 512 (i = 1): i-major sums 2^24, +1 (absorbed), -2^24 = 0.
    w[2, 0], w[2, 1], w[2, 512] = P, 1.0, -P
    # row 3: all zero
    return _bf16(x), _bf16(w), np.array([1.0, 0.0, 0.0, 0.0], np.float32)


def _logits_in_order(x, w, lane_of, seq_key, tree):
    """A mutant router (f32 throughout): products grouped per lane by lane_of(k), each lane's products
    summed in the order of seq_key(k), then the 64 lane partials combined by `tree`."""
    xf, wf = oracle.bf16_to_f32(x)[0], oracle.bf16_to_f32(w)
    out = []
    for row in wf:
        lanes = [np.float32(0.0)] * 64
        for k in sorted(range(len(row)), key=seq_key):
            lanes[lane_of(k)] = np.float32(lanes[lane_of(k)] + np.float32(xf[k] * row[k]))
        out.append(tree(lanes))
    return np.array(out, np.float32)


def _tree(steps):
    def comb(p):
        p = list(p)
        for s in steps:
            p = [np.float32(p[l] + p[l ^ s]) for l in range(64)]
        return p[0]
    return comb


def test_router_order_pins_hand_built_rows():
    x, w, want = _order_pin_inputs()
    got = oracle.router_logits(x, w)[0]
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # the exact sums are all 1 (rows 0..2): the order, not the data, decides these values
    xf, wf = oracle.bf16_to_f32(x)[0].astype(np.float64), oracle.bf16_to_f32(w).astype(np.float64)
    assert list(wf[:3] @ xf) == [1.0, 1.0, 1.0]


def test_router_order_pins_reject_mutant_orders():
    """Each plausible slip in the stated order fails at least one pinned row:
    the pins are able to tell them apart from the stated order."""
    x, w, want = _order_pin_inputs()
    dim = x.shape[1]
    stated_lane = lambda k: (k % 512) // 8
    i_major = lambda k: k
    j_major = lambda k: (k % 8, k)
    mutants = {
        "butterfly s = 1 .. 32": _logits_in_order(x, w, stated_lane, i_major, _tree([1, 2, 4, 8, 16, 32])),
        "j-major inside a lane": _logits_in_order(x, w, stated_lane, j_major, _tree([32, 16, 8, 4, 2, 1])),
        "lane l takes k = l + 64 j": _logits_in_order(x, w, lambda k: k % 64, i_major, _tree([32, 16, 8, 4, 2, 1])),
        "one sequential sum": np.array([np.float32(sum_seq) for sum_seq in (
            _seq_sum(oracle.bf16_to_f32(x)[0], oracle.bf16_to_f32(w)[r]) for r in range(4))], np.float32),
    }
    stated = _logits_in_order(x, w, stated_lane, i_major, _tree([32, 16, 8, 4, 2, 1]))
    assert np.array_equal(stated, want)   # the emulation of the stated order agrees with the pins
    for name, got in mutants.items():
        assert not np.array_equal(got, want), name


def _seq_sum(xf, row):
    acc = np.float32(0.0)
    for k in range(len(row)):
        acc = np.float32(acc + np.float32(xf[k] * row[k]))
    return acc


# ----------------------------------------------------------- combine order
# The reading of the combine [moe_v41.rs, Kernels: accumulate, finish;
# fn shared_side]: acc = +0; acc = RN(acc + RN(w_e * y_e)) over the plan in
# ascending expert id; then acc = RN(acc + sd), the shared output added after
# the routed sum. Hand-built terms where any other order, or a fused
# multiply-add, gives another value.
def test_combine_order_pins():
    T = np.float32(2.0 ** 24)
    # shared after the routed sum: 2^24 - 2^24 = 0, then + 1 = 1; shared first gives 1 + 2^24 = 2^24, - 2^24 = 0
    out, _ = oracle.combine(np.array([[T], [-T]], np.float32), np.array([1.0, 1.0], np.float32),
                            np.array([1.0], np.float32))
    assert out[0] == 1.0
    # plan order: 2^24 + 1 = 2^24 (a tie, to even), then - 2^24 = 0; the reverse order gives
    # -2^24 + 1 = -16777215 (exact), then + 2^24 = 1
    out, _ = oracle.combine(np.array([[T], [1.0], [-T]], np.float32), np.ones(3, np.float32))
    assert out[0] == 0.0
    # each product rounded before its add: 1 + RN(-(1 + 2^-23)^2) = 1 - (1 + 2^-22) = -2^-22; a fused
    # multiply-add would keep the 2^-46 term: -(2^-22 + 2^-46)
    a = np.float32(1.0 + 2.0 ** -23)
    out, _ = oracle.combine(np.array([[1.0], [a]], np.float32), np.array([1.0, -a], np.float32))
    assert out[0] == np.float32(-(2.0 ** -22))
    # the bf16 output is the round to nearest even of the f32 sum
    out, ob = oracle.combine(np.array([[1.0 + 2.0 ** -8]], np.float32), np.ones(1, np.float32))
    assert ob[0] == 0x3F80          # 1 + 2^-8 is a tie between bf16 1.0 and 1.0078125: to even (1.0)

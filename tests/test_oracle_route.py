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

"""The glibc score mode on the host: the oracle's glibc chain pinned against
the exact function within glibc's error bound and on its special cases, the
mode wired through the oracle's selection, and the library's exception table
(built from the host libm) checked entry by entry against the oracle.

The mode follows the pages' host reference, which evaluates the softplus
chain with the platform's f32 exp / ln_1p / sqrt and asks the device path for
its selection bit for bit [device_route.rs, module doc; moe_v41.rs, fn
softplus, fn route_from_logits]."""
import ctypes
import dataclasses

import numpy as np
import pytest

import oracle
import routing_quant_expert_amd as R
import synth

RNG = np.random.default_rng(23)
SH = synth.SHAPE_TINY
SHG = dataclasses.replace(SH, score_mode=1)


def _ulp32(v: np.ndarray) -> np.ndarray:
    v = np.abs(v.astype(np.float32))
    return (np.nextafter(v, np.float32(np.inf)) - v).astype(np.float64)


@pytest.fixture(scope="module")
def table():
    return R.glibc_score_table()


def test_glibc_chain_within_error_bound():
    """glibc's expf and log1pf are each within about one ulp of the exact
    value, sqrt halves the relative error and adds half an ulp: the chain
    stays within 2 ulps of sqrt(log1p(exp(z))) evaluated in float64 (itself
    within 1e-15 relative) while exp(z) is a normal f32 (z > -87). Below,
    exp(z) is an f32 subnormal, good to half its absolute spacing 2^-149:
    score^2 is exp(z) within that plus a few ulps. A wrong branch, a dropped
    sqrt or an exp(-z) would be off by far more."""
    z = np.concatenate([RNG.uniform(-87, 25, 400_000), RNG.uniform(-2, 2, 400_000),
                        RNG.normal(0, 6, 200_000)]).astype(np.float32)
    z = z[z > -87]
    got = oracle.scores_glibc(z, 1.0).astype(np.float64)
    zd = z.astype(np.float64)
    exact = np.sqrt(np.where(zd > 20, zd, np.log1p(np.exp(zd))))
    err = np.abs(got - exact) / _ulp32(exact)
    assert err.max() <= 2.0, err.max()
    zs = RNG.uniform(-103.9, -87, 100_000).astype(np.float32)
    g2 = oracle.scores_glibc(zs, 1.0).astype(np.float64) ** 2
    ex = np.exp(zs.astype(np.float64))
    assert np.all(np.abs(g2 - ex) <= 2.0 ** -149 + 4 * 2.0 ** -24 * ex)


def test_glibc_chain_special_cases():
    """Above the cut (z > 20) softplus is z itself and sqrt is correctly
    rounded in every libm: the two modes agree bit for bit; exp(-inf) = 0
    gives score 0; the division by temp happens in f32 before the chain."""
    z = np.concatenate([RNG.uniform(20.0001, 1e4, 10_000), [20.5, 1e30, np.inf]]).astype(np.float32)
    g = oracle.scores_glibc(z, 1.0)
    assert np.array_equal(g.view(np.uint32), np.sqrt(z).view(np.uint32))
    assert np.array_equal(g.view(np.uint32), oracle.scores(z, 1.0).view(np.uint32))
    assert oracle.scores_glibc(np.array([-np.inf], np.float32), 1.0)[0] == 0.0
    lg = RNG.normal(0, 4, 10_000).astype(np.float32)
    for temp in (0.5, 1.7):
        assert np.array_equal(oracle.scores_glibc(lg, temp).view(np.uint32),
                              oracle.scores_glibc((lg / np.float32(temp)).astype(np.float32), 1.0).view(np.uint32))


def _crafted_logits(table, m, n):
    """Logits whose top picks all sit on inputs where the two chains differ."""
    keys = table[0]
    ex = keys.view(np.float32)
    hi = ex[(ex > 0.5) & (ex < 20)]
    lo = ex[(ex < -0.5) & (ex > -20)]
    lg = RNG.choice(lo, (m, n)).astype(np.float32)
    for t in range(m):
        picks = RNG.choice(n, 8, replace=False)
        lg[t, picks] = RNG.choice(hi, 8, replace=False)
    return lg


def test_select_uses_the_mode(table):
    """The selection in the glibc mode reports glibc's scores, keeps the
    picks (the keys move by an ulp at most, far below the gaps between them
    here), gives the picks' glibc scores normalised and scaled in pick order
    as weights, and so differs in the weights from the correctly rounded mode
    on tokens whose picks sit on inputs where the chains differ."""
    m = 64
    lg = _crafted_logits(table, m, SH.n_routed)
    bias = np.zeros(SH.n_routed, np.float32)
    h1, s1 = oracle.select(SHG, lg, bias)
    h0, s0 = oracle.select(SH, lg, bias)
    assert np.array_equal(s1.view(np.uint32), oracle.scores_glibc(lg, 1.0).view(np.uint32))
    assert np.array_equal(s0.view(np.uint32), oracle.scores(lg, 1.0).view(np.uint32))
    _, p1, w1, _ = oracle.header_fields(h1, SH.topk)
    _, p0, w0, _ = oracle.header_fields(h0, SH.topk)
    # picks: the keys differ by an ulp at most, far below the gaps between them here
    assert np.array_equal(p1, p0)
    # weights: the picks' glibc scores, normalised and scaled in pick order
    w = np.take_along_axis(s1, p1, 1)
    ssum = np.zeros(m, np.float32)
    for i in range(SH.topk):
        ssum = (ssum + w[:, i]).astype(np.float32)
    ssum = (ssum + np.float32(1e-20)).astype(np.float32)
    want = ((w / ssum[:, None]).astype(np.float32) * np.float32(SH.route_scale)).astype(np.float32)
    assert np.array_equal(w1.view(np.uint32), want.view(np.uint32))
    assert (w1 != w0).any(axis=1).sum() >= m // 2


def test_library_table_against_oracle(table):
    """The library's table: ascending keys, a consistent bucket index, glibc's
    value at every key (the oracle's glibc chain), a correctly rounded value
    different from it at every sampled key (the oracle's quad-precision
    chain), and no missing input among sampled non-keys."""
    keys, vals, index = table
    assert keys.size > 0 and np.all(np.diff(keys.astype(np.int64)) > 0)
    z = keys.view(np.float32)
    assert np.all(z <= 20) and not np.isnan(z).any()
    pre = (keys >> 8).astype(np.int64)
    want = np.searchsorted(pre, np.arange(1 << 24), side="left")
    assert np.array_equal(index[:-1].astype(np.int64), want) and index[-1] == keys.size
    assert np.array_equal(oracle.scores_glibc(z, 1.0).view(np.uint32), vals)
    s = RNG.choice(keys.size, 300_000, replace=False)
    assert np.all(oracle.scores(z[s], 1.0).view(np.uint32) != vals[s])
    bits = RNG.integers(0, 1 << 32, 2_000_000, dtype=np.uint64).astype(np.uint32)
    zz = bits.view(np.float32)
    keep = ~np.isin(bits, keys) & (zz <= 20)
    zz = zz[keep]
    assert np.array_equal(oracle.scores_glibc(zz, 1.0).view(np.uint32), oracle.scores(zz, 1.0).view(np.uint32))


def test_host_lookup_matches_oracle(table):
    """The library's host build of the device lookup (scores flag bit 1) on
    every key and on random logits at several temperatures."""
    z = table[0].view(np.float32)
    assert np.array_equal(R.scores_host(z, 1.0, flags=2).view(np.uint32), table[1])
    lg = np.concatenate([RNG.normal(0, 3, 1_000_000), RNG.uniform(-1, 0, 1_000_000)]).astype(np.float32)
    for temp in (1.0, 0.8, 1.3):
        got = R.scores_host(lg, temp, flags=2)
        assert np.array_equal(got.view(np.uint32), oracle.scores_glibc(lg, temp).view(np.uint32)), temp


def test_mode_checked():
    """score_mode outside {0, 1} is refused; the glibc mode with no table
    registered for the current device is refused before any argument is
    read (checked where there is no device at all)."""
    bad = R.cfg_from_shape(dataclasses.replace(SH, score_mode=2))
    assert R.workspace_bytes(bad, 1) == 0
    c = R.cfg_from_shape(SHG)
    assert R.workspace_bytes(c, 1) > 0
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present: the registration check is covered by the GPU tests")
    buf = np.zeros(1 << 16, np.uint8)
    p = ctypes.c_void_p(buf.ctypes.data)
    rc = R.lib().moe_route_select(ctypes.byref(c), p, 1, p, p, None, p, p, buf.size, None)
    assert rc != 0 and "moe_set_score_table" in R.lib().moe_last_error().decode()


def test_table_call_checked(table):
    """The table call reports the count with keys = NULL and refuses a
    buffer smaller than the count."""
    n = ctypes.c_int64(0)
    assert R.lib().moe_glibc_score_table(None, None, None, 0, ctypes.byref(n)) == 0 and n.value == table[0].size
    small = np.empty(4, np.uint32)
    idx = np.empty(R.binding.SCORE_INDEX_LEN, np.uint32)
    rc = R.lib().moe_glibc_score_table(small.ctypes.data, small.ctypes.data, idx.ctypes.data, 4, ctypes.byref(n))
    assert rc != 0 and "cap" in R.lib().moe_last_error().decode()
    assert R.lib().moe_glibc_score_table(None, None, None, 0, None) != 0

"""Oracle pins: number formats, elementary functions, K-quant blocks, q8_1.

Each test pins an oracle function to something other than itself: numpy's
IEEE conversions, mpmath at 200 bits, exact rational arithmetic, or an
independent packer (dense fields -> bytes, the inverse direction)."""
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle
from tests._exact import f16_bits, fp16_fraction, pack_q2k, pack_q3k, round_to_f32

RNG = np.random.default_rng(12345)


# ------------------------------------------------------------------ bf16
def _bf16_by_comparison(v: np.ndarray) -> np.ndarray:
    """RNE to bf16 by choosing the nearer of the two bracketing bf16 values
    (exact float64 distances; ties to the even one). Overflow: the candidate
    above the largest finite bf16 is 2^128, as IEEE rounding prescribes."""
    b = v.view(np.uint32)
    lo = b & np.uint32(0xFFFF0000)
    lo_v = lo.view(np.float32).astype(np.float64)
    hi = lo.astype(np.uint64) + np.uint64(0x10000)
    hi_v = (hi.astype(np.uint32)).view(np.float32).astype(np.float64)
    hi_v = np.where((hi & np.uint64(0x7F800000)) == np.uint64(0x7F800000),
                    np.sign(lo_v) * 2.0 ** 128, hi_v)
    x = v.astype(np.float64)
    dlo, dhi = np.abs(x - lo_v), np.abs(x - hi_v)
    even_lo = ((lo >> np.uint32(16)) & np.uint32(1)) == 0
    take_hi = (dhi < dlo) | ((dhi == dlo) & ~even_lo)
    return np.where(take_hi, (hi >> np.uint64(16)).astype(np.uint16), (lo >> np.uint32(16)).astype(np.uint16))


def test_bf16_rne_matches_comparison_rounding():
    bits = RNG.integers(0, 2 ** 32, size=1 << 21, dtype=np.uint64).astype(np.uint32)
    exps = np.arange(0, 255, dtype=np.uint32)
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    struct = (exps[:, None, None] << np.uint32(23)) | (np.array([0, 0x10000], np.uint32)[None, :, None]) | lows[None, None, :]
    bits = np.concatenate([bits, struct.reshape(-1), struct.reshape(-1) | np.uint32(0x80000000)])
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(oracle.f32_to_bf16(v), _bf16_by_comparison(v))
    # bf16 -> f32 is exact: the bits are the top half
    b16 = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    back = oracle.bf16_to_f32(b16)
    assert np.array_equal(back.view(np.uint32), b16.astype(np.uint32) << np.uint32(16))


# ------------------------------------------------------------------ fp16
def test_fp16_decode_exhaustive():
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.fp16_to_f64(h)
    ref = h.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_fp16_encode_exhaustive_over_the_fp16_range():
    """Every f32 with biased exponent 96..143 (|x| from 2^-31, which rounds
    to zero, through subnormals and normals up to 2^17, which overflows),
    both signs, against numpy's float32 -> float16 conversion."""
    man = np.arange(0, 1 << 23, dtype=np.uint32)
    for e in range(96, 144):
        for sign in (0, 1):
            bits = (np.uint32(sign) << np.uint32(31)) | (np.uint32(e) << np.uint32(23)) | man
            v = bits.view(np.float32)
            ref = v.astype(np.float16).view(np.uint16)
            got = oracle.f32_to_fp16(v)
            if not np.array_equal(got, ref):
                i = np.nonzero(got != ref)[0][0]
                pytest.fail(f"f32 {v[i]!r} bits {bits[i]:#x}: oracle {got[i]:#x} numpy {ref[i]:#x}")
    # zero, tiny, inf, nan
    sp = np.array([0.0, -0.0, 1e-30, -1e-30, np.inf, -np.inf, 65504.0, 65519.99, 65520.0], np.float32)
    assert np.array_equal(oracle.f32_to_fp16(sp), sp.astype(np.float16).view(np.uint16))
    assert (oracle.f32_to_fp16(np.array([np.nan], np.float32))[0] & 0x7C00) == 0x7C00


# -------------------------------------------------- correctly rounded maths
def _cr(fn, x: float) -> np.float32:
    """Correct f32 rounding of fn(x) evaluated by mpmath at 200 bits."""
    with mpmath.workprec(200):
        v = fn(mpmath.mpf(float(x)))
        man, exp = v.man_exp
        return round_to_f32(Fraction(int(man)) * Fraction(2) ** int(exp))


def _sample_inputs():
    xs = [0.0, -0.0, 1e-45, -1e-45, 1e-30, -1e-30, 2.0 ** -25, -2.0 ** -25, 1.0, -1.0, 20.0, -20.0, 19.999998,
          20.000002, 88.0, -87.0, -100.0, -103.9, 0.5, -0.5, 1e-8, -1e-8]
    xs += list(RNG.normal(0, 1.28, 400)) + list(RNG.normal(0, 8.0, 200))
    xs += list(RNG.uniform(-104, 20, 300)) + list(np.ldexp(RNG.uniform(-1, 1, 100), RNG.integers(-60, 0, 100)))
    return np.array(xs, np.float32)


def test_exp_cr_matches_mpmath():
    xs = _sample_inputs()
    got = oracle.exp_cr(xs)
    for x, g in zip(xs, got):
        want = _cr(mpmath.exp, x)
        assert g.view(np.uint32) == want.view(np.uint32), (x, g, want)


def test_log1p_cr_matches_mpmath():
    xs = np.abs(_sample_inputs())
    xs = np.concatenate([xs, oracle.exp_cr(_sample_inputs())]).astype(np.float32)
    got = oracle.log1p_cr(xs)
    for x, g in zip(xs, got):
        want = _cr(mpmath.log1p, x)
        assert g.view(np.uint32) == want.view(np.uint32), (x, g, want)


def test_score_special_values():
    temp = 1.0
    big = np.array([20.5, 21.0, 100.0, 1e6], np.float32)
    # above the cut the score is the correctly rounded sqrt of the logit itself
    assert np.array_equal(oracle.scores(big, temp), np.sqrt(big))
    # far below: exp underflows to 0, log1p(0) = 0
    assert np.all(oracle.scores(np.array([-200.0, -1e30], np.float32), temp) == 0.0)
    # at 0: sqrt(RN(log1p(1))) = sqrt(RN(ln 2))
    ln2 = _cr(mpmath.log1p, 1.0)
    assert oracle.scores(np.array([0.0], np.float32), temp)[0] == np.sqrt(ln2)
    # the cut is strict: 20 itself goes through log1p(exp(20))
    e20 = _cr(mpmath.exp, 20.0)
    want = np.sqrt(_cr(mpmath.log1p, float(e20)))
    assert oracle.scores(np.array([20.0], np.float32), temp)[0] == want
    # temperature divides first (one f32 rounding)
    lg = np.array([1.5], np.float32)
    z = np.float32(lg[0] / np.float32(0.7))
    want = np.sqrt(_cr(mpmath.log1p, float(_cr(mpmath.exp, float(z)))))
    assert oracle.scores(lg, 0.7)[0] == want


# -------------------------------------------------------------- K-quants
def test_q2k_position_map_one_hot():
    """A block with one code at position w (and scale 1, min 0, d = 1)
    dequantises to a single non-zero weight at w."""
    for w in range(256):
        codes = np.zeros(256, int)
        codes[w] = 3
        blk = pack_q2k(codes, [1] * 16, [0] * 16, f16_bits(1.0), 0)
        dq = oracle.q2k_dequant(blk)
        assert dq[w] == 3.0 and np.count_nonzero(dq) == 1, w


def test_q2k_scale_and_min_nibbles():
    for s in range(16):
        sc = [0] * 16
        mn = [0] * 16
        sc[s], mn[s] = 5, 9
        blk = pack_q2k([2] * 256, sc, mn, f16_bits(0.5), f16_bits(0.25))
        dq = oracle.q2k_dequant(blk)
        want = np.zeros(256)
        want[16 * s:16 * s + 16] = 0.5 * 5 * 2 - 0.25 * 9
        assert np.array_equal(dq, want), s


def test_q2k_random_roundtrip_exact():
    for _ in range(20):
        codes = RNG.integers(0, 4, 256)
        sc = RNG.integers(0, 16, 16)
        mn = RNG.integers(0, 16, 16)
        d, dm = RNG.integers(0, 0x7C00, 2)
        blk = pack_q2k(codes, sc, mn, int(d), int(dm))
        dq = oracle.q2k_dequant(blk)
        fd, fm = fp16_fraction(int(d)), fp16_fraction(int(dm))
        for w in range(256):
            assert Fraction(dq[w]) == fd * int(sc[w // 16]) * int(codes[w]) - fm * int(mn[w // 16])


def test_q3k_position_map_and_sign_bit():
    for w in range(256):
        for val in (-4, -1, 1, 3):
            vals = np.zeros(256, int)
            vals[w] = val
            blk = pack_q3k(vals, [33] * 16, f16_bits(1.0))   # scale 33 -> factor 1
            dq = oracle.q3k_dequant(blk)
            assert dq[w] == val and np.count_nonzero(dq) == 1, (w, val)


def test_q3k_all_sixteen_6bit_scales():
    scales = np.arange(16) * 4 + 1          # 1, 5, ..., 61: distinct, both nibbles and top bits vary
    for perm in range(4):
        sc = np.roll(scales, perm * 3)
        blk = pack_q3k([2] * 256, sc, f16_bits(1.0))
        dq = oracle.q3k_dequant(blk)
        want = np.repeat((sc - 32) * 2.0, 16)
        assert np.array_equal(dq, want)
    blk = pack_q3k([-4] * 256, list(range(48, 64)), f16_bits(0.125))
    assert np.array_equal(oracle.q3k_dequant(blk), np.repeat((np.arange(48, 64) - 32) * -4 * 0.125, 16))


def test_q3k_random_roundtrip_exact():
    for _ in range(20):
        vals = RNG.integers(-4, 4, 256)
        sc = RNG.integers(0, 64, 16)
        d = int(RNG.integers(0, 0x7C00))
        dq = oracle.q3k_dequant(pack_q3k(vals, sc, d))
        fd = fp16_fraction(d)
        for w in range(256):
            assert Fraction(dq[w]) == fd * (int(sc[w // 16]) - 32) * int(vals[w])


# ------------------------------------------------------------------ q8_1
def test_q8_1_invariants():
    x = (RNG.normal(0, 1, 32 * 300) * np.exp(RNG.normal(0, 2, 32 * 300))).astype(np.float32)
    x[:32] = 0.0                                        # all-zero block
    x[32:64] = 0.0
    x[40] = -3.25                                       # single non-zero
    q, d16 = oracle.q8_1(x)
    qb, xb = q.reshape(-1, 32).astype(np.int64), x.reshape(-1, 32)
    amax = np.abs(xb).max(axis=1)
    d = (amax / np.float32(127.0)).astype(np.float32)
    assert np.all(qb[0] == 0) and d16[0] == 0
    assert qb[1, 8] == -127 and np.count_nonzero(qb[1]) == 1
    nz = amax > 0
    ratio = xb[nz].astype(np.float64) / d[nz, None].astype(np.float64)
    assert np.all(np.abs(ratio - qb[nz]) <= 0.5 + 1e-6)
    # the largest magnitude gets +-127
    arg = np.abs(xb).argmax(axis=1)
    assert np.all(np.abs(qb[nz, arg[nz]]) == 127)
    # odd symmetry
    qn, dn = oracle.q8_1(-x)
    assert np.array_equal(qn, -q) and np.array_equal(dn, d16)
    # stored scale is fp16(d)
    assert np.array_equal(d16, d.astype(np.float16).view(np.uint16))


def test_q8_1_half_rounds_away_from_zero():
    x = np.zeros(32, np.float32)
    x[0] = 127.0                 # amax 127 -> d = 1 exactly
    x[1], x[2], x[3], x[4] = 2.5, -2.5, 0.5, -1.5
    q, d16 = oracle.q8_1(x)
    assert list(q[:5]) == [127, 3, -3, 1, -2]
    assert d16[0] == f16_bits(1.0)


def test_q8_1_requantise_fixed_point():
    x = RNG.normal(0, 1, 32 * 64).astype(np.float32)
    q, _ = oracle.q8_1(x)
    amax = np.abs(x.reshape(-1, 32)).max(axis=1).astype(np.float32)
    d = (amax / np.float32(127.0)).astype(np.float32)
    dec = (q.reshape(-1, 32).astype(np.float32) * d[:, None]).astype(np.float32).reshape(-1)
    q2, _ = oracle.q8_1(dec)
    assert np.array_equal(q, q2)

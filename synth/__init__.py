"""Seeded synthetic inputs for the MoE decode layer.

This module only draws inputs; it holds none of the layer's arithmetic. The
same recipe is implemented twice: here in numpy (host) and in
``synth_device.hip`` (device, for the multi-GB expert arenas). Every value is
produced by integer operations plus single IEEE-754 roundings (add, multiply,
float64->float32, float32->float16), so both sides emit identical bytes; a
test checks that.

Random stream: a splitmix64 sequence (Steele, Lea, Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014). Stream ``(seed, tag)`` starts
from ``s0 = mix(seed ^ tag + G)`` and its draw ``i`` is ``mix(s0 + (i+1)*G)``,
so any draw can be computed on its own (counter-based).

Value recipes (one per field kind):
  * normal N(0, sigma) as bf16: Irwin-Hall sum of 12 uniform u32 (six draws
    per value), z = (S - 6*2^32) * 2^-32 exactly in float64, v = z*sigma
    rounded to float64, then to float32 (RN), then to bf16 (RNE on the bits).
  * uniform U(lo, lo+span): u = (r >> 11) * 2^-53 (or u32 * 2^-32 for the
    block scales), v = lo + span*u in float64 (two roundings, no FMA), then
    float32 (RN) and, for block scales, float16 (RNE).
  * Q2_K super-block (84 B): 11 draws; draws 0..9 give bytes [0,80) (the 16
    scale/min bytes and the 64 code bytes) little-endian, draw 10's low and
    high u32 give d and dmin as float16 U(1e-3, 1e-2).
  * Q3_K super-block (110 B): 15 draws; draws 0..13 give bytes [0,108)
    (hmask 32, codes 64, packed 6-bit scales 12), draw 14's low u32 gives d.
"""
from __future__ import annotations

import dataclasses
import numpy as np

M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

# tag kinds (bits 56..63 of a tag)
K_X = 1
K_GATE_W = 2
K_BIAS = 3
K_EXP_GATE = 4
K_EXP_UP = 5
K_EXP_DOWN = 6
K_SH_W1 = 7
K_SH_W3 = 8
K_SH_W2 = 9
K_X_COMMON = 10
K_PERM = 11

Q2K_BYTES = 84
Q3K_BYTES = 110
Q2K_DRAWS = 11
Q3K_DRAWS = 15
QK = 256

SCALE_LO = 1e-3
SCALE_SPAN = 9e-3


def make_tag(kind: int, layer: int = 0, index: int = 0, sub: int = 0) -> int:
    assert 0 <= kind < 256 and 0 <= layer < 65536 and 0 <= index < 16777216 and 0 <= sub < 65536
    return (kind << 56) | (layer << 40) | (index << 16) | sub


def _mix_scalar(z: int) -> int:
    z &= M64
    z = ((z ^ (z >> 30)) * MIX1) & M64
    z = ((z ^ (z >> 27)) * MIX2) & M64
    return z ^ (z >> 31)


def stream_start(seed: int, tag: int) -> int:
    return _mix_scalar(((seed ^ tag) + GOLDEN) & M64)


_CHUNK = 1 << 18
_scratch = {}


def _buf(name: str, n: int, dtype) -> np.ndarray:
    """Reused scratch arrays (fresh allocations are slow where page faults are costly)."""
    b = _scratch.get(name)
    if b is None or b.size < n or b.dtype != dtype:
        b = np.empty(max(n, _CHUNK), dtype)
        _scratch[name] = b
    return b[:n]


_count = np.arange(1, 2 * _CHUNK + 1, dtype=np.uint64)


def _counting(n: int) -> np.ndarray:
    """1, 2, ..., n (uint64), from a cached array."""
    global _count
    if _count.size < n:
        _count = np.arange(1, n + 1, dtype=np.uint64)
    return _count[:n]


def _draws_into(z: np.ndarray, s0: np.uint64, i0: int) -> None:
    """z[k] = mix(s0 + (i0+k+1)*G) for the length of z (in place)."""
    n = z.size
    ar = _counting(n)
    t = _buf("tmp", n, np.uint64)
    with np.errstate(over="ignore"):
        np.add(ar, np.uint64(i0), out=z)
        np.multiply(z, np.uint64(GOLDEN), out=z)
        np.add(z, s0, out=z)
        np.right_shift(z, np.uint64(30), out=t)
        np.bitwise_xor(z, t, out=z)
        np.multiply(z, np.uint64(MIX1), out=z)
        np.right_shift(z, np.uint64(27), out=t)
        np.bitwise_xor(z, t, out=z)
        np.multiply(z, np.uint64(MIX2), out=z)
        np.right_shift(z, np.uint64(31), out=t)
        np.bitwise_xor(z, t, out=z)


def draws(seed: int, tag: int, i0: int, n: int) -> np.ndarray:
    """Draws i0 .. i0+n-1 of stream (seed, tag) as uint64."""
    s0 = np.uint64(stream_start(seed, tag))
    out = np.empty(n, np.uint64)
    for c0 in range(0, n, _CHUNK):
        _draws_into(out[c0:c0 + _CHUNK], s0, i0 + c0)
    return out


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even on the bits."""
    b = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    return ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_chunk(s0: np.uint64, i0: int, n: int, out: np.ndarray) -> None:
    r = _buf("nraw", 6 * n, np.uint64)
    _draws_into(r, s0, 6 * i0)
    r = r.reshape(n, 6)
    lo = _buf("nlo", 6 * n, np.uint64).reshape(n, 6)
    np.bitwise_and(r, np.uint64(0xFFFFFFFF), out=lo)
    np.right_shift(r, np.uint64(32), out=r)
    np.add(r, lo, out=r)                     # each < 2^33, six of them < 2^36: no wrap
    s = r.sum(axis=1, dtype=np.uint64).astype(np.int64) - np.int64(6 << 32)
    np.multiply(s.astype(np.float64), 2.0 ** -32, out=out)


def normal_f64(seed: int, tag: int, i0: int, n: int) -> np.ndarray:
    """Irwin-Hall N(0,1) values i0..i0+n-1 as exact float64."""
    s0 = np.uint64(stream_start(seed, tag))
    out = np.empty(n, np.float64)
    ch = _CHUNK // 4
    for c0 in range(0, n, ch):
        c1 = min(n, c0 + ch)
        _normal_chunk(s0, i0 + c0, c1 - c0, out[c0:c1])
    return out


def normal_bf16(seed: int, tag: int, i0: int, n: int, sigma: float) -> np.ndarray:
    s0 = np.uint64(stream_start(seed, tag))
    out = np.empty(n, np.uint16)
    ch = _CHUNK // 4
    z = _buf("nz", ch, np.float64)
    for c0 in range(0, n, ch):
        c1 = min(n, c0 + ch)
        zz = z[:c1 - c0]
        _normal_chunk(s0, i0 + c0, c1 - c0, zz)
        np.multiply(zz, np.float64(sigma), out=zz)
        out[c0:c1] = f32_to_bf16_bits(zz.astype(np.float32))
    return out


def uniform_f32(seed: int, tag: int, i0: int, n: int, lo: float, span: float) -> np.ndarray:
    r = draws(seed, tag, i0, n)
    u = (r >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    return (np.float64(lo) + np.float64(span) * u).astype(np.float32)


def _u32_to_scale_f16(u32: np.ndarray) -> np.ndarray:
    u = u32.astype(np.float64) * (2.0 ** -32)
    v = (np.float64(SCALE_LO) + np.float64(SCALE_SPAN) * u).astype(np.float32)
    return v.astype(np.float16).view(np.uint16)


def q2k_blocks(seed: int, tag: int, b0: int, nb: int) -> np.ndarray:
    """Q2_K super-blocks b0..b0+nb-1 of stream (seed, tag): uint8 [nb, 84]."""
    r = draws(seed, tag, Q2K_DRAWS * b0, Q2K_DRAWS * nb).reshape(nb, Q2K_DRAWS)
    out = np.empty((nb, Q2K_BYTES), dtype=np.uint8)
    out[:, :80] = np.ascontiguousarray(r[:, :10]).view(np.uint8).reshape(nb, 80)
    last = r[:, 10]
    d = _u32_to_scale_f16(last & np.uint64(0xFFFFFFFF))
    dmin = _u32_to_scale_f16(last >> np.uint64(32))
    out[:, 80:82] = d.view(np.uint8).reshape(nb, 2)
    out[:, 82:84] = dmin.view(np.uint8).reshape(nb, 2)
    return out


def q3k_blocks(seed: int, tag: int, b0: int, nb: int) -> np.ndarray:
    """Q3_K super-blocks b0..b0+nb-1 of stream (seed, tag): uint8 [nb, 110]."""
    r = draws(seed, tag, Q3K_DRAWS * b0, Q3K_DRAWS * nb).reshape(nb, Q3K_DRAWS)
    out = np.empty((nb, Q3K_BYTES), dtype=np.uint8)
    out[:, :108] = np.ascontiguousarray(r[:, :14]).view(np.uint8).reshape(nb, 112)[:, :108]
    d = _u32_to_scale_f16(r[:, 14] & np.uint64(0xFFFFFFFF))
    out[:, 108:110] = d.view(np.uint8).reshape(nb, 2)
    return out


# --------------------------------------------------------------------------
# Layer shapes and the expert arena layout
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Shape:
    dim: int
    inter: int
    n_routed: int = 384
    topk: int = 6
    gate_temp: float = 1.0
    route_scale: float = 2.5
    swiglu_limit: float = 7.0
    norm_topk_prob: bool = True
    score_mode: int = 0          # 0: correctly rounded scores, 1: the host glibc's

    @property
    def gate_rows(self) -> int:
        return self.inter

    @property
    def nsb_gate(self) -> int:      # Q2_K super-blocks per gate/up row
        return self.dim // QK

    @property
    def nsb_down(self) -> int:      # Q3_K super-blocks per down row
        return self.inter // QK

    @property
    def gate_bytes(self) -> int:
        return self.inter * self.nsb_gate * Q2K_BYTES

    @property
    def down_bytes(self) -> int:
        return self.dim * self.nsb_down * Q3K_BYTES

    @property
    def expert_stride(self) -> int:
        return 2 * self.gate_bytes + self.down_bytes

    @property
    def gate_off(self) -> int:
        return 0

    @property
    def up_off(self) -> int:
        return self.gate_bytes

    @property
    def down_off(self) -> int:
        return 2 * self.gate_bytes


SHAPE_TINY = Shape(dim=512, inter=256)       # single layer, the small correctness case
SHAPE_DS41 = Shape(dim=4096, inter=2048)     # realistic decode shape

# (kind, sigma) of the bf16 tensors
SIGMA_X = 1.0
SIGMA_W = 0.02
BIAS_LO, BIAS_SPAN = -0.1, 0.2


@dataclasses.dataclass
class LayerSpec:
    """Everything needed to regenerate one layer's inputs on either side."""
    shape: Shape
    seed: int = 1
    layer: int = 0
    zipf_bias: bool = False
    shared_quant: bool = False   # the shared expert as K-quant blocks (Q2_K gate/up, Q3_K down) instead of bf16

    def tag(self, kind: int, index: int = 0, sub: int = 0) -> int:
        return make_tag(kind, self.layer, index, sub)


def gate_w(spec: LayerSpec) -> np.ndarray:
    s = spec.shape
    return normal_bf16(spec.seed, spec.tag(K_GATE_W), 0, s.n_routed * s.dim, SIGMA_W).reshape(s.n_routed, s.dim)


def zipf_bias(spec: LayerSpec, s_exp: float = 1.1) -> np.ndarray:
    """bias[perm(r)] = r^-s / sum_r' r'^-s over a seeded random expert permutation."""
    n = spec.shape.n_routed
    r = draws(spec.seed, spec.tag(K_PERM), 0, n)
    perm = np.arange(n)
    for i in range(n - 1, 0, -1):          # Fisher-Yates, j uniform in [0, i]
        j = int(r[i] % np.uint64(i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    ranks = np.arange(1, n + 1, dtype=np.float64)
    w = ranks ** (-s_exp)
    w = w / w.sum()
    bias = np.empty(n, dtype=np.float32)
    bias[perm] = w.astype(np.float32)
    return bias


def bias(spec: LayerSpec) -> np.ndarray:
    if spec.zipf_bias:
        return zipf_bias(spec)
    return uniform_f32(spec.seed, spec.tag(K_BIAS), 0, spec.shape.n_routed, BIAS_LO, BIAS_SPAN)


def shared_w(spec: LayerSpec, which: str) -> np.ndarray:
    s = spec.shape
    kind = {"w1": K_SH_W1, "w3": K_SH_W3, "w2": K_SH_W2}[which]
    rows, cols = (s.dim, s.inter) if which == "w2" else (s.inter, s.dim)
    return normal_bf16(spec.seed, spec.tag(kind), 0, rows * cols, SIGMA_W).reshape(rows, cols)


def expert_blocks(spec: LayerSpec, e: int, which: str) -> np.ndarray:
    """Raw blocks of expert e: gate/up -> uint8 [inter, nsb_gate*84]; down -> [dim, nsb_down*110]."""
    s = spec.shape
    if which in ("gate", "up"):
        kind = K_EXP_GATE if which == "gate" else K_EXP_UP
        nb = s.inter * s.nsb_gate
        return q2k_blocks(spec.seed, spec.tag(kind, e), 0, nb).reshape(s.inter, s.nsb_gate * Q2K_BYTES)
    nb = s.dim * s.nsb_down
    return q3k_blocks(spec.seed, spec.tag(K_EXP_DOWN, e), 0, nb).reshape(s.dim, s.nsb_down * Q3K_BYTES)


def shared_q_blocks(spec: LayerSpec, which: str) -> np.ndarray:
    """The K-quant shared expert's raw blocks: drawn exactly like a routed
    expert's, under the expert index n_routed (no routed expert has it)."""
    return expert_blocks(spec, spec.shape.n_routed, which)


def expert_bytes(spec: LayerSpec, e: int) -> np.ndarray:
    """Expert e's slice of the arena (stride bytes): gate | up | down."""
    return np.concatenate([expert_blocks(spec, e, w).reshape(-1) for w in ("gate", "up", "down")])


def tokens(spec: LayerSpec, t0: int, m: int) -> np.ndarray:
    """bf16 N(0,1) input rows t0..t0+m-1: uint16 [m, dim]."""
    d = spec.shape.dim
    out = np.empty((m, d), dtype=np.uint16)
    for i in range(m):
        out[i] = normal_bf16(spec.seed, make_tag(K_X, spec.layer, t0 + i), 0, d, SIGMA_X)
    return out


def correlated_tokens(spec: LayerSpec, m: int, weight: float = 0.5, group: int = 0) -> np.ndarray:
    """x_t = bf16(w*c + sqrt(1-w^2)*z_t): rows sharing one N(0,1) component c.
    Group g uses its own c and the z of rows g*m .. g*m+m-1."""
    d = spec.shape.dim
    c = normal_f64(spec.seed, make_tag(K_X_COMMON, spec.layer, group), 0, d)
    a = np.float64(weight)
    b = np.sqrt(np.float64(1.0) - a * a)
    out = np.empty((m, d), dtype=np.uint16)
    for i in range(m):
        z = normal_f64(spec.seed, make_tag(K_X, spec.layer, group * m + i), 0, d)
        v = (a * c + b * z).astype(np.float32)
        out[i] = f32_to_bf16_bits(v)
    return out

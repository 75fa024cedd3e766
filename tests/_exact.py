"""Independent helpers for the oracle's pins: exact rational rounding and a
K-quant *packer* (the inverse of the oracle's decoder, written from the GGUF
layout description in the other direction: dense fields -> bytes)."""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def f32_neighbours(f: np.float32):
    f = np.float32(f)
    return np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))


def round_to_f32(v) -> np.float32:
    """Correct round-to-nearest-even of an exact rational (Fraction or mpmath
    value convertible to Fraction) to float32, by comparing with neighbours."""
    fr = Fraction(v)
    guess = np.float32(float(fr))  # within an ulp or two
    best = None
    for _ in range(4):
        cands = f32_neighbours(guess)
        dists = [abs(Fraction(float(c)) - fr) if np.isfinite(c) else None for c in cands]
        finite = [(d, c) for d, c in zip(dists, cands) if d is not None]
        finite.sort(key=lambda dc: dc[0])
        d0, c0 = finite[0]
        ties = [c for d, c in finite if d == d0]
        if len(ties) > 1:  # exact midpoint: even mantissa wins
            c0 = [c for c in ties if (np.array(c, np.float32).view(np.uint32) & 1) == 0][0]
        if c0 == guess:
            best = c0
            break
        guess = c0
    assert best is not None
    return np.float32(best)


def fp16_fraction(bits: int) -> Fraction:
    s, e, m = bits >> 15, (bits >> 10) & 31, bits & 1023
    assert e != 31
    v = Fraction(m, 1 << 24) if e == 0 else Fraction(1024 + m) * Fraction(2) ** (e - 25)
    return -v if s else v


# ---------------------------------------------------------------- packers
def pack_q2k(codes, sc, mn, d_bits: int, dmin_bits: int) -> np.ndarray:
    """codes: 256 ints in 0..3 (weight order); sc, mn: 16 ints in 0..15 per
    16-weight sub-block. Weight w lives in code byte 32*(w//128) + w%32 at
    bit pair (w%128)//32."""
    blk = np.zeros(84, np.uint8)
    for s in range(16):
        blk[s] = (int(sc[s]) & 15) | ((int(mn[s]) & 15) << 4)
    for w in range(256):
        byte = 16 + 32 * (w // 128) + (w % 32)
        shift = 2 * ((w % 128) // 32)
        blk[byte] |= (int(codes[w]) & 3) << shift
    blk[80], blk[81] = d_bits & 255, d_bits >> 8
    blk[82], blk[83] = dmin_bits & 255, dmin_bits >> 8
    return blk


def pack_q3k(vals, scales6, d_bits: int) -> np.ndarray:
    """vals: 256 ints in -4..3; scales6: 16 ints in 0..63 (the stored 6-bit
    scale, weight = d*(scale-32)*val). Low 2 bits of val+4 go to the code
    bytes like Q2_K; the third bit (val >= 0) goes to hmask byte w%32 at bit
    (w//128)*4 + (w%128)//32. Scale s keeps its low nibble in byte s (s<8,
    low half) or byte s-8 (high half) and its top 2 bits in byte 8 + s%4 at
    bit 2*(s//4)."""
    blk = np.zeros(110, np.uint8)
    for w in range(256):
        v = int(vals[w]) + 4            # 0..7
        lo2, hb = v & 3, v >> 2
        byte = 32 + 32 * (w // 128) + (w % 32)
        blk[byte] |= lo2 << (2 * ((w % 128) // 32))
        blk[w % 32] |= hb << (4 * (w // 128) + (w % 128) // 32)
    for s in range(16):
        u = int(scales6[s])
        if s < 8:
            blk[96 + s] |= u & 15
        else:
            blk[96 + s - 8] |= (u & 15) << 4
        blk[96 + 8 + s % 4] |= (u >> 4) << (2 * (s // 4))
    blk[108], blk[109] = d_bits & 255, d_bits >> 8
    return blk


def f16_bits(x: float) -> int:
    return int(np.array(x, np.float16).view(np.uint16))

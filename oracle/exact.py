"""Exact rational brute force for tiny inputs (test infrastructure only).

Every value is a ``fractions.Fraction``: bf16 inputs are exact binary fractions,
their products and sums are exact, and rounding to bf16 is done once, on the
exact rational, to the nearest representable value with ties to even.  This is
the yardstick the double-precision oracle (``oracle.c``) is pinned against; it
shares no code with it.

Definitions follow "Reproducible LoRA Inference Through Deterministic Split-K
Reduction" (Balusamy & Mohan): Eq. 1 (shrink X A^T, expand s (.) B^T added to
Y) and section 6.2 (fp32 shrink values converted to bf16 downstream).
"""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np

BF16_MAX = Fraction(255) * Fraction(2) ** 120          # (2 - 2^-7) * 2^127
BF16_SUB_QUANTUM = Fraction(1, 2 ** 133)               # spacing below 2^-126


def bf16_bits_to_fraction(b: int) -> Fraction:
    f = struct.unpack("<f", struct.pack("<I", (int(b) & 0xFFFF) << 16))[0]
    return Fraction(f)


def f32_to_fraction(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def _floor_log2(q: Fraction) -> int:
    """Largest E with 2^E <= q, for q > 0."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    while Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def rne_bf16(q: Fraction) -> Fraction:
    """Nearest bf16 value to the exact rational q, ties to the even significand.

    bf16 keeps 8 significant bits, so for 2^E <= |q| < 2^(E+1) neighbours are
    2^(E-7) apart; below the smallest normal 2^-126 the spacing is fixed at
    2^-133.  Returns +-inf (as float) on overflow."""
    if q == 0:
        return Fraction(0)
    sign = 1 if q > 0 else -1
    a = abs(q)
    E = _floor_log2(a)
    quantum = Fraction(2) ** (E - 7) if E >= -126 else BF16_SUB_QUANTUM
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    res = fl * quantum
    if res > BF16_MAX:
        return float("inf") * sign
    return sign * res


def fraction_to_bf16_bits(q) -> int:
    """Bits of a value that is already exactly a bf16 number."""
    if isinstance(q, float):
        f = q
    else:
        f = float(q)
        assert Fraction(f) == q
    u = struct.unpack("<I", struct.pack("<f", f))[0]
    assert (u & 0xFFFF) == 0
    return u >> 16


def shrink(x_bits, A_bits, scale=1):
    """Exact h[i][j] = scale * sum_k x[i][k] A[j][k]; x [M,K], A [r,K]."""
    x_bits = np.asarray(x_bits)
    A_bits = np.asarray(A_bits)
    M, K = x_bits.shape
    r = A_bits.shape[0]
    xs = [[bf16_bits_to_fraction(x_bits[i, k]) for k in range(K)] for i in range(M)]
    As = [[bf16_bits_to_fraction(A_bits[j, k]) for k in range(K)] for j in range(r)]
    sc = Fraction(scale)
    return [[sc * sum((xs[i][k] * As[j][k] for k in range(K)), Fraction(0)) for j in range(r)]
            for i in range(M)]


def expand(h_f32, B_bits, y_bits, scale):
    """Exact e = y + scale * sum_j rne_bf16(h[i][j]) B[n][j] and its bf16 rounding."""
    h_f32 = np.asarray(h_f32, dtype=np.float32)
    B_bits = np.asarray(B_bits)
    y_bits = np.asarray(y_bits)
    M, r = h_f32.shape
    N = B_bits.shape[0]
    sc = Fraction(float(np.float32(scale))) if not isinstance(scale, Fraction) else scale
    E = []
    O = []
    for i in range(M):
        hb = [rne_bf16(f32_to_fraction(h_f32[i, j])) for j in range(r)]
        erow, orow = [], []
        for n in range(N):
            s = sum((hb[j] * bf16_bits_to_fraction(B_bits[n, j]) for j in range(r)), Fraction(0))
            e = bf16_bits_to_fraction(y_bits[i, n]) + sc * s
            erow.append(e)
            orow.append(fraction_to_bf16_bits(rne_bf16(e)))
        E.append(erow)
        O.append(orow)
    return O, E


def expand_compensated(h_f32, B_bits, y_bits, scale):
    """Exact compensated expand: hi = rne_bf16(h), lo = rne_bf16(h - hi),
    e = y + scale * sum_j (hi + lo) B[n][j], and its bf16 rounding (the HEAL
    page, section 3, Eq. 10, with bf16 halves)."""
    h_f32 = np.asarray(h_f32, dtype=np.float32)
    B_bits = np.asarray(B_bits)
    y_bits = np.asarray(y_bits)
    M, r = h_f32.shape
    N = B_bits.shape[0]
    sc = Fraction(float(np.float32(scale))) if not isinstance(scale, Fraction) else scale
    E, O = [], []
    for i in range(M):
        hv = [f32_to_fraction(h_f32[i, j]) for j in range(r)]
        hi = [rne_bf16(v) for v in hv]
        lo = [rne_bf16(v - a) for v, a in zip(hv, hi)]
        erow, orow = [], []
        for n in range(N):
            s = sum(((hi[j] + lo[j]) * bf16_bits_to_fraction(B_bits[n, j]) for j in range(r)), Fraction(0))
            e = bf16_bits_to_fraction(y_bits[i, n]) + sc * s
            erow.append(e)
            orow.append(fraction_to_bf16_bits(rne_bf16(e)))
        E.append(erow)
        O.append(orow)
    return O, E

"""CPU reference ("the oracle") for the deterministic Split-K LoRA shrink/expand.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The GPU library
never loads it, and the two share no code: the arithmetic lives in
``oracle.c`` (plain C, double precision) and ``exact.py`` (exact rationals),
each function citing the passage of "Reproducible LoRA Inference Through
Deterministic Split-K Reduction" (Balusamy & Mohan) it writes out.

Pinning status (what checks each function against something other than itself;
the tests live in ``tests/test_oracle.py``):

* ``bf16_rne``        - the bf16 values printed in section 6.2 / Fig. 5 of the
                        paper (tests/golden/bf16_rne_paper.json), exhaustive
                        comparison with an independent bit-level rounding on
                        every fp32 pattern class, ties, subnormals, overflow.
* ``shrink``          - exact rational brute force on tiny inputs; integer
                        inputs (exact in any order); zero / one-hot special
                        cases; the associativity identity (x A^T) B^T = x (A^T B^T).
* ``split_partials``  - sums of the partials equal the shrink (Eq. 3);
                        one-hot inputs place each product in its partition.
* ``combine_tree_f32``/``combine_sequential_f32`` - the Eq. 4 worked example of
                        the paper (10^30, -10^30, 1) and the crafted partials
                        (2^100, 1, -2^100, 1) whose tree / sequential results
                        are 0 / 1 by hand.
* ``expand``          - exact rational brute force; B = 0 leaves y bitwise
                        unchanged; integer inputs exact; the bf16 conversion of
                        h pinned by the paper's midpoint value.
* ``sgmv_*``          - per-token equality with the single-adapter functions,
                        invalid ids leave rows untouched.
* ``shrink_bounds``   - hand values on a 2 x 4 case with Pythagorean rows
                        (norms 5, 13 and 1, 3) and mixed signs (sum|xA| = 22
                        where the signed sum is 2); exact rationals on random
                        tiny inputs; the Cauchy-Schwarz chain
                        |h| <= sum|xA| <= ||x|| ||A|| on random inputs.
* ``shrink_tolerance``- the same hand case with scale -2 (a transposed outer
                        product, a lost |scale| or a squared norm all fail).
* ``bf16_ulp``        - hand values at 1, 2, below 2, the smallest and largest
                        subnormal, the smallest normal, zero and the largest
                        finite value; every finite bf16 pattern against the
                        gap to its successor (computed from the successor's
                        bits, not from the exponent field).
* ``expand_compensated`` - exact rational brute force (``exact.py``); the
                        hand-derived cases of tests/golden/compensated_expand.json
                        (where it and the plain expand differ); hi + lo equals h
                        for every h with at most 16 significant bits; equal to
                        ``expand`` when h is already bf16.  Follows the HEAL page
                        ("Demystifying Numerical Instability in LLM Inference"),
                        section 3, Eq. 10, read with bf16 halves.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC"]


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (a CPU library; no GPU code)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-lm", "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        L.oracle_bf16_to_double.restype = ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_rne_from_double.restype = ctypes.c_uint16
        L.oracle_bf16_rne_from_double.argtypes = [ctypes.c_double]
        L.oracle_bf16_rne_from_float.restype = ctypes.c_uint16
        L.oracle_bf16_rne_from_float.argtypes = [ctypes.c_float]
        L.oracle_bf16_rne_array.argtypes = [_f64p, _i64, _u16p]
        L.oracle_shrink.argtypes = [_u16p, _u16p, _i64, _i64, _i64, ctypes.c_double, _f64p]
        L.oracle_shrink_bounds.argtypes = [_u16p, _u16p, _i64, _i64, _i64, _f64p, _f64p, _f64p]
        L.oracle_split_partials.argtypes = [_u16p, _u16p, _i64, _i64, _i64, _i64, _f64p]
        L.oracle_combine_tree_f32.argtypes = [_f32p, _i64, _i64, ctypes.c_float, _f32p]
        L.oracle_combine_sequential_f32.argtypes = [_f32p, _i64, _i64, ctypes.c_float, _f32p]
        L.oracle_expand.argtypes = [_f32p, _u16p, _u16p, _i64, _i64, _i64, ctypes.c_double,
                                    _f64p, _u16p, _f64p]
        L.oracle_expand_compensated.argtypes = [_f32p, _u16p, _u16p, _i64, _i64, _i64, ctypes.c_double,
                                                _f64p, _u16p, _f64p]
        L.oracle_sgmv_shrink.argtypes = [_u16p, ctypes.POINTER(_u16p), _i32p, _f32p, _i32p,
                                         ctypes.c_int32, _i64, _i64, _i64, _f64p]
        L.oracle_sgmv_expand.argtypes = [_f32p, ctypes.POINTER(_u16p), _i32p, _f32p, _i32p,
                                         ctypes.c_int32, _u16p, _i64, _i64, _i64, _f64p, _u16p, _f64p]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _p(a: np.ndarray, ptype):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ptype)


def _u16(a):
    return np.ascontiguousarray(a, dtype=np.uint16)


# ----------------------------------------------------------------------------
# bf16 helpers
# ----------------------------------------------------------------------------
def bf16_to_f64(bits) -> np.ndarray:
    b = _u16(np.atleast_1d(bits))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(np.shape(bits))


def bf16_rne(values) -> np.ndarray:
    """Round float64 (or float32) values to bf16, nearest-even, one rounding."""
    v = np.ascontiguousarray(np.asarray(values, dtype=np.float64))
    out = np.empty(v.shape, dtype=np.uint16)
    lib().oracle_bf16_rne_array(_p(v.reshape(-1), _f64p), v.size, _p(out.reshape(-1), _u16p))
    return out


# ----------------------------------------------------------------------------
# Shrink (Eq. 1 / Eq. 3)
# ----------------------------------------------------------------------------
def shrink(x, A, scale: float = 1.0) -> np.ndarray:
    """h[i][j] = scale * sum_k x[i][k] A[j][k] in float64.  x [M,K], A [r,K] bf16 bits."""
    x, A = _u16(x), _u16(A)
    M, K = x.shape
    r = A.shape[0]
    assert A.shape[1] == K
    h = np.empty((M, r), dtype=np.float64)
    lib().oracle_shrink(_p(x, _u16p), _p(A, _u16p), M, K, r, float(scale), _p(h, _f64p))
    return h


def shrink_bounds(x, A):
    """(sum_k |x A|  [M,r], ||x_i||  [M], ||A_j|| [r])."""
    x, A = _u16(x), _u16(A)
    M, K = x.shape
    r = A.shape[0]
    s = np.empty((M, r), dtype=np.float64)
    xn = np.empty((M,), dtype=np.float64)
    an = np.empty((r,), dtype=np.float64)
    lib().oracle_shrink_bounds(_p(x, _u16p), _p(A, _u16p), M, K, r, _p(s, _f64p), _p(xn, _f64p),
                               _p(an, _f64p))
    return s, xn, an


def split_partials(x, A, S: int) -> np.ndarray:
    """P[s][i][j] = sum over the s-th contiguous K/S chunk, float64.  [S, M, r]."""
    x, A = _u16(x), _u16(A)
    M, K = x.shape
    r = A.shape[0]
    assert K % S == 0
    P = np.empty((S, M, r), dtype=np.float64)
    lib().oracle_split_partials(_p(x, _u16p), _p(A, _u16p), M, K, r, S, _p(P, _f64p))
    return P


def combine_tree_f32(P, scale: float = 1.0) -> np.ndarray:
    """Fixed pairwise tree over axis 0 of fp32 partials P [S, ...], then x scale."""
    P = np.ascontiguousarray(P, dtype=np.float32)
    S = P.shape[0]
    assert S >= 1 and (S & (S - 1)) == 0 and S <= 64
    n = P[0].size
    out = np.empty(P.shape[1:], dtype=np.float32)
    lib().oracle_combine_tree_f32(_p(P.reshape(-1), _f32p), S, n, float(scale), _p(out.reshape(-1), _f32p))
    return out


def combine_sequential_f32(P, scale: float = 1.0) -> np.ndarray:
    """Sequential fold in increasing partition order, fp32, then x scale."""
    P = np.ascontiguousarray(P, dtype=np.float32)
    S = P.shape[0]
    n = P[0].size
    out = np.empty(P.shape[1:], dtype=np.float32)
    lib().oracle_combine_sequential_f32(_p(P.reshape(-1), _f32p), S, n, float(scale),
                                        _p(out.reshape(-1), _f32p))
    return out


# ----------------------------------------------------------------------------
# Expand (Eq. 1)
# ----------------------------------------------------------------------------
def expand(h, B, y, scale: float):
    """Returns (y_out bf16 bits [M,N], e float64 [M,N], sum|s hb B| [M,N]).

    h fp32 [M,r] (the exact bits the GPU expand consumed), B bf16 [N,r],
    y bf16 [M,N]."""
    h = np.ascontiguousarray(h, dtype=np.float32)
    B, y = _u16(B), _u16(y)
    M, r = h.shape
    N = B.shape[0]
    assert B.shape[1] == r and y.shape == (M, N)
    e = np.empty((M, N), dtype=np.float64)
    yo = np.empty((M, N), dtype=np.uint16)
    ab = np.empty((M, N), dtype=np.float64)
    lib().oracle_expand(_p(h, _f32p), _p(B, _u16p), _p(y, _u16p), M, r, N, float(scale),
                        _p(e, _f64p), _p(yo, _u16p), _p(ab, _f64p))
    return yo, e, ab


def expand_compensated(h, B, y, scale: float):
    """The compensated expand (h split into bf16 hi + bf16 lo of the residual,
    the two products summed); returns (y_out, e, sum|s (hi + lo) B|) like
    expand()."""
    h = np.ascontiguousarray(h, dtype=np.float32)
    B, y = _u16(B), _u16(y)
    M, r = h.shape
    N = B.shape[0]
    assert B.shape[1] == r and y.shape == (M, N)
    e = np.empty((M, N), dtype=np.float64)
    yo = np.empty((M, N), dtype=np.uint16)
    ab = np.empty((M, N), dtype=np.float64)
    lib().oracle_expand_compensated(_p(h, _f32p), _p(B, _u16p), _p(y, _u16p), M, r, N, float(scale),
                                    _p(e, _f64p), _p(yo, _u16p), _p(ab, _f64p))
    return yo, e, ab


# ----------------------------------------------------------------------------
# Multi-adapter (mapping information: one adapter id per token)
# ----------------------------------------------------------------------------
def _ptr_array(mats):
    arr = (_u16p * len(mats))()
    for i, m in enumerate(mats):
        arr[i] = _p(m, _u16p)
    return arr


def sgmv_shrink(x, As, ranks, scales, ids, r_max: int) -> np.ndarray:
    x = _u16(x)
    As = [_u16(a) for a in As]
    ranks = np.ascontiguousarray(ranks, dtype=np.int32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    M, K = x.shape
    sc = None if scales is None else np.ascontiguousarray(scales, dtype=np.float32)
    h = np.empty((M, r_max), dtype=np.float64)
    lib().oracle_sgmv_shrink(_p(x, _u16p), _ptr_array(As), _p(ranks, _i32p),
                             None if sc is None else _p(sc, _f32p), _p(ids, _i32p), len(As),
                             M, K, r_max, _p(h, _f64p))
    return h


def sgmv_expand(h, Bs, ranks, scales, ids, y):
    h = np.ascontiguousarray(h, dtype=np.float32)
    Bs = [_u16(b) for b in Bs]
    y = _u16(y)
    ranks = np.ascontiguousarray(ranks, dtype=np.int32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    M, r_max = h.shape
    N = y.shape[1]
    sc = None if scales is None else np.ascontiguousarray(scales, dtype=np.float32)
    e = np.empty((M, N), dtype=np.float64)
    yo = np.empty((M, N), dtype=np.uint16)
    ab = np.empty((M, N), dtype=np.float64)
    lib().oracle_sgmv_expand(_p(h, _f32p), _ptr_array(Bs), _p(ranks, _i32p),
                             None if sc is None else _p(sc, _f32p), _p(ids, _i32p), len(Bs),
                             _p(y, _u16p), M, N, r_max, _p(e, _f64p), _p(yo, _u16p), _p(ab, _f64p))
    return yo, e, ab


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_threads(n: int) -> int:
    """Thread count for later calls; returns the previous one."""
    return int(lib().oracle_set_threads(int(n)))


# ----------------------------------------------------------------------------
# Tolerances.  Both follow from the arithmetic and are applied by the tests.
# ----------------------------------------------------------------------------
def shrink_tolerance(x, A, scale: float = 1.0) -> np.ndarray:
    """Per-element bound for an fp32 shrink: 1e-3 * |scale| * ||x_i||_2 * ||A_j||_2
    for element (i, j) (token i, rank j): the Cauchy-Schwarz bound of that dot
    product, scaled by 1e-3.  Shape [M, r]."""
    _, xn, an = shrink_bounds(x, A)
    return 1e-3 * abs(scale) * np.outer(xn, an)


def bf16_ulp(bits) -> np.ndarray:
    """Spacing of the bf16 values in the binade of |v| (v given as bf16 bits),
    i.e. the distance from |v| to the next bf16 magnitude above it, taken as
    if the exponent range were unbounded: 2^(E-7) for 2^E <= |v| < 2^(E+1)
    (8 significant bits), 2^-133 for the subnormals and zero.  At a power of
    two this is the larger of the two neighbouring gaps, and at the largest
    finite value it is 2^120 (the gap to the next value is not infinite).
    NaN for infinities and NaNs."""
    b = _u16(bits).astype(np.int64) & 0x7FFF
    e = b >> 7                                    # biased exponent field
    out = np.where(e == 0, 2.0 ** -133, np.exp2(np.maximum(e, 1) - 127 - 7))
    return np.where(e == 0xFF, np.nan, out).reshape(np.shape(bits))

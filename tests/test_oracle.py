"""Pins for the CPU oracle: each check ties an oracle function to something other
than itself - numbers printed in "Reproducible LoRA Inference Through
Deterministic Split-K Reduction" (Balusamy & Mohan), exact rational brute force,
closed forms and special cases - so a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails here.  CPU only."""
import json
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import exact
from synth import integer_bf16, normal_bf16, bf16_bits_to_f32

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _bits_to_f64(b):
    return oracle.bf16_to_f64(np.asarray(b, dtype=np.uint16))


# ---------------------------------------------------------------------------
# bf16 round-to-nearest-even
# ---------------------------------------------------------------------------
def test_bf16_rne_paper_vectors():
    g = _gold("bf16_rne_paper.json")
    for pair in g["pairs"]:
        v = np.array(pair["fp32"], dtype=np.float64)
        assert np.all(v.astype(np.float32).astype(np.float64) == v), "printed values are fp32 values"
        got = _bits_to_f64(oracle.bf16_rne(v))
        assert got.tolist() == pair["bf16"]
        # the printed differences
        assert abs(abs(v[0] - v[1]) - pair["fp32_printed_difference"]) < 0.01 * pair["fp32_printed_difference"]
        assert abs(abs(got[0] - got[1]) - pair["bf16_printed_difference"]) < 0.01 * pair["bf16_printed_difference"]
        # float32 entry point agrees
        for k in range(2):
            b = oracle.lib().oracle_bf16_rne_from_float(float(np.float32(v[k])))
            assert _bits_to_f64([b])[0] == pair["bf16"][k]
        if "printed_midpoint" in pair:
            mid = pair["printed_midpoint"]
            # the midpoint is halfway between the two printed bf16 results
            assert Fraction(mid) == (Fraction(pair["bf16"][0]) + Fraction(pair["bf16"][1])) / 2
            # ... and ties to the neighbour with an even significand
            assert _bits_to_f64(oracle.bf16_rne([mid]))[0] == -0.38671875
        if pair["first_is_midpoint"]:
            q = Fraction(pair["fp32"][0])
            lo, hi = Fraction(pair["bf16"][1]), Fraction(pair["bf16"][0])
            assert q == (lo + hi) / 2


def _bitlevel_rne_f32(u32):
    """Independent fp32 -> bf16 rounding on the bit pattern: add 0x7FFF plus the
    lowest kept bit, then drop 16 bits (nearest, ties to even).  NaNs are
    quieted separately."""
    u = u32.astype(np.uint64)
    exp_all_ones = (u & 0x7F800000) == 0x7F800000
    is_nan = exp_all_ones & ((u & 0x007FFFFF) != 0)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = np.where(is_nan, (u >> 16) | 0x0040, r)
    return r.astype(np.uint16)


def test_bf16_rne_matches_bitlevel_rounding_on_fp32():
    rng = np.random.default_rng(1234)
    u = rng.integers(0, 2 ** 32, size=300_000, dtype=np.uint64).astype(np.uint32)
    # every exponent with ties, ties +- 1 and the largest finite values
    exps = np.arange(0, 255, dtype=np.uint32) << 23
    extra = []
    for low in (0x8000, 0x7FFF, 0x8001, 0x18000, 0x17FFF, 0x0, 0xFFFF, 0x10000):
        extra.append(exps | np.uint32(low))
        extra.append(exps | np.uint32(low) | np.uint32(0x80000000))
    extra.append(np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00000001, 0x00008000, 0x00018000,
                           0x7F800000, 0xFF800000, 0x7FC00000, 0x80000000], dtype=np.uint32))
    u = np.concatenate([u] + extra).astype(np.uint32)
    with np.errstate(invalid="ignore"):
        f = u.view(np.float32).astype(np.float64)
    got = oracle.bf16_rne(f)
    want = _bitlevel_rne_f32(u)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all((got[nan] & 0x7F) != 0)


def test_bf16_rne_matches_exact_rational_on_doubles():
    rng = np.random.default_rng(99)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 38, 3000))
    # doubles just off and exactly on bf16 midpoints (not fp32 values)
    for e in (-130, -127, -126, -20, 0, 5, 127):
        for m in (129.5, 130.5, 255.5, 128.5):
            mid = m * 2.0 ** (e - 7)
            vals += [mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf), -mid]
    vals = np.array(vals, dtype=np.float64)
    got = oracle.bf16_rne(vals)
    for v, b in zip(vals, got):
        want = exact.rne_bf16(Fraction(float(v)))
        if isinstance(want, float):
            assert (int(b) & 0x7FFF) == 0x7F80
        else:
            assert Fraction(float(_bits_to_f64([b])[0])) == want, v


# ---------------------------------------------------------------------------
# shrink
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,r,seed", [(1, 8, 1, 0), (3, 32, 4, 1), (4, 64, 3, 2), (2, 48, 2, 3)])
def test_shrink_against_exact_rationals(M, K, r, seed):
    x = normal_bf16((M, K), 1.0, seed, "x")
    A = normal_bf16((r, K), 0.5, seed, "A")
    scale = 0.75
    h = oracle.shrink(x, A, scale)
    ex = exact.shrink(x, A, Fraction(scale))
    absum, _, _ = oracle.shrink_bounds(x, A)
    for i in range(M):
        for j in range(r):
            err = abs(Fraction(float(h[i, j])) - ex[i][j])
            assert err <= Fraction(K + 2) * Fraction(1, 2 ** 53) * Fraction(float(absum[i, j])) + Fraction(1, 2 ** 1000)


def test_shrink_integer_inputs_exact():
    M, K, r = 7, 256, 5
    x = integer_bf16((M, K), -4, 4, 5, "xi")
    A = integer_bf16((r, K), -4, 4, 5, "Ai")
    h = oracle.shrink(x, A, 1.0)
    xi = bf16_bits_to_f32(x).astype(np.int64)
    Ai = bf16_bits_to_f32(A).astype(np.int64)
    assert np.array_equal(h, (xi @ Ai.T).astype(np.float64))


def test_shrink_special_cases():
    M, K, r = 3, 64, 4
    x = normal_bf16((M, K), 1.0, 7, "x")
    A0 = np.zeros((r, K), dtype=np.uint16)
    assert np.all(oracle.shrink(x, A0, 2.0) == 0.0)
    # one nonzero k: h[i][j] = x[i][k] * A[j][k] exactly; distinct values per (i, j)
    A = normal_bf16((r, K), 1.0, 7, "A")
    k = 37
    x1 = np.zeros_like(x)
    x1[:, k] = x[:, k]
    h = oracle.shrink(x1, A, 1.0)
    xv = _bits_to_f64(x[:, k])
    Av = _bits_to_f64(A[:, k])
    assert np.array_equal(h, np.outer(xv, Av))


def test_shrink_then_expand_associativity_identity():
    """(x A^T) B^T == x (A^T B^T) with integer values small enough that every
    intermediate (h, the bf16 rounding of h, and y) is exact: a transposed or
    mis-indexed operand in either function breaks the identity."""
    M, K, r, N = 5, 64, 3, 11
    x = integer_bf16((M, K), -2, 2, 11, "x")
    A = integer_bf16((r, K), -1, 1, 11, "A")
    B = integer_bf16((N, r), -2, 2, 11, "B")
    y = integer_bf16((M, N), -8, 8, 11, "y")
    h = oracle.shrink(x, A, 1.0)
    assert np.all(np.abs(h) <= 128)              # exact in bf16
    yo, e, _ = oracle.expand(h.astype(np.float32), B, y, 2.0)
    xm = bf16_bits_to_f32(x).astype(np.int64)
    Am = bf16_bits_to_f32(A).astype(np.int64)    # [r, K]
    Bm = bf16_bits_to_f32(B).astype(np.int64)    # [N, r]
    ym = bf16_bits_to_f32(y).astype(np.int64)
    W = Am.T @ Bm.T                              # [K, N]: the merged low-rank update
    want = ym + 2 * (xm @ W)
    assert np.array_equal(e, want.astype(np.float64))
    assert np.all(np.abs(want) <= 256)
    assert np.array_equal(_bits_to_f64(yo), want.astype(np.float64))


# ---------------------------------------------------------------------------
# Split-K partials and the fixed-order combine
# ---------------------------------------------------------------------------
def test_split_partials_sum_to_shrink_and_place_products():
    M, K, r, S = 3, 128, 4, 8
    x = integer_bf16((M, K), -3, 3, 4, "x")
    A = integer_bf16((r, K), -3, 3, 4, "A")
    P = oracle.split_partials(x, A, S)
    assert np.array_equal(P.sum(axis=0), oracle.shrink(x, A, 1.0))
    # a single product at k lands in partition k // (K/S) only
    for k in (0, 15, 16, 77, 127):
        x1 = np.zeros_like(x)
        A1 = np.zeros_like(A)
        x1[0, k] = x[0, k] | 0x3F80 if x[0, k] == 0 else x[0, k]
        A1[1, k] = 0x4000                        # 2.0
        P1 = oracle.split_partials(x1, A1, S)
        nz = {int(s) for s in np.nonzero(P1)[0]}
        assert nz == {k // (K // S)}


def test_combine_eq4_worked_example():
    g = _gold("eq4_nonassociativity.json")
    a, b, c = g["a"], g["b"], g["c"]
    # sequential: (a + b) + c
    assert oracle.combine_sequential_f32(np.array([[a], [b], [c]]))[0] == g["left_to_right"]
    # pairwise tree over [a, b, c, 0]: (a + b) + (c + 0)
    assert oracle.combine_tree_f32(np.array([[a], [b], [c], [0.0]]))[0] == g["left_to_right"]
    # pairwise tree over [b, c, a, 0]: (b + c) + (a + 0) = a + (b + c)
    assert oracle.combine_tree_f32(np.array([[b], [c], [a], [0.0]]))[0] == g["right_first"]


def test_combine_crafted_partials():
    g = _gold("crafted_partials.json")
    P = np.array(g["partials"], dtype=np.float64).reshape(8, 1)
    assert P[0, 0] == 2.0 ** 100
    assert oracle.combine_tree_f32(P)[0] == g["neighbour_pairwise_tree"]
    assert oracle.combine_sequential_f32(P)[0] == g["increasing_partition_order_fold"]
    # the scale is applied once, after the sum
    assert oracle.combine_sequential_f32(P, 2.0)[0] == 2.0 * g["increasing_partition_order_fold"]
    # every order of a sequential fold lands in the documented set
    import itertools
    seen = set()
    for perm in itertools.permutations(range(8)):
        seen.add(float(oracle.combine_sequential_f32(P[list(perm)])[0]))
    assert seen == set(g["any_order_results"])


def test_combine_tree_is_fp32_and_pairs_neighbours():
    # fp32 (not double) arithmetic: 1 + 2^-24 + 2^-24 ... rounds in fp32
    P = np.array([[1.0], [2.0 ** -24], [2.0 ** -24], [0.0]])
    # (1 + 2^-24) = 1 in fp32 (tie to even), (2^-24 + 0) = 2^-24, 1 + 2^-24 = 1
    assert oracle.combine_tree_f32(P)[0] == 1.0
    Q = np.array([[2.0 ** -24], [2.0 ** -24], [1.0], [0.0]])
    # (2^-24 + 2^-24) = 2^-23, (1 + 0) = 1, 2^-23 + 1 = 1 + 2^-23 exactly
    assert oracle.combine_tree_f32(Q)[0] == np.float32(1.0 + 2.0 ** -23)
    # S = 1 is the identity times the scale; S = 16 is four levels
    assert oracle.combine_tree_f32(np.array([[3.0]]), 2.0)[0] == 6.0
    R = np.zeros((16, 1))
    R[0, 0], R[8, 0], R[15, 0] = 2.0 ** 30, -2.0 ** 30, 1.0
    # levels: ... (P0..P7) = 2^30, (P8..P15) = -2^30 + 1 = -2^30 (fp32) -> 0
    assert oracle.combine_tree_f32(R)[0] == 0.0


# ---------------------------------------------------------------------------
# expand
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,r,N,seed", [(1, 1, 3, 0), (2, 4, 5, 1), (3, 8, 4, 2)])
def test_expand_against_exact_rationals(M, r, N, seed):
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal((M, r)) * 0.3).astype(np.float32)
    B = normal_bf16((N, r), 0.5, seed, "B")
    y = normal_bf16((M, N), 1.0, seed, "y")
    yo, e, _ = oracle.expand(h, B, y, 2.0)
    O, E = exact.expand(h, B, y, 2.0)
    assert yo.tolist() == O
    for i in range(M):
        for n in range(N):
            assert abs(Fraction(float(e[i, n])) - E[i][n]) <= \
                abs(E[i][n]) * Fraction(r + 2, 2 ** 52) + Fraction(1, 2 ** 200)


def test_expand_B_zero_leaves_y_bitwise():
    M, r, N = 4, 16, 64
    h = np.random.default_rng(3).standard_normal((M, r)).astype(np.float32)
    y = normal_bf16((M, N), 1.0, 3, "y")
    yo, _, _ = oracle.expand(h, np.zeros((N, r), np.uint16), y, 2.0)
    assert np.array_equal(yo, y)


def test_expand_integer_exact():
    M, r, N = 3, 8, 9
    h = np.random.default_rng(4).integers(-3, 4, (M, r)).astype(np.float32)
    B = integer_bf16((N, r), -3, 3, 4, "B")
    y = integer_bf16((M, N), -10, 10, 4, "y")
    yo, e, _ = oracle.expand(h, B, y, 2.0)
    want = bf16_bits_to_f32(y).astype(np.int64) + 2 * (h.astype(np.int64) @ bf16_bits_to_f32(B).astype(np.int64).T)
    assert np.array_equal(e, want.astype(np.float64))
    assert np.array_equal(_bits_to_f64(yo), want.astype(np.float64))


def test_expand_rounds_h_to_bf16_first():
    """The paper's midpoint value 0.010345458984375 = 169.5 * 2^-14 must become
    170 * 2^-14 before it meets B.  With B = 1, y = 0 and scale 3 the result is
    3 * 170 * 2^-14 = 255 * 2^-13 (exact in bf16); skipping the conversion
    would give 3 * 169.5 * 2^-14 = 254.25 * 2^-13, which rounds to 254 * 2^-13."""
    h = np.array([[0.010345458984375]], dtype=np.float32)
    B = np.array([[0x3F80]], dtype=np.uint16)     # 1.0
    y = np.zeros((1, 1), dtype=np.uint16)
    yo, e, _ = oracle.expand(h, B, y, 3.0)
    assert e[0, 0] == 255 * 2.0 ** -13
    assert _bits_to_f64(yo)[0, 0] == 255 * 2.0 ** -13
    # the second printed value rounds to 169 * 2^-14 first: 507 * 2^-14 -> bf16
    h2 = np.array([[0.010345457121729851]], dtype=np.float32)
    yo2, e2, _ = oracle.expand(h2, B, y, 3.0)
    assert e2[0, 0] == 507 * 2.0 ** -14
    assert _bits_to_f64(yo2)[0, 0] == 254 * 2.0 ** -13     # 253.5 ties to even 254


# ---------------------------------------------------------------------------
# multi-adapter
# ---------------------------------------------------------------------------
def test_sgmv_matches_single_adapter_per_token():
    M, K, N = 9, 64, 24
    ranks = np.array([8, 16, 4], dtype=np.int32)
    x = normal_bf16((M, K), 1.0, 21, "x")
    As = [normal_bf16((int(r), K), 0.1, 21, f"A{a}") for a, r in enumerate(ranks)]
    Bs = [normal_bf16((N, int(r)), 0.1, 21, f"B{a}") for a, r in enumerate(ranks)]
    y = normal_bf16((M, N), 1.0, 21, "y")
    ids = np.array([0, 0, 2, -1, 1, 1, 7, 2, 0], dtype=np.int32)
    scales = np.array([2.0, 0.5, 1.0], dtype=np.float32)
    r_max = 16
    h = oracle.sgmv_shrink(x, As, ranks, scales, ids, r_max)
    hf = h.astype(np.float32)
    yo, e, _ = oracle.sgmv_expand(hf, Bs, ranks, scales, ids, y)
    for i in range(M):
        a = ids[i]
        if a < 0 or a >= len(ranks):
            assert np.all(h[i] == 0.0)
            assert np.array_equal(yo[i], y[i])
            continue
        r = int(ranks[a])
        hs = oracle.shrink(x[i:i + 1], As[a], float(scales[a]))
        assert np.array_equal(h[i, :r], hs[0])
        assert np.all(h[i, r:] == 0.0)
        ys, es, _ = oracle.expand(hf[i:i + 1, :r], Bs[a], y[i:i + 1], float(scales[a]))
        assert np.array_equal(yo[i], ys[0])
        assert np.array_equal(e[i], es[0])


# ---------------------------------------------------------------------------
# compensated expand (h split into bf16 hi + bf16 lo of the residual)
# ---------------------------------------------------------------------------
def _exact_bf16_bits(vals):
    """bf16 bits of values that are exactly bf16 numbers (checked)."""
    a = np.asarray(vals, dtype=np.float32)
    u = a.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def test_expand_compensated_golden_cases():
    """The hand-derived cases: the compensated expand keeps the residual of h
    that the plain expand drops when h is rounded to bf16."""
    for c in _gold("compensated_expand.json")["cases"]:
        h = np.array(c["h"], dtype=np.float32)
        B = _exact_bf16_bits(c["B"])
        y = _exact_bf16_bits(c["y"])
        yo, e, _ = oracle.expand_compensated(h, B, y, c["scale"])
        assert np.array_equal(_bits_to_f64(yo), np.array(c["compensated_out"])), c["name"]
        assert np.array_equal(e, np.array(c["compensated_out"])), c["name"]
        yp, _, _ = oracle.expand(h, B, y, c["scale"])
        assert np.array_equal(_bits_to_f64(yp), np.array(c["plain_out"])), c["name"]
        O, E = exact.expand_compensated(h, B, y, c["scale"])
        assert O == yo.tolist() and float(E[0][0]) == c["compensated_out"][0][0], c["name"]


@pytest.mark.parametrize("M,r,N,seed", [(1, 1, 3, 0), (2, 4, 5, 1), (3, 8, 4, 2)])
def test_expand_compensated_against_exact_rationals(M, r, N, seed):
    rng = np.random.default_rng(100 + seed)
    h = (rng.standard_normal((M, r)) * 0.3).astype(np.float32)      # full 24-bit significands
    B = normal_bf16((N, r), 0.5, seed, "cB")
    y = normal_bf16((M, N), 1.0, seed, "cy")
    yo, e, _ = oracle.expand_compensated(h, B, y, 2.0)
    O, E = exact.expand_compensated(h, B, y, 2.0)
    assert yo.tolist() == O
    for i in range(M):
        for n in range(N):
            assert abs(Fraction(float(e[i, n])) - E[i][n]) <= abs(E[i][n]) * Fraction(2 * r + 2, 2 ** 52) + \
                Fraction(1, 2 ** 200)


def test_expand_compensated_recovers_16_bit_inputs_exactly():
    """With B = 1, y = 0 and scale 1 the compensated expand returns hi + lo
    before rounding.  That sum equals h for every h with at most 16
    significant bits (the residual of an 8-bit rounding then has at most 8
    bits), and is within 2^-16 relative of h for full fp32 h; the plain
    expand is only within 2^-8."""
    rng = np.random.default_rng(7)
    n = 4000
    sig = rng.integers(2 ** 15, 2 ** 16, n)                     # exactly 16 significant bits
    ex = rng.integers(-40, 20, n)
    sign = rng.choice([-1.0, 1.0], n)
    h16 = (sign * sig * np.exp2(ex - 15.0)).astype(np.float32)
    assert np.all(h16.astype(np.float64) == sign * sig * np.exp2(ex - 15.0))
    one = _exact_bf16_bits([[1.0]])
    zero = np.zeros((1, 1), np.uint16)
    for v in h16[:600]:
        _, e, _ = oracle.expand_compensated(np.array([[v]], np.float32), one, zero, 1.0)
        assert e[0, 0] == float(v)
    hf = (rng.standard_normal(600) * np.exp2(rng.integers(-30, 30, 600))).astype(np.float32)
    worst_c = worst_p = 0.0
    for v in hf:
        _, ec, _ = oracle.expand_compensated(np.array([[v]], np.float32), one, zero, 1.0)
        _, ep, _ = oracle.expand(np.array([[v]], np.float32), one, zero, 1.0)
        worst_c = max(worst_c, abs(ec[0, 0] - float(v)) / abs(float(v)))
        worst_p = max(worst_p, abs(ep[0, 0] - float(v)) / abs(float(v)))
    assert worst_c <= 2.0 ** -16 and worst_p <= 2.0 ** -8 and worst_c < worst_p / 64


def test_expand_compensated_equals_plain_for_bf16_inputs():
    """When h is already a bf16 value the residual is 0 and both expands agree."""
    M, r, N = 3, 16, 40
    hb = normal_bf16((M, r), 0.5, 9, "ch")
    h = bf16_bits_to_f32(hb).astype(np.float32)
    B = normal_bf16((N, r), 0.02, 9, "cB2")
    y = normal_bf16((M, N), 1.0, 9, "cy2")
    a, ea, _ = oracle.expand_compensated(h, B, y, 2.0)
    b, eb, _ = oracle.expand(h, B, y, 2.0)
    assert np.array_equal(a, b) and np.array_equal(ea, eb)


# ---------------------------------------------------------------------------
# tolerance helpers: the norms, |x A| sums and bf16 spacing the parity tests
# compare against (a slip here would silently loosen every GPU check)
# ---------------------------------------------------------------------------
def _bf16_exact(vals):
    return _exact_bf16_bits(np.asarray(vals, dtype=np.float64))


def test_shrink_bounds_hand_values():
    """x rows (3, 4, 0, 0) and (0, 0, 5, 12) have norms 5 and 13; A rows
    (1, 0, 0, 0) and (0, 2, -2, 1) have norms 1 and 3.  sum_k |x_ik A_jk|:
    (0,0) 3, (0,1) 8, (1,0) 0, (1,1) |5 * -2| + |12 * 1| = 22, where the signed
    sum is 2.  Norms over the wrong axis would have length K = 4, not 2."""
    x = _bf16_exact([[3, 4, 0, 0], [0, 0, 5, 12]])
    A = _bf16_exact([[1, 0, 0, 0], [0, 2, -2, 1]])
    absum, xn, an = oracle.shrink_bounds(x, A)
    assert xn.shape == (2,) and an.shape == (2,) and absum.shape == (2, 2)
    assert xn.tolist() == [5.0, 13.0]
    assert an.tolist() == [1.0, 3.0]
    assert absum.tolist() == [[3.0, 8.0], [0.0, 22.0]]
    assert oracle.shrink(x, A, 1.0).tolist() == [[3.0, 8.0], [0.0, 2.0]]


def test_shrink_tolerance_hand_values():
    """1e-3 |s| ||x_i|| ||A_j|| with s = -2 on the case above:
    [[10, 30], [26, 78]] * 1e-3 (the transpose would be [[10, 26], [30, 78]])."""
    x = _bf16_exact([[3, 4, 0, 0], [0, 0, 5, 12]])
    A = _bf16_exact([[1, 0, 0, 0], [0, 2, -2, 1]])
    tol = oracle.shrink_tolerance(x, A, -2.0)
    want = np.array([[10.0, 30.0], [26.0, 78.0]]) * 1e-3
    assert tol.shape == (2, 2)
    assert np.allclose(tol, want, rtol=1e-15, atol=0)
    # M != r: the shape follows (tokens, ranks)
    x3 = _bf16_exact([[3, 4, 0, 0], [0, 0, 5, 12], [1, 0, 0, 0]])
    assert oracle.shrink_tolerance(x3, A, 1.0).shape == (3, 2)


@pytest.mark.parametrize("M,K,r,seed", [(2, 8, 3, 0), (3, 24, 2, 1), (1, 64, 4, 2)])
def test_shrink_bounds_against_exact_rationals(M, K, r, seed):
    import math
    x = normal_bf16((M, K), 1.0, seed, "bx")
    A = normal_bf16((r, K), 0.5, seed, "bA")
    absum, xn, an = oracle.shrink_bounds(x, A)
    X = [[exact.bf16_bits_to_fraction(v) for v in row] for row in x]
    Am = [[exact.bf16_bits_to_fraction(v) for v in row] for row in A]
    for i in range(M):
        sq = sum(v * v for v in X[i])
        assert abs(xn[i] - math.sqrt(float(sq))) <= 2.0 ** -50 * xn[i]
        for j in range(r):
            s = sum(abs(X[i][k] * Am[j][k]) for k in range(K))
            assert abs(Fraction(float(absum[i, j])) - s) <= s * Fraction(K, 2 ** 53)
    for j in range(r):
        sq = sum(v * v for v in Am[j])
        assert abs(an[j] - math.sqrt(float(sq))) <= 2.0 ** -50 * an[j]


def test_shrink_bounds_cauchy_schwarz_chain():
    """|h_ij| <= sum_k |x_ik A_jk| <= ||x_i|| ||A_j|| on random inputs, with
    the middle inequality strict somewhere (it is not an identity)."""
    x = normal_bf16((6, 512), 1.0, 3, "cx")
    A = normal_bf16((5, 512), 0.02, 3, "cA")
    h = oracle.shrink(x, A, 1.0)
    absum, xn, an = oracle.shrink_bounds(x, A)
    cs = np.outer(xn, an)
    assert np.all(np.abs(h) <= absum * (1 + 1e-12))
    assert np.all(absum <= cs * (1 + 1e-12))
    assert np.any(absum < 0.9 * cs) and np.any(np.abs(h) < 0.5 * absum)


def test_bf16_ulp_hand_values():
    cases = {
        0x3F80: 2.0 ** -7,       # 1.0
        0xBF80: 2.0 ** -7,       # -1.0: the sign does not matter
        0x3FFF: 2.0 ** -7,       # 1.9921875, the last value below 2
        0x4000: 2.0 ** -6,       # 2.0: the gap above a power of two
        0x0000: 2.0 ** -133,     # +0
        0x8000: 2.0 ** -133,     # -0
        0x0001: 2.0 ** -133,     # smallest subnormal
        0x007F: 2.0 ** -133,     # largest subnormal
        0x0080: 2.0 ** -133,     # smallest normal 2^-126
        0x0100: 2.0 ** -132,     # 2^-125
        0x7F7F: 2.0 ** 120,      # largest finite (2 - 2^-7) 2^127: finite spacing
        0x3C23: 2.0 ** -14,      # 0.00994873046875 = 163 * 2^-14 (binade [2^-7, 2^-6))
    }
    bits = np.array(list(cases), dtype=np.uint16)
    assert oracle.bf16_ulp(bits).tolist() == list(cases.values())
    assert np.all(np.isnan(oracle.bf16_ulp(np.array([0x7F80, 0xFF80, 0x7FC0], np.uint16))))
    # the shape follows the input
    assert oracle.bf16_ulp(np.zeros((2, 3), np.uint16)).shape == (2, 3)


def test_bf16_ulp_is_the_gap_to_the_successor():
    """For every finite bf16 magnitude below the largest, the spacing equals
    value(bits + 1) - value(bits), computed from the successor's bit pattern."""
    b = np.arange(0, 0x7F7F, dtype=np.uint32)            # +0 .. the value below the largest finite
    val = (b << 16).view(np.float32).astype(np.float64)
    nxt = ((b + 1) << 16).view(np.float32).astype(np.float64)
    got = oracle.bf16_ulp(b.astype(np.uint16))
    assert np.array_equal(got, nxt - val)
    neg = (b | 0x8000).astype(np.uint16)
    assert np.array_equal(oracle.bf16_ulp(neg), nxt - val)

"""GPU path vs the CPU oracle, through the C-ABI library (MI355X / gfx950).

Floating-point results are compared element by element within the tolerances
written in tests/helpers.py; integer-valued inputs, the crafted Split-K
partials and the fixed-order combine are compared bit for bit.  Self-
comparisons (repeats, batch sizes, scale placement, multi-adapter vs single)
compare raw bits, never float ==.
"""
import zlib

import numpy as np
import pytest

import deterministic_split_lora_amd as dsl
import oracle
from synth import integer_bf16, normal_bf16, single_adapter_case, sgmv_case, segments_to_ids
from tests.helpers import (bf16_from_gpu, bf16_to_gpu, check_expand, check_shrink, counted_workspace, f32_bits,
                           f32_to_gpu, gpu_available, torch, workspace)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _say(*a):
    print(*a, flush=True)


def run_shrink(x, A, S, scale=1.0, atomic=False):
    t = torch()
    M, K = x.shape
    r = A.shape[0]
    xg, Ag = bf16_to_gpu(x), bf16_to_gpu(A)
    h = t.full((M, r), float("nan"), dtype=t.float32, device="cuda")
    if atomic:
        dsl.lora_shrink_splitk_atomic(xg, Ag, h, split_k=S, scale=scale)
    else:
        ws = workspace(dsl.lora_shrink_workspace_bytes(M, r, S))
        dsl.lora_shrink_splitk(xg, Ag, h, ws if S > 1 else None, split_k=S, scale=scale)
    t.cuda.synchronize()
    return h.cpu().numpy()


# ---------------------------------------------------------------------------
# shrink parity
# ---------------------------------------------------------------------------
SHRINK_CASES = [
    # (M, K, r, S, scale, label)
    (8, 1024, 8, 8, 1.0, "single adapter 8x1024 rank 8, 128-wide chunks"),
    (1, 4096, 16, 8, 1.0, "q_proj M=1"),
    (16, 4096, 16, 8, 1.0, "q_proj M=16"),
    (64, 4096, 16, 8, 1.0, "q_proj M=64"),
    (256, 4096, 16, 8, 2.0, "q_proj M=256 scale 2"),
    (17, 4096, 16, 8, 1.0, "ragged M"),
    (33, 1024, 5, 4, 1.0, "rank 5"),
    (3, 2048, 64, 16, 1.0, "rank 64, S=16"),
    (40, 3072, 24, 8, 0.5, "rank 24, hidden 3072"),
    (5, 4096, 33, 2, 1.0, "rank 33, S=2"),
    (100, 4096, 48, 1, 1.0, "S=1 direct"),
    (1, 8192, 64, 16, 2.0, "decode rank 64 S=16"),
    (300, 14336, 32, 8, 1.0, "down-proj shape, 7 steps per wave"),
    (3, 32, 16, 1, 1.0, "minimal K: one step, one wave"),
    (17, 64, 64, 2, 1.0, "minimal K per split, S=2"),
    (1, 512, 7, 16, 2.0, "minimal K per split, S=16"),
    (33, 96, 5, 1, 1.0, "three steps on one wave (odd step count)"),
    (20, 4096, 128, 8, 1.0, "rank 128: two groups of four rank tiles"),
    (33, 2048, 96, 16, 2.0, "rank 96, S=16"),
    (7, 4096, 65, 1, 1.0, "rank 65, S=1 direct"),
    (2100, 4096, 128, 8, 1.0, "rank 128 at large M: rank groups, one row block per workgroup"),
    (1, 8192, 112, 8, 2.0, "decode rank 112"),
    (5, 65536, 16, 16, 1.0, "long chains: K = 65536, 16 steps per wave"),
    (3, 131072, 32, 8, 1.0, "long chains: K = 131072, 64 steps per wave"),
]


@pytest.mark.parametrize("M,K,r,S,scale,label", SHRINK_CASES)
def test_shrink_parity(M, K, r, S, scale, label):
    _say(f"shrink parity: {label} M={M} K={K} r={r} S={S}")
    c = single_adapter_case(M, K, r, 0, split_k=S, scale=scale, seed=M + K + r)
    h = run_shrink(c.x, c.A, S, scale)
    plan = dsl.lora_shrink_plan(K, r, S)
    a, b = check_shrink(h, c.x, c.A, scale, plan, label)
    _say(f"  max err / stated tol {a:.3g}, / rounding bound {b:.3g}")


@pytest.mark.parametrize("M,K,r,S", [(8, 1024, 8, 8), (19, 4096, 16, 8), (5, 2048, 40, 16), (33, 1024, 64, 1),
                                     (9, 2048, 128, 8), (18, 1024, 77, 4)])
def test_shrink_integer_inputs_bit_exact(M, K, r, S):
    """Integer inputs with every partial sum below 2^24: any summation order is
    exact, so deterministic, atomic and split_k == 1 all equal the oracle
    bit for bit; a wrong index or layout cannot hide."""
    _say(f"integer shrink M={M} K={K} r={r} S={S}")
    x = integer_bf16((M, K), -3, 3, 1, "ix")
    A = integer_bf16((r, K), -3, 3, 1, "iA")
    ref = oracle.shrink(x, A, 2.0)
    assert np.all(np.abs(ref) < 2 ** 23)
    for atomic in (False, True):
        h = run_shrink(x, A, S, 2.0, atomic)
        assert np.array_equal(h.astype(np.float64), ref), f"atomic={atomic}"
    h1 = run_shrink(x, A, 1, 2.0)
    assert np.array_equal(h1.astype(np.float64), ref)


def _crafted_x_A(K, S, r, values, seed):
    """One nonzero product per split: split s gets x[0, s*K/S + off_s] = a_s and
    A[j, same k] = b_s[j], so its fp32 partial is exactly a_s * b_s[j] (a bf16
    x bf16 product is exact in fp32) whatever order the hardware sums in."""
    rng = np.random.default_rng(seed)
    Kc = K // S
    x = np.zeros((1, K), dtype=np.uint16)
    A = np.zeros((r, K), dtype=np.uint16)
    for s in range(S):
        k = s * Kc + int(rng.integers(0, Kc))
        xa, Ab = values(s, rng)
        x[0, k] = xa
        A[:, k] = Ab
    return x, A


def test_fixed_order_combine_crafted_partials():
    """P = (2^100, 1, -2^100, 1, 0, 0, 0, 0): the neighbour pairwise tree gives
    0, the increasing-order fold 1, a stride-paired tree 2 (hand-derived in
    tests/golden/crafted_partials.json).  The GPU must give exactly 0."""
    K, S, r = 1024, 8, 8
    two50 = 0x5880      # bf16 bits of 2^50
    one = 0x3F80
    vals = {0: (two50, two50), 1: (one, one), 2: (two50, 0xD880), 3: (one, one)}

    def v(s, rng):
        return vals.get(s, (0, 0))
    x, A = _crafted_x_A(K, S, r, v, 5)
    P = oracle.split_partials(x, A, S)
    assert P[0, 0, 0] == 2.0 ** 100 and P[2, 0, 0] == -2.0 ** 100
    want = oracle.combine_tree_f32(P.astype(np.float32), 1.0)
    assert np.all(want == 0.0)
    h = run_shrink(x, A, S, 1.0)
    assert np.array_equal(f32_bits_np(h), f32_bits_np(want))
    assert np.all(oracle.combine_sequential_f32(P.astype(np.float32)) == 1.0)


def f32_bits_np(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.int32)


@pytest.mark.parametrize("S", [2, 4, 8, 16])
def test_fixed_order_combine_random_exponents(S):
    """Partials with random signs and exponents spread over 2^-40..2^40: their
    fp32 sum rounds differently for almost every order, so bit equality with
    the oracle's fixed pairwise tree pins the combine order and the single
    scale multiply."""
    K, r = 32 * S * 8, 16

    def v(s, rng):
        ea = int(rng.integers(-20, 21))
        xa = np.float32(rng.uniform(1, 2) * 2.0 ** ea * rng.choice([-1, 1]))
        b = (rng.uniform(1, 2, r) * 2.0 ** rng.integers(-20, 21, r) * rng.choice([-1, 1], r)).astype(np.float32)
        return (oracle.bf16_rne([xa])[0], oracle.bf16_rne(b))
    differs_from_fold = 0
    for seed in range(4):
        x, A = _crafted_x_A(K, S, r, v, 100 * S + seed)
        P = oracle.split_partials(x, A, S).astype(np.float32)   # exact
        for scale in (1.0, 0.75):
            want = oracle.combine_tree_f32(P, scale)
            h = run_shrink(x, A, S, scale)
            assert np.array_equal(f32_bits_np(h), f32_bits_np(want)), (seed, scale)
            seq = oracle.combine_sequential_f32(P, scale)
            differs_from_fold += int(np.sum(f32_bits_np(seq) != f32_bits_np(want)))
    if S >= 4:
        # the inputs do discriminate between summation orders
        assert differs_from_fold > 0


@pytest.mark.parametrize("M,K,r,S", [(8, 1024, 8, 8), (64, 4096, 16, 8), (7, 8192, 64, 16), (5, 4096, 128, 8)])
def test_atomic_parity(M, K, r, S):
    _say(f"atomic shrink parity M={M} K={K} r={r} S={S}")
    c = single_adapter_case(M, K, r, 0, split_k=S, seed=3)
    h = run_shrink(c.x, c.A, S, 2.0, atomic=True)
    check_shrink(h, c.x, c.A, 2.0, dsl.lora_shrink_plan(K, r, S), "atomic", atomic=True)


@pytest.mark.parametrize("M,K,r,S", [(1024, 14336, 32, 8), (2100, 4096, 24, 8), (4100, 8192, 64, 16)])
def test_atomic_parity_large_m_schedules(M, K, r, S):
    """The atomic contrast runs the partial kernel the deterministic path picks
    for these sizes - two row blocks per workgroup sharing A (M = 1024,
    K = 14336), A kept in registers over 4 and 16 row blocks (the others) -
    with fp32 atomic adds in place of the workspace stores: sampled rows within
    the atomic rounding bound of the oracle."""
    _say(f"atomic shrink large M: M={M} K={K} r={r} S={S}")
    c = single_adapter_case(M, K, r, 0, split_k=S, seed=8)
    h = run_shrink(c.x, c.A, S, 2.0, atomic=True)
    rows = np.unique(np.concatenate([np.linspace(0, M - 1, 40).astype(int), [M - 1, M - 2, 15, 16]]))
    check_shrink(h[rows], c.x[rows], c.A, 2.0, dsl.lora_shrink_plan(K, r, S), "atomic large M", atomic=True)


def _sgmv_atomic(c):
    """lora_sgmv_shrink_atomic on a case: h [M, r_max] (host)."""
    t = torch()
    n = len(c.ranks)
    As = [bf16_to_gpu(a) for a in c.As]
    Ap = t.tensor([a.data_ptr() for a in As], dtype=t.int64, device="cuda")
    _, plan = _build_plan(c.ids, n)
    h = t.full((c.M, c.r_max), float("nan"), dtype=t.float32, device="cuda")
    dsl.lora_sgmv_shrink_atomic(bf16_to_gpu(c.x), Ap, c.K, t.from_numpy(c.ranks).cuda(),
                                t.from_numpy(c.scales).cuda(), n, plan, h, c.r_max, c.split_k)
    t.cuda.synchronize()
    return h.cpu().numpy()


@pytest.mark.parametrize("case", ["qkv", "mixed", "many", "prefill"])
def test_sgmv_atomic_parity(case):
    """The multi-adapter atomic contrast (fill, then the multi-adapter partial
    kernel with atomic adds of each split's partial times the adapter's scale):
    per token within the atomic rounding bound of the oracle, zero rows for
    tokens without an adapter, zero columns from the adapter's rank on."""
    rng = np.random.default_rng(31)
    if case == "qkv":
        c = sgmv_case(512, 4096, 8, [64] * 4, 1, 64, 8, seed=0, tag="cfg3")
        rows = list(range(512))
    elif case == "mixed":
        ids = rng.choice([-1, 0, 1, 2, 3, 4, 5, 9], 300).astype(np.int32)
        ids[100:180] = 3
        c = sgmv_case(300, 2048, 8, [8, 16, 32, 64, 24, 5], 0, 0, 4, seed=1, tag="mix", ids=ids)
        rows = list(range(300))
    elif case == "many":
        n = 300
        ranks = [int(v) for v in rng.integers(1, 25, n)]
        ids = rng.permutation(np.concatenate([np.arange(n), rng.integers(250, n, 12), -np.ones(8)])).astype(np.int32)
        c = sgmv_case(len(ids), 1024, 8, ranks, 0, 0, 8, seed=5, tag="many", ids=ids)
        c.scales[:] = rng.choice([0.5, 1.0, 1.5, 2.0, 3.0], n)
        rows = list(range(len(ids)))
    else:
        c = sgmv_case(4096, 8192, 8, [8, 16, 32, 64] * 8, 32, 512, 16, seed=0, tag="b5")
        rows = sorted(set(np.linspace(0, 4095, 48).astype(int).tolist()) | {0, 4095})
    _say(f"sgmv atomic {case}: M={c.M} K={c.K} n={len(c.ranks)} S={c.split_k}")
    h = _sgmv_atomic(c)
    n = len(c.ranks)
    for i in rows:
        a = c.ids[i]
        if a < 0 or a >= n:
            assert np.all(h[i] == 0.0), f"{case}: row {i} without adapter"
            continue
        r = int(c.ranks[a])
        assert np.all(h[i, r:] == 0.0), f"{case}: row {i} past rank {r}"
        check_shrink(h[i:i + 1, :r], c.x[i:i + 1], c.As[a], float(c.scales[a]),
                     dsl.lora_shrink_plan(c.K, r, c.split_k), f"{case} atomic row {i}", atomic=True)


# ---------------------------------------------------------------------------
# expand parity
# ---------------------------------------------------------------------------
EXPAND_CASES = [
    (1, 16, 4096, 2.0), (16, 16, 4096, 2.0), (64, 16, 4096, 2.0), (256, 16, 4096, 2.0),
    (17, 1, 264, 2.0), (9, 8, 520, 1.0), (33, 24, 1000, 2.0), (5, 40, 4096, 0.5), (20, 64, 6144, 2.0),
    (3, 37, 8, 2.0), (37, 128, 1032, 2.0), (6, 65, 264, 1.0), (300, 100, 2048, 2.0), (1, 128, 4096, 2.0),
    (3, 64, 65536, 2.0),
]


@pytest.mark.parametrize("M,r,N,scale", EXPAND_CASES)
def test_expand_parity(M, r, N, scale):
    _say(f"expand parity M={M} r={r} N={N}")
    t = torch()
    rng = np.random.default_rng(M * 7 + r)
    h = (rng.standard_normal((M, r)) * 1.3).astype(np.float32)
    B = normal_bf16((N, r), 0.02, 1, f"eB{r}")
    y = normal_bf16((M, N), 1.0, 1, f"ey{M}")
    # B rows padded to a multiple of 8 columns as the ABI requires
    ldb = (r + 7) // 8 * 8
    Bp = np.zeros((N, ldb), dtype=np.uint16)
    Bp[:, :r] = B
    hp = np.zeros((M, (r + 3) // 4 * 4), dtype=np.float32)
    hp[:, :r] = h
    yg = bf16_to_gpu(y)
    dsl.lora_expand(f32_to_gpu(hp), bf16_to_gpu(Bp), yg, scale, r=r)
    t.cuda.synchronize()
    got = bf16_from_gpu(yg)
    yo, e, ab = oracle.expand(h, B, y, scale)
    frac = check_expand(got, yo, e, ab, y, f"M={M} r={r} N={N}", r=r)
    _say(f"  fraction differing from the correctly rounded value: {frac:.2e}")


def test_expand_B_zero_leaves_y_bitwise():
    t = torch()
    M, r, N = 40, 16, 1024
    y = normal_bf16((M, N), 1.0, 2, "y0")
    yg = bf16_to_gpu(y)
    h = f32_to_gpu(np.random.default_rng(1).standard_normal((M, r)).astype(np.float32))
    dsl.lora_expand(h, t.zeros((N, r), dtype=t.bfloat16, device="cuda"), yg, 2.0)
    t.cuda.synchronize()
    assert np.array_equal(bf16_from_gpu(yg), y)


def test_expand_integer_bit_exact_and_h_rounding():
    t = torch()
    M, r, N = 20, 32, 512
    rng = np.random.default_rng(9)
    h = rng.integers(-4, 5, (M, r)).astype(np.float32)
    B = integer_bf16((N, r), -3, 3, 9, "iB")
    y = integer_bf16((M, N), -50, 50, 9, "iy")
    yg = bf16_to_gpu(y)
    dsl.lora_expand(f32_to_gpu(h), bf16_to_gpu(B), yg, 2.0)
    t.cuda.synchronize()
    yo, _, _ = oracle.expand(h, B, y, 2.0)
    assert np.array_equal(bf16_from_gpu(yg), yo)
    # the paper's midpoint value must be rounded to bf16 before meeting B
    h2 = np.zeros((1, 8), np.float32)
    h2[0, 0] = 0.010345458984375
    B2 = np.zeros((8, 8), np.uint16)
    B2[:, 0] = 0x3F80
    y2 = np.zeros((1, 8), np.uint16)
    yg2 = bf16_to_gpu(y2)
    dsl.lora_expand(f32_to_gpu(h2), bf16_to_gpu(B2), yg2, 3.0)
    t.cuda.synchronize()
    assert np.all(oracle.bf16_to_f64(bf16_from_gpu(yg2)) == 255 * 2.0 ** -13)


def test_scale_placement_bitwise():
    """scale 2 in the shrink or in the expand: multiplying by a power of two
    is exact, so both pipelines give the same bits."""
    t = torch()
    c = single_adapter_case(64, 4096, 16, 4096, seed=4)
    xg, Ag, Bg = bf16_to_gpu(c.x), bf16_to_gpu(c.A), bf16_to_gpu(c.B)
    ws = workspace(dsl.lora_shrink_workspace_bytes(64, 16, 8))
    outs = []
    for s_shrink, s_expand in ((1.0, 2.0), (2.0, 1.0)):
        h = t.empty((64, 16), dtype=t.float32, device="cuda")
        dsl.lora_shrink_splitk(xg, Ag, h, ws, 8, s_shrink)
        yg = bf16_to_gpu(c.y)
        dsl.lora_expand(h, Bg, yg, s_expand)
        t.cuda.synchronize()
        outs.append(bf16_from_gpu(yg))
    assert np.array_equal(outs[0], outs[1])


# ---------------------------------------------------------------------------
# determinism: repeats and batch sizes
# ---------------------------------------------------------------------------
def test_repeat_1000_bitwise():
    t = torch()
    M, K, r, N, S = 64, 4096, 16, 4096, 8
    c = single_adapter_case(M, K, r, N, seed=6)
    xg, Ag, Bg = bf16_to_gpu(c.x), bf16_to_gpu(c.A), bf16_to_gpu(c.B)
    ws = workspace(dsl.lora_shrink_workspace_bytes(M, r, S))
    h = t.empty((M, r), dtype=t.float32, device="cuda")
    y0 = bf16_to_gpu(c.y)
    hs, ys = [], []
    for rep in range(1000):
        dsl.lora_shrink_splitk(xg, Ag, h, ws, S, 1.0)
        yg = y0.clone()
        dsl.lora_expand(h, Bg, yg, 2.0)
        hs.append(h.view(t.int32).clone())
        ys.append(yg.view(t.int16))
    t.cuda.synchronize()
    H = t.stack(hs)
    Y = t.stack(ys)
    assert bool((H == H[0]).all()) and bool((Y == Y[0]).all())
    check_shrink(hs[0].view(t.float32).cpu().numpy(), c.x, c.A, 1.0, dsl.lora_shrink_plan(K, r, S), "repeat")


def test_batch_invariance_sweep():
    """16 probe rows of the MLP down-projection shape (K=14336, r=32, N=4096,
    S=8) placed at random positions among N(0,1) filler rows in batches of
    1, 2, 4, ..., 1024 tokens (20 layouts per size - fresh filler rows and
    fresh probe positions each - the first launched 1000 times): every probe
    row's h (fp32 bits) and y (bf16 bits) must be identical across repeats,
    positions, neighbours and batch sizes."""
    t = torch()
    K, r, N, S, P = 14336, 32, 4096, 8, 16
    probe = normal_bf16((P, K), 1.0, 0, "probe_x")
    A = normal_bf16((r, K), 0.02, 0, "probe_A")
    B = normal_bf16((N, r), 0.02, 0, "probe_B")
    ybase = normal_bf16((P, N), 1.0, 0, "probe_y")
    Ag, Bg = bf16_to_gpu(A), bf16_to_gpu(B)
    ref_h = ref_y = None
    rng = np.random.default_rng(0)
    for b in [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]:
        for layout in range(20):
            # which probe rows go in this batch and where
            groups = [list(range(i, i + b)) for i in range(0, P, b)] if b < P else [list(range(P))]
            for grp in groups:
                M = max(b, len(grp))
                x = normal_bf16((M, K), 1.0, 1000 * b + layout, "filler")
                y = normal_bf16((M, N), 1.0, 1000 * b + layout, "filler_y")
                pos = rng.choice(M, size=len(grp), replace=False)
                x[pos] = probe[grp]
                y[pos] = ybase[grp]
                xg, yg = bf16_to_gpu(x), bf16_to_gpu(y)
                h = t.empty((M, r), dtype=t.float32, device="cuda")
                ws = workspace(dsl.lora_shrink_workspace_bytes(M, r, S))
                yw = yg.clone()
                dsl.lora_shrink_splitk(xg, Ag, h, ws, S, 1.0)
                dsl.lora_expand(h, Bg, yw, 2.0)
                h0, y0 = h.view(t.int32).clone(), yw.view(t.int16).clone()
                # the same through lora_shrink_expand (whose schedule depends on M)
                hf = t.empty_like(h)
                yf = yg.clone()
                dsl.lora_shrink_expand(xg, Ag, Bg, yf, workspace(dsl.lora_shrink_expand_workspace_bytes(M, r, S)),
                                       S, 1.0, 2.0, h=hf)
                assert t.equal(hf.view(t.int32), h0) and t.equal(yf.view(t.int16), y0), f"batch {b}"
                # the first layout of each batch size is launched 1000 times,
                # every repeat compared on the GPU with the first
                bad = t.zeros((), dtype=t.int64, device="cuda")
                for _ in range(999 if layout == 0 else 0):
                    yw = yg.clone()
                    dsl.lora_shrink_splitk(xg, Ag, h, ws, S, 1.0)
                    dsl.lora_expand(h, Bg, yw, 2.0)
                    bad += (h.view(t.int32) != h0).sum() + (yw.view(t.int16) != y0).sum()
                assert int(bad) == 0, f"batch {b}: repeats differ"
                hb = f32_bits(h)[pos]
                yb = bf16_from_gpu(yw)[pos]
                if ref_h is None:
                    ref_h = np.zeros((P, r), np.int32)
                    ref_y = np.zeros((P, N), np.uint16)
                    seen = np.zeros(P, bool)
                for k, gi in enumerate(grp):
                    if not seen[gi]:
                        ref_h[gi], ref_y[gi], seen[gi] = hb[k], yb[k], True
                    else:
                        assert np.array_equal(hb[k], ref_h[gi]), f"h of probe {gi} changed at batch {b}"
                        assert np.array_equal(yb[k], ref_y[gi]), f"y of probe {gi} changed at batch {b}"
        _say(f"  batch {b}: probe rows identical")
    # and the probe rows are right
    check_shrink(ref_h.view(np.float32), probe, A, 1.0, dsl.lora_shrink_plan(K, r, S), "probe")
    yo, e, ab = oracle.expand(ref_h.view(np.float32), B, ybase, 2.0)
    check_expand(ref_y, yo, e, ab, ybase, "probe expand", r=r)


def test_atomic_variant_varies_on_crafted_input(record_property):
    """The atomic variant's result depends on the order its splits land.  With
    P = (2^100, 1, -2^100, 1, 0...) every order gives 0, 1 or 2.  The
    deterministic path gives 0 every time.  Reports (prints and records as a
    test property) the distinct atomic results 2000 launches produced and how
    often each occurred; how many appear depends on scheduling, so no count
    is asserted."""
    t = torch()
    K, S, r = 1024, 8, 8
    two50, one = 0x5880, 0x3F80
    vals = {0: (two50, two50), 1: (one, one), 2: (two50, 0xD880), 3: (one, one)}
    x, A = _crafted_x_A(K, S, r, lambda s, rng: vals.get(s, (0, 0)), 5)
    xg, Ag = bf16_to_gpu(x), bf16_to_gpu(A)
    h = t.empty((1, r), dtype=t.float32, device="cuda")
    ws = workspace(dsl.lora_shrink_workspace_bytes(1, r, S))
    det, atom = [], []
    for _ in range(2000):
        dsl.lora_shrink_splitk(xg, Ag, h, ws, S, 1.0)
        det.append(h.clone())
        dsl.lora_shrink_splitk_atomic(xg, Ag, h, S, 1.0)
        atom.append(h.clone())
    t.cuda.synchronize()
    D = t.stack(det).cpu().numpy()
    Aa = t.stack(atom).cpu().numpy()
    assert np.all(D == 0.0)
    vals, counts = np.unique(Aa.reshape(-1), return_counts=True)
    seen = {float(v): int(n) for v, n in zip(vals, counts)}
    assert set(seen) <= {0.0, 1.0, 2.0}
    record_property("atomic_results_seen", seen)
    _say(f"  atomic results over 2000 launches x {r} columns (value: count): {seen}; deterministic: 0 every time")


# ---------------------------------------------------------------------------
# multi-adapter
# ---------------------------------------------------------------------------
def _plan_reference(ids, n):
    """The plan's tiles (first row, row span, adapter, row mask): runs of equal
    id cut into pieces of 16 in token order, or - up to 4096 tokens, where the
    runs make at least two tiles per 16-token block and the blocks strictly
    fewer - one tile per distinct id of each aligned block, ordered by adapter
    (-1 first) and then block."""
    tiles = []
    M = len(ids)
    i = 0
    norm = [a if 0 <= a < n else -1 for a in ids]
    while i < M:
        j = i
        while j < M and norm[j] == norm[i]:
            j += 1
        for s in range(i, j, 16):
            c = min(16, j - s)
            tiles.append((s, c, norm[i], (1 << c) - 1))
        i = j
    if M <= 4096 and n < 2 ** 22 and len(tiles) >= 2 * ((M + 15) // 16):
        pairs = []
        for b in range((M + 15) // 16):
            r0, c = 16 * b, min(16, M - 16 * b)
            seen = []
            for q in range(c):
                if norm[r0 + q] not in seen:
                    seen.append(norm[r0 + q])
            for a in seen:
                mask = sum(1 << q for q in range(c) if norm[r0 + q] == a)
                pairs.append((a, b, (r0, c, a, mask)))
        if len(pairs) < len(tiles):
            return [e[2] for e in sorted(pairs, key=lambda e: (e[0], e[1]))]
    return tiles


def _build_plan(ids, n):
    t = torch()
    M = len(ids)
    idg = t.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    plan = t.zeros(dsl.lora_sgmv_plan_bytes(M), dtype=t.uint8, device="cuda")
    dsl.lora_sgmv_plan(idg, n, plan)
    return idg, plan


@pytest.mark.parametrize("case", ["segments", "singletons", "invalid", "long", "one_adapter", "large",
                                  "runs_across_passes", "pass_edges", "one_run_8193", "interleaved",
                                  "interleaved_4096", "interleaved_4097", "one_per_token_tie", "ragged_blocks"])
def test_sgmv_plan_tiles(case):
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    if case == "segments":
        ids, n = segments_to_ids(512, [(s, l, a) for s, l, a in _segs(512, 1, 64, 4, rng)]), 4
    elif case == "singletons":
        ids, n = rng.integers(0, 32, 37).astype(np.int32), 32
    elif case == "invalid":
        ids, n = rng.choice([-1, 0, 1, 2, 7, -5], 300).astype(np.int32), 3
    elif case == "long":
        ids, n = segments_to_ids(5000, [(s, l, a) for s, l, a in _segs(5000, 32, 512, 32, rng)]), 32
    elif case == "one_adapter":
        ids, n = np.zeros(1025, np.int32), 1
    elif case == "runs_across_passes":     # runs of 1000-9000 tokens over the 8192-token passes
        ids, n = segments_to_ids(30000, [(s, l, a) for s, l, a in _segs(30000, 1000, 9000, 3, rng)]), 3
    elif case == "pass_edges":             # run changes right at and next to the pass boundaries
        ids = np.zeros(16390, np.int32)
        for cut in (8190, 8191, 8192, 8193, 16383, 16384, 16385):
            ids[cut:] += 1
        ids, n = ids % 3, 3
    elif case == "one_run_8193":
        ids, n = np.full(8193, 2, np.int32), 3
    elif case == "interleaved":            # decode tokens of many requests over 4 adapters: block tiles
        ids, n = (np.arange(512) % 4).astype(np.int32), 4
    elif case == "interleaved_4096":       # the largest batch the block tiling considers
        ids, n = rng.integers(-1, 9, 4096).astype(np.int32), 8
    elif case == "interleaved_4097":       # one token more: runs only
        ids, n = rng.integers(-1, 9, 4097).astype(np.int32), 8
    elif case == "one_per_token_tie":      # as many block pairs as runs: runs
        ids, n = np.arange(40, dtype=np.int32), 40
    elif case == "ragged_blocks":          # a partial last block, ids outside the range
        ids, n = rng.choice([-3, 0, 1, 5, 9], 999).astype(np.int32), 6
    else:
        ids, n = rng.integers(0, 2, 20000).astype(np.int32), 2
    _say(f"plan {case}: M={len(ids)}")
    _, plan = _build_plan(ids, n)
    torch().cuda.synchronize()
    raw = plan.cpu().numpy().view(np.int32)
    ref = _plan_reference(ids.tolist(), n)
    assert raw[0] == len(ref) and raw[1] == len(ids) and raw[2] == n
    got = [tuple(int(v) for v in raw[4 + 4 * k: 8 + 4 * k]) for k in range(raw[0])]
    assert got == ref


def _segs(M, lo, hi, n, rng):
    out, s = [], 0
    while s < M:
        ln = min(int(rng.integers(lo, hi + 1)), M - s)
        out.append((s, ln, int(rng.integers(0, n))))
        s += ln
    return out


def _sgmv_gpu(c, plan_ids=None):
    t = torch()
    n = len(c.ranks)
    K = c.K
    As = [bf16_to_gpu(a) for a in c.As]
    Bs = []
    for b in c.Bs:
        r = b.shape[1]
        rb = (r + 7) // 8 * 8
        bp = np.zeros((c.N, rb), np.uint16)
        bp[:, :r] = b
        Bs.append(bf16_to_gpu(bp))
    Ap = t.tensor([a.data_ptr() for a in As], dtype=t.int64, device="cuda")
    Bp = t.tensor([b.data_ptr() for b in Bs], dtype=t.int64, device="cuda")
    ranks = t.from_numpy(c.ranks).cuda()
    scales = t.from_numpy(c.scales).cuda()
    idg, plan = _build_plan(c.ids, n)
    xg = bf16_to_gpu(c.x)
    h = t.full((c.M, c.r_max), float("nan"), dtype=t.float32, device="cuda")
    ws = workspace(dsl.lora_sgmv_workspace_bytes(c.M, c.r_max, c.split_k))
    dsl.lora_sgmv_shrink(xg, Ap, K, ranks, scales, idg, n, plan, h, c.r_max, c.split_k, ws)
    yg = bf16_to_gpu(c.y)
    dsl.lora_sgmv_expand(h, Bp, ranks, scales, idg, n, yg, c.r_max)
    t.cuda.synchronize()
    return h.cpu().numpy(), bf16_from_gpu(yg), (As, Bs)


def _check_sgmv(c, h, y, rows, label):
    """Per-token comparison with the oracle on the given rows."""
    n = len(c.ranks)
    ids = c.ids[rows]
    for k, i in enumerate(rows):
        a = ids[k]
        if a < 0 or a >= n:
            assert np.all(h[i] == 0.0) and np.array_equal(y[i], c.y[i]), f"{label}: row {i} without adapter"
            continue
        r = int(c.ranks[a])
        assert np.all(h[i, r:] == 0.0)
        check_shrink(h[i:i + 1, :r], c.x[i:i + 1], c.As[a], float(c.scales[a]),
                     dsl.lora_shrink_plan(c.K, r, c.split_k), f"{label} row {i}")
    yo, e, ab = oracle.sgmv_expand(h[rows], c.Bs, c.ranks, c.scales, c.ids[rows], c.y[rows])
    ids_r = c.ids[rows]
    valid = (ids_r >= 0) & (ids_r < len(c.ranks))
    row_rank = np.where(valid, c.ranks[np.where(valid, ids_r, 0)], 0)[:, None]
    return check_expand(y[rows], yo, e, ab, c.y[rows], label, r=row_rank)


def test_sgmv_fused_qkv_parity():
    """4 adapters of rank 64, x [512 x 4096], segments of 1..64 tokens, B [64 x 6144], S=8."""
    c = sgmv_case(512, 4096, 6144, [64, 64, 64, 64], 1, 64, 8, seed=0, tag="cfg3")
    _say(f"sgmv 512x4096 -> 6144, {len(c.segs)} segments")
    h, y, _ = _sgmv_gpu(c)
    frac = _check_sgmv(c, h, y, list(range(512)), "sgmv qkv")
    _say(f"  fraction of y differing from the correctly rounded value: {frac:.2e}")


def test_sgmv_mixed_ranks_and_invalid_ids():
    ranks = [8, 16, 32, 64, 24, 5]
    rng = np.random.default_rng(11)
    M = 300
    ids = rng.choice([-1, 0, 1, 2, 3, 4, 5, 9], M).astype(np.int32)
    ids[100:180] = 3
    c = sgmv_case(M, 2048, 520, ranks, 0, 0, 4, seed=1, tag="mix", ids=ids)
    h, y, _ = _sgmv_gpu(c)
    _check_sgmv(c, h, y, list(range(M)), "sgmv mixed")


def test_sgmv_many_adapters():
    """300 adapters with ranks 1..24, one or a few tokens each, ids spread over
    the whole range (also past the first 256, whose rank and scale the
    multi-adapter kernels may look up in a table) and some tokens without an
    adapter."""
    rng = np.random.default_rng(300)
    n = 300
    ranks = [int(v) for v in rng.integers(1, 25, n)]
    M = 320
    ids = rng.permutation(np.concatenate([np.arange(n), rng.integers(250, n, M - n - 8), -np.ones(8)]))
    ids = ids.astype(np.int32)
    assert (ids >= 256).sum() > 40
    c = sgmv_case(M, 1024, 264, ranks, 0, 0, 8, seed=5, tag="many", ids=ids)
    c.scales[:] = rng.choice([0.5, 1.0, 1.5, 2.0, 3.0], n)      # a scale per adapter
    _say(f"sgmv many adapters: n={n} M={M}")
    h, y, _ = _sgmv_gpu(c)
    _check_sgmv(c, h, y, list(range(M)), "sgmv 300 adapters")


def test_sgmv_ranks_above_64():
    """Ranks 65..128 next to small ones (r_max 128: two groups of four rank
    tiles in the shrink, four matrix-core steps in the expand), -1 and
    out-of-range ids; at a small M and at a large one that walks several
    tiles per expand workgroup."""
    ranks = [128, 65, 8, 100, 16, 96]
    for M, K, N, S in ((300, 2048, 520, 8), (2100, 1024, 4104, 4)):
        rng = np.random.default_rng(M)
        ids = np.empty(M, np.int32)
        pos = 0
        while pos < M:
            run = int(rng.integers(1, 200))
            ids[pos:pos + run] = rng.choice([-1, 0, 1, 2, 3, 4, 5, 11])
            pos += run
        c = sgmv_case(M, K, N, ranks, 0, 0, S, seed=M, tag=f"r128_{M}", ids=ids)
        _say(f"sgmv ranks up to 128: M={M} K={K} N={N} S={S}")
        h, y, _ = _sgmv_gpu(c)
        rows = list(range(M)) if M <= 300 else sorted(rng.choice(M, 60, replace=False).tolist())
        _check_sgmv(c, h, y, rows, f"sgmv r<=128 M={M}")


@pytest.mark.parametrize("M,N,r", [(40, 4096, 64), (130, 1032, 16), (48, 2048, 128)])
def test_sgmv_expand_one_adapter_per_token_bitwise(M, N, r):
    """Decode-style ids - most tokens with an adapter of their own, some
    sharing one, some without: every token's y equals the single-adapter
    lora_expand of its adapter on that row, bit for bit (the blocks' many
    adapters are dealt out to several workgroups); tokens without an adapter
    keep y."""
    t = torch()
    rng = np.random.default_rng(M + r)
    n = M
    ids = np.arange(M, dtype=np.int32)
    ids[rng.choice(M, M // 5, replace=False)] = -1
    ids[rng.choice(M, M // 5, replace=False)] = 3
    ranks = rng.choice([r, max(1, r // 2), 8], n).astype(np.int32)
    ranks[0] = r
    ldh = (r + 3) // 4 * 4
    h = np.zeros((M, ldh), np.float32)
    h[:, :r] = rng.normal(0, 0.5, (M, r)).astype(np.float32)
    y = normal_bf16((M, N), 1.0, M, "otpy")
    Bg, Bs = [], []
    for a in range(n):
        ra = int(ranks[a])
        Bm = normal_bf16((N, ra), 0.02, a, f"otpB{r}")
        Bp = np.zeros((N, (ra + 7) // 8 * 8), np.uint16)
        Bp[:, :ra] = Bm
        Bs.append(Bm)
        Bg.append(bf16_to_gpu(Bp))
    scales = rng.choice([0.5, 1.0, 2.0], n).astype(np.float32)
    Bptr = t.tensor([b.data_ptr() for b in Bg], dtype=t.int64, device="cuda")
    hg = f32_to_gpu(h)
    yg = bf16_to_gpu(y)
    dsl.lora_sgmv_expand(hg, Bptr, t.from_numpy(ranks).cuda(), t.from_numpy(scales).cuda(),
                         t.from_numpy(ids).cuda(), n, yg, r)
    got = bf16_from_gpu(yg)
    none = ids < 0
    assert np.array_equal(got[none], y[none])
    for i in range(M):
        a = int(ids[i])
        if a < 0:
            continue
        ra = int(ranks[a])
        hs = np.zeros((1, (ra + 3) // 4 * 4), np.float32)
        hs[0, :ra] = h[i, :ra]
        ys = bf16_to_gpu(y[i:i + 1])
        dsl.lora_expand(f32_to_gpu(hs), Bg[a], ys, float(scales[a]), r=ra)
        assert np.array_equal(bf16_from_gpu(ys), got[i:i + 1]), f"token {i} adapter {a}"
    pick = [i for i in range(M) if ids[i] == 3][:4]
    if pick:
        ra = int(ranks[3])
        yo, e, ab = oracle.expand(h[pick, :ra], Bs[3], y[pick], float(scales[3]))
        check_expand(got[pick], yo, e, ab, y[pick], "one adapter per token", r=ra)


def test_sgmv_equals_single_adapter_bitwise():
    """All tokens on one adapter: the multi-adapter path must reproduce the
    single-adapter calls bit for bit (same per-token arithmetic)."""
    t = torch()
    for r in (16, 64, 128):
        M, K, N, S = 77, 4096, 1024, 8
        c = sgmv_case(M, K, N, [r], 0, 0, S, seed=2, tag=f"one{r}", ids=np.zeros(M, np.int32))
        h, y, (As, Bs) = _sgmv_gpu(c)
        xg = bf16_to_gpu(c.x)
        hs = t.empty((M, r), dtype=t.float32, device="cuda")
        dsl.lora_shrink_splitk(xg, As[0], hs, workspace(dsl.lora_shrink_workspace_bytes(M, r, S)), S, 2.0)
        ys = bf16_to_gpu(c.y)
        dsl.lora_expand(hs, Bs[0], ys, 2.0, r=r)
        t.cuda.synchronize()
        assert np.array_equal(f32_bits(hs), f32_bits_np(h[:, :r]))
        assert np.array_equal(bf16_from_gpu(ys), y)


@pytest.mark.parametrize("case", ["cycling", "random_invalid", "stream", "counted_multi"])
def test_sgmv_block_tiles_bitwise(case):
    """Interleaved ids, for which the plan makes one masked tile per adapter
    and 16-token block: every token's h and y bits equal those of the
    single-adapter shrink and expand run on that adapter's tokens alone (the
    tiling changes no bit), tokens without an adapter get zero h and keep y,
    the pipeline and the single-launch shrink agree bit for bit, and the
    atomic contrast stays within its rounding bound."""
    t = torch()
    rng = np.random.default_rng(zlib.crc32(case.encode()))
    if case == "cycling":                  # decode-like: every block holds all four adapters
        c = sgmv_case(512, 4096, 1024, [16, 64, 32, 8], 0, 0, 8, seed=41, tag="bt_c",
                      ids=(np.arange(512) % 4).astype(np.int32))
    elif case == "random_invalid":         # partial last block, ids outside the range, rank 128
        c = sgmv_case(300, 2048, 520, [5, 16, 37, 64, 128], 0, 0, 16, seed=42, tag="bt_r",
                      ids=rng.choice([-2, 0, 1, 2, 3, 4, 7], 300).astype(np.int32))
    elif case == "stream":                 # many tiles: the A-in-registers partial kernel
        c = sgmv_case(4096, 1024, 264, [8, 16, 32, 64] * 2, 0, 0, 4, seed=43, tag="bt_s",
                      ids=rng.integers(-1, 8, 4096).astype(np.int32))
    else:                                  # large items of the single-launch multi-adapter shrink
        c = sgmv_case(2048, 4096, 264, [16, 64, 32, 8], 0, 0, 8, seed=44, tag="bt_m",
                      ids=rng.integers(0, 4, 2048).astype(np.int32))
    n = len(c.ranks)
    _say(f"sgmv block tiles {case}: M={c.M} K={c.K} n={n} S={c.split_k}")
    ref = _plan_reference(c.ids.tolist(), n)
    assert any(tl[3] != (1 << tl[1]) - 1 for tl in ref), "the case must take the block tiling"
    _, plan = _build_plan(c.ids, n)
    raw = plan.cpu().numpy().view(np.int32)
    assert [tuple(int(v) for v in raw[4 + 4 * k: 8 + 4 * k]) for k in range(raw[0])] == ref
    h, y, gpu = _sgmv_gpu(c)
    _sgmv_other_schedules(c, h, y, gpu)
    As, Bs = gpu
    for a in range(n):
        rows = np.nonzero(c.ids == a)[0]
        if len(rows) == 0:
            continue
        r, S = int(c.ranks[a]), c.split_k
        xs = bf16_to_gpu(c.x[rows])
        # rows padded to a multiple of 4 floats: the expand reads h with 16-byte loads
        hs = t.empty((len(rows), (r + 3) // 4 * 4), dtype=t.float32, device="cuda")[:, :r]
        dsl.lora_shrink_splitk(xs, As[a], hs, workspace(dsl.lora_shrink_workspace_bytes(len(rows), r, S)), S,
                               float(c.scales[a]))
        ys = bf16_to_gpu(c.y[rows])
        dsl.lora_expand(hs, Bs[a], ys, float(c.scales[a]), r=r)
        t.cuda.synchronize()
        assert np.array_equal(f32_bits(hs), f32_bits_np(h[rows, :r])), f"{case}: h of adapter {a}"
        assert np.array_equal(bf16_from_gpu(ys), y[rows]), f"{case}: y of adapter {a}"
    none = np.nonzero((c.ids < 0) | (c.ids >= n))[0]
    assert np.all(h[none] == 0.0) and np.array_equal(y[none], c.y[none])
    ha = _sgmv_atomic(c)
    for i in sorted(rng.choice(c.M, 24, replace=False).tolist()):
        a = int(c.ids[i])
        if a < 0 or a >= n:
            assert np.all(ha[i] == 0.0)
            continue
        r = int(c.ranks[a])
        check_shrink(ha[i:i + 1, :r], c.x[i:i + 1], c.As[a], float(c.scales[a]),
                     dsl.lora_shrink_plan(c.K, r, c.split_k), f"{case} atomic row {i}", atomic=True)
    _check_sgmv(c, h, y, sorted(rng.choice(c.M, 12, replace=False).tolist()), f"block tiles {case}")


def test_sgmv_permuting_segments_keeps_token_bits():
    ranks = [16, 32, 64]
    M = 200
    c = sgmv_case(M, 4096, 512, ranks, 1, 40, 8, seed=5, tag="perm")
    h1, y1, _ = _sgmv_gpu(c)
    # reverse the order of the segments (tokens move with their ids, x and y)
    order = np.concatenate([np.arange(s, s + l) for s, l, _ in reversed(c.segs)])
    c2 = sgmv_case(M, 4096, 512, ranks, 1, 40, 8, seed=5, tag="perm")
    c2.x, c2.y, c2.ids = c.x[order], c.y[order], c.ids[order]
    h2, y2, _ = _sgmv_gpu(c2)
    assert np.array_equal(f32_bits_np(h2), f32_bits_np(h1[order]))
    assert np.array_equal(y2, y1[order])


def _sgmv_other_schedules(c, h, y, gpu):
    """lora_sgmv_shrink_expand (the scales as shrink and expand scales) and
    lora_sgmv_shrink_counted give the h and y bits of the separate shrink and
    expand that _sgmv_gpu ran."""
    t = torch()
    As, Bs = gpu
    n = len(c.ranks)
    Ap = t.tensor([a.data_ptr() for a in As], dtype=t.int64, device="cuda")
    Bp = t.tensor([b.data_ptr() for b in Bs], dtype=t.int64, device="cuda")
    ranks = t.from_numpy(c.ranks).cuda()
    scales = t.from_numpy(c.scales).cuda()
    idg, plan = _build_plan(c.ids, n)
    xg = bf16_to_gpu(c.x)
    ws = workspace(dsl.lora_sgmv_workspace_bytes(c.M, c.r_max, c.split_k))
    h2 = t.full((c.M, c.r_max), float("nan"), dtype=t.float32, device="cuda")
    y2 = bf16_to_gpu(c.y)
    dsl.lora_sgmv_shrink_expand(xg, Ap, c.K, Bp, ranks, scales, scales, idg, n, plan, y2, c.r_max, c.split_k, ws,
                                h=h2)
    cnt = t.zeros(dsl.lora_sgmv_counter_bytes(c.M) // 4, dtype=t.int32, device="cuda")
    h3 = t.full((c.M, c.r_max), float("nan"), dtype=t.float32, device="cuda")
    dsl.lora_sgmv_shrink_counted(xg, Ap, c.K, ranks, scales, n, plan, h3, c.r_max, c.split_k,
                                 counted_workspace(c.M, c.r_max, c.split_k), cnt)
    t.cuda.synchronize()
    assert np.array_equal(f32_bits_np(h), f32_bits(h2)), "pipeline h"
    assert np.array_equal(f32_bits_np(h), f32_bits(h3)), "single-launch shrink h"
    assert np.array_equal(y, bf16_from_gpu(y2)), "pipeline y"


def test_sgmv_prefill_full_size_sampled():
    """32 adapters with ranks cycling 8, 16, 32, 64, x [4096 x 8192], segments
    of 32..512 tokens, B_i [r_i x 28672], S=16, at full size; the oracle checks
    64 sampled tokens (and untouched rows are checked by value).  The shrink +
    expand pipeline and the single-launch shrink, also timed at this size,
    give the same bits."""
    c = sgmv_case(4096, 8192, 28672, [8, 16, 32, 64] * 8, 32, 512, 16, seed=0, tag="cfg5")
    _say(f"sgmv prefill 4096x8192 -> 28672, {len(c.segs)} segments")
    h, y, gpu = _sgmv_gpu(c)
    rows = sorted(np.random.default_rng(3).choice(4096, 64, replace=False).tolist())
    _check_sgmv(c, h, y, rows, "sgmv prefill")
    _sgmv_other_schedules(c, h, y, gpu)


@pytest.mark.parametrize("M", [32, 128])
def test_sgmv_decode_probe_shapes(M):
    """The decode probes' shapes: M tokens, each with its own rank-64 adapter,
    hidden 8192, Split-K 8, N = 4096.  Sampled rows agree with the oracle; the
    pipeline and the single-launch shrink give the bits of the separate shrink
    and expand."""
    c = sgmv_case(M, 8192, 4096, [64] * M, 0, 0, 8, seed=7, tag=f"dp{M}", ids=np.arange(M, dtype=np.int32))
    _say(f"sgmv decode probe shape: {M} tokens")
    h, y, gpu = _sgmv_gpu(c)
    rows = sorted(np.random.default_rng(M).choice(M, 16, replace=False).tolist())
    _check_sgmv(c, h, y, rows, f"decode probe {M}")
    _sgmv_other_schedules(c, h, y, gpu)


# ---------------------------------------------------------------------------
# fused shrink + expand (two launches) and HIP graph capture
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,r,N,S", [(1, 4096, 16, 4096, 8), (16, 4096, 16, 4096, 8), (64, 4096, 16, 4096, 8),
                                       (256, 4096, 16, 4096, 8), (1, 32, 16, 256, 1), (20, 1024, 64, 8, 16),
                                       (37, 8192, 64, 1032, 16), (5, 1024, 8, 512, 1), (70, 2048, 40, 264, 4),
                                       (3, 3072, 1, 8, 2), (64, 14336, 32, 4096, 8), (65, 4096, 24, 1000, 8),
                                       (9, 1024, 33, 520, 4), (2, 16384, 64, 512, 16),
                                       (300, 2048, 64, 8200, 16), (40, 1024, 24, 16384, 8),
                                       (1, 4096, 128, 4096, 8), (20, 1024, 96, 1032, 16),
                                       (300, 2048, 128, 8200, 16), (33, 2048, 72, 264, 1),
                                       (2100, 1024, 64, 1032, 8), (17, 2048, 32, 1544, 8),
                                       (1, 2048, 20, 3000, 8), (33, 2048, 16, 1024, 8), (1, 4096, 5, 1032, 8),
                                       (250, 4096, 16, 2056, 8)])
def test_shrink_expand_fused_bitwise(M, K, r, N, S):
    """Every schedule of the deterministic shrink + expand - lora_shrink_splitk
    then lora_expand (three launches), lora_shrink_partials then
    lora_expand_combine (two), lora_shrink_expand_fused (one),
    lora_shrink_expand_counted (one, with arrival counters) and
    lora_shrink_expand (which picks by M) - gives the same h and y bits, and
    y agrees with the oracle."""
    _say(f"fused shrink+expand M={M} K={K} r={r} N={N} S={S}")
    t = torch()
    c = single_adapter_case(M, K, r, N, split_k=S, seed=M + r)
    ldb = (r + 7) // 8 * 8
    Bp = np.zeros((N, ldb), np.uint16)
    Bp[:, :r] = c.B
    xg, Ag, Bg = bf16_to_gpu(c.x), bf16_to_gpu(c.A), bf16_to_gpu(Bp)
    # two calls
    h1 = t.empty((M, r), dtype=t.float32, device="cuda")
    ws1 = workspace(dsl.lora_shrink_workspace_bytes(M, r, S))
    dsl.lora_shrink_splitk(xg, Ag, h1, ws1 if S > 1 else None, S, 1.0)
    hpad = t.zeros((M, (r + 3) // 4 * 4), dtype=t.float32, device="cuda")
    hpad[:, :r] = h1
    y1 = bf16_to_gpu(c.y)
    dsl.lora_expand(hpad, Bg, y1, 2.0, r=r)
    # fused, with and without h
    ws2 = workspace(dsl.lora_shrink_expand_workspace_bytes(M, r, S))
    h2 = t.full((M, r), float("nan"), dtype=t.float32, device="cuda")
    y2 = bf16_to_gpu(c.y)
    dsl.lora_shrink_expand(xg, Ag, Bg, y2, ws2, S, 1.0, 2.0, h=h2)
    y3 = bf16_to_gpu(c.y)
    dsl.lora_shrink_expand(xg, Ag, Bg, y3, ws2, S, 1.0, 2.0)
    # the two schedules explicitly: two launches, and the single launch
    h4 = t.full((M, r), float("nan"), dtype=t.float32, device="cuda")
    y4 = bf16_to_gpu(c.y)
    dsl.lora_shrink_partials(xg, Ag, ws2, S)
    dsl.lora_expand_combine(ws2, Bg, y4, S, 1.0, 2.0, h=h4, r=r)
    h5 = t.full((M, r), float("nan"), dtype=t.float32, device="cuda")
    y5 = bf16_to_gpu(c.y)
    y6 = bf16_to_gpu(c.y)
    if r <= 64:
        dsl.lora_shrink_expand_fused(xg, Ag, Bg, y5, S, 1.0, 2.0, h=h5)
        dsl.lora_shrink_expand_fused(xg, Ag, Bg, y6, S, 1.0, 2.0)
    else:                                          # the recompute kernel stops at rank 64
        with pytest.raises(RuntimeError):
            dsl.lora_shrink_expand_fused(xg, Ag, Bg, y5, S, 1.0, 2.0, h=h5)
        h5, y5, y6 = h2, y2, y3
    # one launch with arrival counters, twice on the same counters
    cnt = t.zeros(dsl.lora_shrink_expand_counter_bytes(M) // 4, dtype=t.int32, device="cuda")
    h7 = t.full((M, r), float("nan"), dtype=t.float32, device="cuda")
    y7 = bf16_to_gpu(c.y)
    dsl.lora_shrink_expand_counted(xg, Ag, Bg, y7, ws2, cnt, S, 1.0, 2.0, h=h7)
    y8 = bf16_to_gpu(c.y)
    dsl.lora_shrink_expand_counted(xg, Ag, Bg, y8, ws2, cnt, S, 1.0, 2.0)
    t.cuda.synchronize()
    assert int(cnt.abs().sum()) == 0
    for hh_ in (h2, h4, h5, h7):
        assert np.array_equal(f32_bits(h1), f32_bits(hh_))
    for yy in (y2, y3, y4, y5, y6, y7, y8):
        assert np.array_equal(bf16_from_gpu(y1), bf16_from_gpu(yy))
    hh = h2.cpu().numpy()
    check_shrink(hh, c.x, c.A, 1.0, dsl.lora_shrink_plan(K, r, S), "fused h")
    yo, e, ab = oracle.expand(hh, c.B, c.y, 2.0)
    check_expand(bf16_from_gpu(y2), yo, e, ab, c.y, "fused y", r=r)


def test_graph_capture_replays_match_eager():
    """The deterministic pipeline captured in a HIP graph: several replays, with
    eager work and synchronisations in between, each equal to the eager bits."""
    t = torch()
    M, K, r, N, S = 64, 4096, 16, 4096, 8
    c = single_adapter_case(M, K, r, N, seed=12)
    xg, Ag, Bg = bf16_to_gpu(c.x), bf16_to_gpu(c.A), bf16_to_gpu(c.B)
    y0 = bf16_to_gpu(c.y)
    ws = workspace(dsl.lora_shrink_expand_workspace_bytes(M, r, S))
    wsa = workspace(dsl.lora_shrink_workspace_bytes(M, r, S))
    h = t.empty((M, r), dtype=t.float32, device="cuda")
    ha = t.empty((M, r), dtype=t.float32, device="cuda")
    y = y0.clone()
    ya = y0.clone()

    def step():
        y.copy_(y0)
        dsl.lora_shrink_expand(xg, Ag, Bg, y, ws, S, 1.0, 2.0, h=h)
        dsl.lora_shrink_splitk(xg, Ag, ha, wsa, S, 1.0)
        ya.copy_(y0)
        dsl.lora_expand(ha, Bg, ya, 2.0)
    step()
    t.cuda.synchronize()
    ref = (f32_bits(h), bf16_from_gpu(y), f32_bits(ha), bf16_from_gpu(ya))
    assert np.array_equal(ref[1], ref[3])
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        step()
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    for rep in range(5):
        h.fill_(float("nan")); y.zero_(); ha.fill_(float("nan")); ya.zero_()
        junk = t.randn(1 << 20, device="cuda") * 3.0        # eager work between replays
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        got = (f32_bits(h), bf16_from_gpu(y), f32_bits(ha), bf16_from_gpu(ya))
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), f"replay {rep}"
        del junk


@pytest.mark.parametrize("M,interleaved", [(300, False), (2100, False), (700, True)])
def test_sgmv_graph_replays(M, interleaved):
    """The multi-adapter path captured in a HIP graph - the device-side plan,
    the shrink + expand pipeline and the single-launch shrink (whose kernel
    puts its counters back to zero) - replayed several times with eager work
    and synchronisations in between: every replay gives the eager bits.  At
    M = 2100 the shrink walks several plan tiles per workgroup with A held in
    registers; with interleaved ids the plan takes the block tiling (its sort
    included in the graph)."""
    t = torch()
    rng = np.random.default_rng(M)
    ids = np.empty(M, np.int32)
    pos = 0
    while pos < M:
        run = 1 if interleaved else int(rng.integers(1, 200))
        ids[pos:pos + run] = rng.choice([-1, 0, 1, 2, 3])
        pos += run
    if interleaved:
        assert any(tl[3] != (1 << tl[1]) - 1 for tl in _plan_reference(ids.tolist(), 4))
    c = sgmv_case(M, 1024, 1032, [16, 64, 8, 32], 0, 0, 8, seed=M, tag=f"gr{M}", ids=ids)
    n = len(c.ranks)
    As = [bf16_to_gpu(a) for a in c.As]
    Bs = []
    for b in c.Bs:
        bp = np.zeros((c.N, (b.shape[1] + 7) // 8 * 8), np.uint16)
        bp[:, :b.shape[1]] = b
        Bs.append(bf16_to_gpu(bp))
    Ap = t.tensor([a.data_ptr() for a in As], dtype=t.int64, device="cuda")
    Bp = t.tensor([b.data_ptr() for b in Bs], dtype=t.int64, device="cuda")
    ranks = t.from_numpy(c.ranks).cuda()
    scales = t.from_numpy(np.array([0.5, 2.0, 1.0, 3.0], np.float32)).cuda()
    idg = t.from_numpy(c.ids).cuda()
    plan = t.zeros(dsl.lora_sgmv_plan_bytes(M), dtype=t.uint8, device="cuda")
    xg, y0 = bf16_to_gpu(c.x), bf16_to_gpu(c.y)
    y = y0.clone()
    ws = workspace(dsl.lora_sgmv_workspace_bytes(M, c.r_max, c.split_k))
    ws2 = counted_workspace(M, c.r_max, c.split_k)
    cnt = t.zeros(dsl.lora_sgmv_counter_bytes(M) // 4, dtype=t.int32, device="cuda")
    h = t.empty((M, c.r_max), dtype=t.float32, device="cuda")
    h2 = t.empty((M, c.r_max), dtype=t.float32, device="cuda")

    def step():
        dsl.lora_sgmv_plan(idg, n, plan)
        y.copy_(y0)
        dsl.lora_sgmv_shrink_expand(xg, Ap, c.K, Bp, ranks, scales, scales, idg, n, plan, y, c.r_max, c.split_k,
                                    ws, h=h)
        dsl.lora_sgmv_shrink_counted(xg, Ap, c.K, ranks, scales, n, plan, h2, c.r_max, c.split_k, ws2, cnt)
    step()
    t.cuda.synchronize()
    ref = (f32_bits(h), bf16_from_gpu(y), f32_bits(h2))
    assert np.array_equal(ref[0], ref[2])
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        step()
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    for rep in range(5):
        h.fill_(float("nan")); h2.fill_(float("nan")); y.zero_(); plan.zero_()
        junk = t.randn(1 << 20, device="cuda") * 3.0        # eager work between replays
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        got = (f32_bits(h), bf16_from_gpu(y), f32_bits(h2))
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), f"replay {rep}"
        assert int(cnt.abs().sum()) == 0, f"counters left non-zero after replay {rep}"
        del junk


@pytest.mark.parametrize("S", [1, 2, 4, 8, 16])
def test_expand_combine_on_given_workspace(S):
    """lora_expand_combine on a workspace filled with seeded fp32 values of
    widely spread exponents: h must equal the oracle's fixed pairwise tree
    (then x shrink_scale) bit for bit, and y the oracle's expand of that h."""
    t = torch()
    M, r, N = 45, 24, 520
    rng = np.random.default_rng(77 + S)
    P = (rng.uniform(-1, 1, (S, M, r)) * 2.0 ** rng.integers(-30, 30, (S, M, r))).astype(np.float32)
    B = normal_bf16((N, r), 0.02, S, "cwB")
    y = normal_bf16((M, N), 1.0, S, "cwy")
    h = t.full((M, r), float("nan"), dtype=t.float32, device="cuda")
    yg = bf16_to_gpu(y)
    dsl.lora_expand_combine(f32_to_gpu(P.reshape(-1)), bf16_to_gpu(B), yg, S, 0.75, 2.0, h=h)
    t.cuda.synchronize()
    want_h = oracle.combine_tree_f32(P, 0.75)
    assert np.array_equal(f32_bits(h), f32_bits_np(want_h))
    yo, e, ab = oracle.expand(want_h, B, y, 2.0)
    check_expand(bf16_from_gpu(yg), yo, e, ab, y, f"combine S={S}", r=r)


@pytest.mark.parametrize("M,K,r,S", [(1, 4096, 16, 8), (33, 8192, 64, 16), (20, 1024, 8, 8)])
def test_shrink_partials_match_oracle(M, K, r, S):
    """Each split's fp32 partial P_s (read back from the documented workspace
    layout) agrees with the oracle's Eq. 3 partial for that chunk."""
    t = torch()
    c = single_adapter_case(M, K, r, 0, split_k=S, seed=21)
    ws = workspace(dsl.lora_shrink_expand_workspace_bytes(M, r, S))
    dsl.lora_shrink_partials(bf16_to_gpu(c.x), bf16_to_gpu(c.A), ws, S)
    t.cuda.synchronize()
    P = ws[: S * M * r * 4].view(t.float32).cpu().numpy().reshape(S, M, r)
    ref = oracle.split_partials(c.x, c.A, S)
    plan = dsl.lora_shrink_plan(K, r, S)
    # per chunk: one matrix-core step per 32 k, k_steps deep, log2(waves)-level tree
    Kc = K // S
    xs = oracle.bf16_to_f64(c.x)
    As = oracle.bf16_to_f64(c.A)
    for s in range(S):
        absum = np.abs(xs[:, s * Kc:(s + 1) * Kc]) @ np.abs(As[:, s * Kc:(s + 1) * Kc]).T
        depth = 32 + plan["k_steps"] + int(np.log2(plan["waves"])) + 1
        assert np.all(np.abs(P[s] - ref[s]) <= depth * 2.0 ** -24 * absum + 1e-30), f"split {s}"


def test_batch_invariance_across_schedule_switch():
    """A shape whose A is small enough (1024 x 8) for lora_shrink_expand to use
    the single-launch schedule up to 64 tokens and two launches above: 16
    probe rows at random positions in batches of 1 .. 512 give the same bits
    as each other and as lora_shrink_splitk + lora_expand."""
    t = torch()
    K, r, N, S, P = 1024, 8, 1024, 8, 16
    assert dsl.lora_shrink_expand_launches(64, K, r, N, S) == 1
    assert dsl.lora_shrink_expand_launches(65, K, r, N, S) == 2
    probe = normal_bf16((P, K), 1.0, 3, "sw_x")
    A = normal_bf16((r, K), 0.02, 3, "sw_A")
    B = normal_bf16((N, r), 0.02, 3, "sw_B")
    ybase = normal_bf16((P, N), 1.0, 3, "sw_y")
    Ag, Bg = bf16_to_gpu(A), bf16_to_gpu(B)
    xg0, yg0 = bf16_to_gpu(probe), bf16_to_gpu(ybase)
    h0 = t.empty((P, r), dtype=t.float32, device="cuda")
    dsl.lora_shrink_splitk(xg0, Ag, h0, workspace(dsl.lora_shrink_workspace_bytes(P, r, S)), S, 1.0)
    dsl.lora_expand(h0, Bg, yg0, 2.0)
    ref_h, ref_y = f32_bits(h0), bf16_from_gpu(yg0)
    rng = np.random.default_rng(5)
    for b in [1, 2, 4, 8, 16, 32, 64, 65, 128, 512]:
        groups = [list(range(i, min(i + b, P))) for i in range(0, P, b)] if b < P else [list(range(P))]
        for grp in groups:
            M = max(b, len(grp))
            x = normal_bf16((M, K), 1.0, 50 + b, "sw_f")
            y = normal_bf16((M, N), 1.0, 50 + b, "sw_fy")
            pos = rng.choice(M, size=len(grp), replace=False)
            x[pos] = probe[grp]
            y[pos] = ybase[grp]
            h = t.empty((M, r), dtype=t.float32, device="cuda")
            yg = bf16_to_gpu(y)
            ws = workspace(dsl.lora_shrink_expand_workspace_bytes(M, r, S))
            dsl.lora_shrink_expand(bf16_to_gpu(x), Ag, Bg, yg, ws, S, 1.0, 2.0, h=h)
            t.cuda.synchronize()
            assert np.array_equal(f32_bits(h)[pos], ref_h[grp]), f"h at batch {b}"
            assert np.array_equal(bf16_from_gpu(yg)[pos], ref_y[grp]), f"y at batch {b}"


# ---------------------------------------------------------------------------
# single-launch shrink with completion counters (the paper's final design)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,r,S", [(1, 4096, 16, 8), (8, 1024, 8, 8), (64, 4096, 16, 8), (256, 4096, 16, 8),
                                     (37, 8192, 64, 16), (100, 2048, 40, 4), (19, 14336, 32, 8), (5, 1024, 5, 2),
                                     (40, 4096, 16, 1), (1100, 2048, 40, 8), (4100, 1024, 64, 8),
                                     (4100, 2048, 16, 8), (2000, 1024, 24, 16), (37, 4096, 128, 8),
                                     (2100, 1024, 100, 8)])
def test_shrink_counted_bitwise(M, K, r, S):
    """lora_shrink_splitk_counted (one launch, the split that starts last
    combines, one row block per workgroup) gives lora_shrink_splitk's bits
    (which shares A loads between 2 or 4 row blocks per workgroup at the
    larger M here), leaves its counters and its tagged workspace at zero, and
    repeats bit for bit on the same buffers."""
    t = torch()
    c = single_adapter_case(M, K, r, 0, split_k=S, seed=31 + M)
    xg, Ag = bf16_to_gpu(c.x), bf16_to_gpu(c.A)
    ws = workspace(dsl.lora_shrink_workspace_bytes(M, r, S))
    h1 = t.empty((M, r), dtype=t.float32, device="cuda")
    dsl.lora_shrink_splitk(xg, Ag, h1, ws if S > 1 else None, S, 2.0)
    cnt = t.zeros(max(1, dsl.lora_shrink_counter_bytes(M) // 4), dtype=t.int32, device="cuda")
    ws2 = counted_workspace(M, r, S)
    outs = []
    for rep in range(20):
        h2 = t.full((M, r), float("nan"), dtype=t.float32, device="cuda")
        dsl.lora_shrink_splitk_counted(xg, Ag, h2, ws2 if S > 1 else None, cnt if S > 1 else None, S, 2.0)
        outs.append(h2)
    t.cuda.synchronize()
    ref = f32_bits(h1)
    for h2 in outs:
        assert np.array_equal(f32_bits(h2), ref)
    assert int(cnt.abs().sum()) == 0
    # every tagged slot written was consumed and cleared by its combining workgroup
    if S > 1:
        assert int(ws2.count_nonzero()) == 0
    check_shrink(outs[0].cpu().numpy(), c.x, c.A, 2.0, dsl.lora_shrink_plan(K, r, S), "counted")


def test_shrink_counted_in_graph_replays():
    t = torch()
    M, K, r, S = 48, 4096, 16, 8
    c = single_adapter_case(M, K, r, 0, split_k=S, seed=8)
    xg, Ag = bf16_to_gpu(c.x), bf16_to_gpu(c.A)
    ws = counted_workspace(M, r, S)
    cnt = t.zeros(dsl.lora_shrink_counter_bytes(M) // 4, dtype=t.int32, device="cuda")
    h = t.empty((M, r), dtype=t.float32, device="cuda")
    dsl.lora_shrink_splitk_counted(xg, Ag, h, ws, cnt, S, 1.0)
    t.cuda.synchronize()
    ref = f32_bits(h)
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        dsl.lora_shrink_splitk_counted(xg, Ag, h, ws, cnt, S, 1.0)
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        for _ in range(3):
            dsl.lora_shrink_splitk_counted(xg, Ag, h, ws, cnt, S, 1.0)
    for rep in range(5):
        h.fill_(float("nan"))
        junk = t.randn(1 << 18, device="cuda").sum()
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        assert np.array_equal(f32_bits(h), ref), f"replay {rep}"
        assert int(cnt.abs().sum()) == 0
        del junk


@pytest.mark.parametrize("case", ["qkv", "mixed", "decode_probe", "prefill", "rank128"])
def test_sgmv_counted_bitwise(case):
    """lora_sgmv_shrink_counted gives lora_sgmv_shrink's bits (rows without an
    adapter and columns beyond a rank zeroed) in one launch; in the prefill
    case the two-pass shrink shares A loads between 4 plan tiles."""
    t = torch()
    if case == "prefill":
        rng = np.random.default_rng(6)
        ids = np.empty(2048, np.int32)
        pos = 0
        while pos < 2048:
            run = int(rng.integers(5, 300))
            ids[pos:pos + run] = rng.choice([-1, 0, 1, 2, 3, 4, 5, 6, 7])
            pos += run
        c = sgmv_case(2048, 2048, 64, [8, 16, 32, 64, 5, 37, 64, 16], 0, 0, 16, seed=3, tag="cp", ids=ids)
    elif case == "qkv":
        c = sgmv_case(512, 4096, 64, [64, 64, 64, 64], 1, 64, 8, seed=0, tag="cq")
    elif case == "rank128":
        rng = np.random.default_rng(8)
        ids = rng.choice([-1, 0, 1, 2, 3], 150).astype(np.int32)
        ids[20:90] = 0
        c = sgmv_case(150, 2048, 64, [128, 72, 16, 100], 0, 0, 8, seed=4, tag="c128", ids=ids)
    elif case == "mixed":
        rng = np.random.default_rng(4)
        ids = rng.choice([-1, 0, 1, 2, 3, 17], 333).astype(np.int32)
        ids[50:150] = 2
        c = sgmv_case(333, 2048, 64, [8, 16, 32, 64], 0, 0, 16, seed=1, tag="cm", ids=ids)
    else:
        c = sgmv_case(32, 8192, 64, [64] * 32, 0, 0, 8, seed=2, tag="cd", ids=np.arange(32, dtype=np.int32))
    n = len(c.ranks)
    As = [bf16_to_gpu(a) for a in c.As]
    Ap = t.tensor([a.data_ptr() for a in As], dtype=t.int64, device="cuda")
    ranks = t.from_numpy(c.ranks).cuda()
    scales = t.from_numpy(c.scales).cuda()
    idg, plan = _build_plan(c.ids, n)
    xg = bf16_to_gpu(c.x)
    h1 = t.full((c.M, c.r_max), float("nan"), dtype=t.float32, device="cuda")
    ws = workspace(dsl.lora_sgmv_workspace_bytes(c.M, c.r_max, c.split_k))
    dsl.lora_sgmv_shrink(xg, Ap, c.K, ranks, scales, idg, n, plan, h1, c.r_max, c.split_k, ws)
    cnt = t.zeros(dsl.lora_sgmv_counter_bytes(c.M) // 4, dtype=t.int32, device="cuda")
    ws2 = counted_workspace(c.M, c.r_max, c.split_k)
    hs = []
    for rep in range(5):
        h2 = t.full((c.M, c.r_max), float("nan"), dtype=t.float32, device="cuda")
        dsl.lora_sgmv_shrink_counted(xg, Ap, c.K, ranks, scales, n, plan, h2, c.r_max, c.split_k, ws2, cnt)
        hs.append(h2)
    t.cuda.synchronize()
    for h2 in hs:
        assert np.array_equal(f32_bits(h2), f32_bits(h1))
    assert int(cnt.abs().sum()) == 0
    assert int(ws2.count_nonzero()) == 0          # every written slot consumed and cleared
    hh = hs[0].cpu().numpy()
    for i in range(0, c.M, max(1, c.M // 40)):
        a = int(c.ids[i])
        if a < 0 or a >= n:
            assert np.all(hh[i] == 0.0)
            continue
        r = int(c.ranks[a])
        assert np.all(hh[i, r:] == 0.0)
        check_shrink(hh[i:i + 1, :r], c.x[i:i + 1], c.As[a], float(c.scales[a]),
                     dsl.lora_shrink_plan(c.K, r, c.split_k), f"{case} row {i}")


def test_sgmv_plan_of_other_batch_processes_nothing():
    """A plan used with another M or n_adapters than it was built for is
    recognised by its header, and the multi-adapter shrinks then process no
    tile, so none of its entries (which may point past the batch) is
    followed. The single launch leaves h, its tagged workspace and its
    counters as they were. The two-pass shrink's partial kernel leaves its
    workspace untouched."""
    t = torch()
    c = sgmv_case(64, 2048, 64, [16, 32, 16], 0, 0, 8, seed=9, tag="pl",
                  ids=(np.arange(64) % 3).astype(np.int32))
    n = len(c.ranks)
    As = [bf16_to_gpu(a) for a in c.As]
    Ap = t.tensor([a.data_ptr() for a in As], dtype=t.int64, device="cuda")
    ranks = t.from_numpy(c.ranks).cuda()
    scales = t.from_numpy(c.scales).cuda()
    xg = bf16_to_gpu(c.x)
    _, plan = _build_plan(c.ids, n)                     # built for M = 64, n_adapters = 3
    m = 16
    for n_used, what in ((n, "other M"), (n - 1, "other n_adapters and M")):
        h = t.full((m, c.r_max), 7.0, dtype=t.float32, device="cuda")
        cws = counted_workspace(m, c.r_max, c.split_k)
        cnt = t.zeros(dsl.lora_sgmv_counter_bytes(m) // 4, dtype=t.int32, device="cuda")
        dsl.lora_sgmv_shrink_counted(xg[:m], Ap, c.K, ranks, scales, n_used, plan, h, c.r_max, c.split_k, cws, cnt)
        t.cuda.synchronize()
        assert bool((h == 7.0).all()), what
        assert int(cnt.abs().sum()) == 0, what
        assert int(cws.count_nonzero()) == 0, what
    ws = t.full((dsl.lora_sgmv_workspace_bytes(m, c.r_max, c.split_k),), 0x5A, dtype=t.uint8, device="cuda")
    idg = t.from_numpy(np.ascontiguousarray(c.ids[:m])).cuda()
    h = t.zeros((m, c.r_max), dtype=t.float32, device="cuda")
    dsl.lora_sgmv_shrink(xg[:m], Ap, c.K, ranks, scales, idg, n, plan, h, c.r_max, c.split_k, ws)
    t.cuda.synchronize()
    assert bool((ws == 0x5A).all())


def test_counted_shrinks_stress_repeats():
    """Back-to-back launches of the single-launch shrinks (single adapter and
    32 one-token adapters of rank 64), each compared bit for bit on the GPU
    with the two-pass result: a partial read before it was visible would show
    up as a mismatch."""
    t = torch()
    M, K, r, S = 64, 4096, 16, 8
    c = single_adapter_case(M, K, r, 0, split_k=S, seed=90)
    xg, Ag = bf16_to_gpu(c.x), bf16_to_gpu(c.A)
    ref = t.empty((M, r), dtype=t.float32, device="cuda")
    dsl.lora_shrink_splitk(xg, Ag, ref, workspace(dsl.lora_shrink_workspace_bytes(M, r, S)), S, 1.0)
    ws = counted_workspace(M, r, S)
    cnt = t.zeros(dsl.lora_shrink_counter_bytes(M) // 4, dtype=t.int32, device="cuda")
    h = t.empty_like(ref)
    bad = t.zeros((), dtype=t.int64, device="cuda")
    for _ in range(500):
        h.fill_(float("nan"))
        dsl.lora_shrink_splitk_counted(xg, Ag, h, ws, cnt, S, 1.0)
        bad += (h.view(t.int32) != ref.view(t.int32)).sum()
    c2 = sgmv_case(32, 8192, 64, [64] * 32, 0, 0, 8, seed=91, tag="st", ids=np.arange(32, dtype=np.int32))
    As = [bf16_to_gpu(a) for a in c2.As]
    Ap = t.tensor([a.data_ptr() for a in As], dtype=t.int64, device="cuda")
    ranks = t.from_numpy(c2.ranks).cuda()
    idg, plan = _build_plan(c2.ids, 32)
    x2 = bf16_to_gpu(c2.x)
    ref2 = t.empty((32, 64), dtype=t.float32, device="cuda")
    dsl.lora_sgmv_shrink(x2, Ap, 8192, ranks, None, idg, 32, plan, ref2, 64, 8,
                         workspace(dsl.lora_sgmv_workspace_bytes(32, 64, 8)))
    ws2 = counted_workspace(32, 64, 8)
    cnt2 = t.zeros(dsl.lora_sgmv_counter_bytes(32) // 4, dtype=t.int32, device="cuda")
    h2 = t.empty_like(ref2)
    for _ in range(500):
        h2.fill_(float("nan"))
        dsl.lora_sgmv_shrink_counted(x2, Ap, 8192, ranks, None, 32, plan, h2, 64, 8, ws2, cnt2)
        bad += (h2.view(t.int32) != ref2.view(t.int32)).sum()
    t.cuda.synchronize()
    assert int(bad) == 0
    assert int(cnt.abs().sum()) == 0 and int(cnt2.abs().sum()) == 0


def test_sgmv_counted_large_m_repeats():
    """The single-launch multi-adapter shrink at a large-M shape (1024 tokens,
    K = 4096, Split-K 16, short runs of 4 adapters of ranks 64, 16, 37 and 8
    and of tokens without one, so items mix tiles of several adapters): 200
    back-to-back launches, each compared bit for bit on the GPU with the
    two-pass result, and the counters back at zero."""
    t = torch()
    rng = np.random.default_rng(93)
    ids = np.empty(1024, np.int32)
    pos = 0
    while pos < 1024:
        run = int(rng.integers(3, 70))
        ids[pos:pos + run] = rng.choice([-1, 0, 1, 2, 3])
        pos += run
    c = sgmv_case(1024, 4096, 64, [64, 16, 37, 8], 0, 0, 16, seed=94, tag="cs", ids=ids)
    As = [bf16_to_gpu(a) for a in c.As]
    Ap = t.tensor([a.data_ptr() for a in As], dtype=t.int64, device="cuda")
    ranks = t.from_numpy(c.ranks).cuda()
    scales = t.from_numpy(c.scales).cuda()
    idg, plan = _build_plan(c.ids, 4)
    xg = bf16_to_gpu(c.x)
    ref = t.full((c.M, c.r_max), float("nan"), dtype=t.float32, device="cuda")
    dsl.lora_sgmv_shrink(xg, Ap, c.K, ranks, scales, idg, 4, plan, ref, c.r_max, c.split_k,
                         workspace(dsl.lora_sgmv_workspace_bytes(c.M, c.r_max, c.split_k)))
    ws = counted_workspace(c.M, c.r_max, c.split_k)
    cnt = t.zeros(dsl.lora_sgmv_counter_bytes(c.M) // 4, dtype=t.int32, device="cuda")
    h = t.empty_like(ref)
    bad = t.zeros((), dtype=t.int64, device="cuda")
    for _ in range(200):
        h.fill_(float("nan"))
        dsl.lora_sgmv_shrink_counted(xg, Ap, c.K, ranks, scales, 4, plan, h, c.r_max, c.split_k, ws, cnt)
        bad += (h.view(t.int32) != ref.view(t.int32)).sum()
    t.cuda.synchronize()
    assert int(bad) == 0
    assert int(cnt.abs().sum()) == 0
    hh = h.cpu().numpy()
    for i in range(0, c.M, 37):
        a = int(c.ids[i])
        if a < 0:
            assert np.all(hh[i] == 0.0)
            continue
        r = int(c.ranks[a])
        assert np.all(hh[i, r:] == 0.0)
        check_shrink(hh[i:i + 1, :r], c.x[i:i + 1], c.As[a], float(c.scales[a]),
                     dsl.lora_shrink_plan(c.K, r, c.split_k), f"large-M counted row {i}")


# ---------------------------------------------------------------------------
# single-launch shrink + expand with arrival counters
# ---------------------------------------------------------------------------
def test_shrink_expand_counted_stress_and_graph():
    """Back-to-back launches of lora_shrink_expand_counted at several M on one
    counter buffer (sized for the largest M), each compared bit for bit on the
    GPU with the two-launch result; then the same calls captured in a HIP
    graph and replayed with eager work in between.  A partial read before it
    was visible, or a counter left non-zero, would show up as a mismatch."""
    t = torch()
    K, r, N, S = 4096, 16, 4096, 8
    Ms = (1, 16, 64, 256, 33)
    cnt = t.zeros(dsl.lora_shrink_expand_counter_bytes(max(Ms)) // 4, dtype=t.int32, device="cuda")
    bad = t.zeros((), dtype=t.int64, device="cuda")
    cases = []
    for M in Ms:
        _say(f"counted shrink+expand stress M={M}")
        c = single_adapter_case(M, K, r, N, split_k=S, seed=300 + M)
        xg, Ag, Bg, y0 = bf16_to_gpu(c.x), bf16_to_gpu(c.A), bf16_to_gpu(c.B), bf16_to_gpu(c.y)
        ws = workspace(dsl.lora_shrink_expand_workspace_bytes(M, r, S))
        href = t.empty((M, r), dtype=t.float32, device="cuda")
        yref = y0.clone()
        dsl.lora_shrink_partials(xg, Ag, ws, S)
        dsl.lora_expand_combine(ws, Bg, yref, S, 1.0, 2.0, h=href, r=r)
        h = t.empty_like(href)
        y = t.empty_like(y0)
        cases.append((M, xg, Ag, Bg, y0, ws, href, yref, h, y))
        for _ in range(200):
            y.copy_(y0)
            h.fill_(float("nan"))
            dsl.lora_shrink_expand_counted(xg, Ag, Bg, y, ws, cnt, S, 1.0, 2.0, h=h)
            bad += (h.view(t.int32) != href.view(t.int32)).sum() + (y.view(t.int16) != yref.view(t.int16)).sum()
    t.cuda.synchronize()
    assert int(bad) == 0
    assert int(cnt.abs().sum()) == 0

    def step():
        for (M, xg, Ag, Bg, y0, ws, href, yref, h, y) in cases:
            y.copy_(y0)
            dsl.lora_shrink_expand_counted(xg, Ag, Bg, y, ws, cnt, S, 1.0, 2.0, h=h)
    side = t.cuda.Stream()
    side.wait_stream(t.cuda.current_stream())
    with t.cuda.stream(side):
        step()
    t.cuda.current_stream().wait_stream(side)
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        step()
    for rep in range(5):
        for case in cases:
            case[8].fill_(float("nan"))
            case[9].zero_()
        junk = t.randn(1 << 18, device="cuda") * 2.0
        t.cuda.synchronize()
        g.replay()
        t.cuda.synchronize()
        for (M, xg, Ag, Bg, y0, ws, href, yref, h, y) in cases:
            assert np.array_equal(f32_bits(h), f32_bits(href)), f"replay {rep} M={M} h"
            assert np.array_equal(bf16_from_gpu(y), bf16_from_gpu(yref)), f"replay {rep} M={M} y"
        assert int(cnt.abs().sum()) == 0
        del junk


# ---------------------------------------------------------------------------
# shrinks whose partial kernel keeps A in registers and walks row blocks
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("M,K,r,S", [(4100, 8192, 64, 16), (4100, 4096, 24, 8), (2100, 16384, 32, 16),
                                     (4100, 1024, 5, 8), (2100, 2048, 37, 16)])
def test_shrink_stream_rows_bitwise(M, K, r, S):
    """At M large enough (at least 1024 row block x split pairs, short wave
    chains) for the partial kernel that keeps each wave's A operands in
    registers while it walks several row blocks, every row's h equals that of
    a small call on the same rows (one-tile kernels) bit for bit, and sampled
    rows agree with the oracle.  Plans with 1, 2 and 4 steps per wave, 4 and 8
    waves, 1 to 4 rank tiles; ragged M and ranks."""
    _say(f"stream shrink M={M} K={K} r={r} S={S}")
    x = normal_bf16((M, K), 1.0, r, "ssx")
    A = normal_bf16((r, K), 0.02, r, "ssA")
    h = run_shrink(x, A, S, 2.0)
    for r0 in (0, 1008, M - 37):
        n = min(64, M - r0)
        hs = run_shrink(np.ascontiguousarray(x[r0:r0 + n]), A, S, 2.0)
        assert np.array_equal(hs.view(np.int32), h[r0:r0 + n].view(np.int32)), f"rows {r0}.."
    rng = np.random.default_rng(r)
    rows = sorted(set([0, 15, 16, M - 1] + rng.choice(M, 16, replace=False).tolist()))
    check_shrink(h[rows], x[rows], A, 2.0, dsl.lora_shrink_plan(K, r, S), f"stream shrink M={M} K={K} r={r}")


# ---------------------------------------------------------------------------
# expands that walk several 16-token tiles per workgroup (large M x N)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("r", [5, 16, 37, 64, 100, 128])
def test_expand_large_m_tiles_bitwise(r):
    """At M x N large enough that lora_expand walks several tiles per
    workgroup (B kept in registers, h staged in LDS), every row equals the
    one-tile-per-workgroup result of a small call on the same rows bit for
    bit, and sampled rows agree with the oracle.  Ragged M and N."""
    t = torch()
    M, N = 4100, 4104
    _say(f"large-M expand r={r} M={M} N={N}")
    ldh = (r + 3) // 4 * 4
    ldb = (r + 7) // 8 * 8
    rng = np.random.default_rng(40 + r)
    h = np.zeros((M, ldh), np.float32)
    h[:, :r] = rng.normal(0, 0.5, (M, r)).astype(np.float32)
    h[:, r:] = np.nan                         # padding must never be read
    Bm = normal_bf16((N, r), 0.02, r, "lmB")
    Bp = np.zeros((N, ldb), np.uint16)
    Bp[:, :r] = Bm
    y = normal_bf16((M, N), 1.0, r, "lmy")
    hg, Bg = f32_to_gpu(h), bf16_to_gpu(Bp)
    yg = bf16_to_gpu(y)
    dsl.lora_expand(hg, Bg, yg, 2.0, r=r)
    got = bf16_from_gpu(yg)
    for r0 in (0, 1008, 4096 - 16, 4100 - 37):
        n = min(64, M - r0)
        ys = bf16_to_gpu(y[r0:r0 + n])
        dsl.lora_expand(hg[r0:r0 + n], Bg, ys, 2.0, r=r)
        assert np.array_equal(bf16_from_gpu(ys), got[r0:r0 + n]), f"rows {r0}.."
    rows = sorted(set([0, 15, 16, 2047, 4095, 4096, 4099] + rng.choice(M, 24, replace=False).tolist()))
    yo, e, ab = oracle.expand(h[rows, :r], Bm, y[rows], 2.0)
    check_expand(got[rows], yo, e, ab, y[rows], f"large-M expand r={r}", r=r)


def test_sgmv_expand_large_m_tiles_bitwise():
    """Multi-adapter expand at a size that walks several tiles per workgroup:
    ids in runs (including -1 and out-of-range ids, runs that straddle tiles),
    ranks 5 / 16 / 37 / 64.  Each token's y bits equal the single-adapter
    lora_expand of its adapter on its rows; tokens without an adapter keep y."""
    t = torch()
    M, N = 4100, 4104
    ranks = [5, 16, 37, 64]
    n = len(ranks)
    rng = np.random.default_rng(9)
    ids = np.empty(M, np.int32)
    pos = 0
    while pos < M:
        run = int(rng.integers(1, 300))
        ids[pos:pos + run] = rng.choice([-1, 0, 1, 2, 3, 9])
        pos += run
    r_max = 64
    h = rng.normal(0, 0.5, (M, r_max)).astype(np.float32)
    y = normal_bf16((M, N), 1.0, 1, "slmy")
    Bs, Bg = [], []
    for a, r in enumerate(ranks):
        ldb = (r + 7) // 8 * 8
        Bm = normal_bf16((N, r), 0.02, a, "slmB")
        Bp = np.zeros((N, ldb), np.uint16)
        Bp[:, :r] = Bm
        Bs.append(Bm)
        Bg.append(bf16_to_gpu(Bp))
    scales = np.array([2.0, 0.5, 1.0, 2.0], np.float32)
    Bptr = t.tensor([b.data_ptr() for b in Bg], dtype=t.int64, device="cuda")
    hg = f32_to_gpu(h)
    yg = bf16_to_gpu(y)
    dsl.lora_sgmv_expand(hg, Bptr, t.from_numpy(np.array(ranks, np.int32)).cuda(), t.from_numpy(scales).cuda(),
                         t.from_numpy(ids).cuda(), n, yg, r_max)
    got = bf16_from_gpu(yg)
    none = (ids < 0) | (ids >= n)
    assert np.array_equal(got[none], y[none])
    for a, r in enumerate(ranks):
        sel = np.nonzero(ids == a)[0]
        if len(sel) == 0:
            continue
        hs = np.ascontiguousarray(h[sel])
        ys = bf16_to_gpu(y[sel])
        dsl.lora_expand(f32_to_gpu(hs), Bg[a], ys, float(scales[a]), r=r)
        assert np.array_equal(bf16_from_gpu(ys), got[sel]), f"adapter {a}"
        pick = sel[rng.choice(len(sel), min(8, len(sel)), replace=False)]
        yo, e, ab = oracle.expand(h[pick, :r], Bs[a], y[pick], float(scales[a]))
        check_expand(got[pick], yo, e, ab, y[pick], f"sgmv large-M adapter {a}", r=r)


# ---------------------------------------------------------------------------
# the pages' decode shape: one token, hidden 3072, three fused QKV slices
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 4, 8, 16])
def test_fused_qkv_decode_slices(S):
    """Three QKV slices of rank 16 on one token, K = 3072: the rank-48 shrink
    over the stacked A rows gives each slice the bits of its own rank-16
    shrink (rank columns are independent chains), for the two-launch and
    single-launch deterministic shrinks; h agrees with the oracle, and the
    atomic variant agrees within the stated tolerance."""
    t = torch()
    K = 3072
    for M in (1, 5):
        c = single_adapter_case(M, K, 48, 0, split_k=S, scale=1.0, seed=70 + M)
        xg, Ag = bf16_to_gpu(c.x), bf16_to_gpu(c.A)
        ws = workspace(dsl.lora_shrink_workspace_bytes(M, 48, S))
        h48 = t.full((M, 48), float("nan"), dtype=t.float32, device="cuda")
        dsl.lora_shrink_splitk(xg, Ag, h48, ws if S > 1 else None, S, 1.0)
        cnt = t.zeros(dsl.lora_shrink_counter_bytes(M) // 4, dtype=t.int32, device="cuda")
        h1 = t.full((M, 48), float("nan"), dtype=t.float32, device="cuda")
        dsl.lora_shrink_splitk_counted(xg, Ag, h1, counted_workspace(M, 48, S) if S > 1 else None,
                                       cnt if S > 1 else None, S, 1.0)
        ha = t.full((M, 48), float("nan"), dtype=t.float32, device="cuda")
        dsl.lora_shrink_splitk_atomic(xg, Ag, ha, S, 1.0)
        slices = []
        for q in range(3):
            hq = t.full((M, 16), float("nan"), dtype=t.float32, device="cuda")
            dsl.lora_shrink_splitk(xg, bf16_to_gpu(np.ascontiguousarray(c.A[16 * q:16 * q + 16])), hq,
                                   ws if S > 1 else None, S, 1.0)
            slices.append(hq)
        t.cuda.synchronize()
        b48 = f32_bits(h48)
        for q in range(3):
            assert np.array_equal(b48[:, 16 * q:16 * q + 16], f32_bits(slices[q])), f"slice {q}"
        assert np.array_equal(f32_bits(h1), b48)
        plan = dsl.lora_shrink_plan(K, 48, S)
        check_shrink(h48.cpu().numpy(), c.x, c.A, 1.0, plan, f"qkv S={S} M={M}")
        check_shrink(ha.cpu().numpy(), c.x, c.A, 1.0, plan, f"qkv atomic S={S} M={M}", atomic=True)


# ---------------------------------------------------------------------------
# compensated expand (h as bf16 hi + bf16 lo)
# ---------------------------------------------------------------------------
def test_expand_compensated_golden_bitwise():
    """The hand-derived cases, on the GPU: bit for bit the oracle's outputs,
    which keep the residual of h that lora_expand drops."""
    import json
    import os
    t = torch()
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "compensated_expand.json")))
    for c in gold["cases"]:
        h = np.array(c["h"], dtype=np.float32)
        r = h.shape[1]
        ldh = (r + 3) // 4 * 4
        hp = np.zeros((h.shape[0], ldh), np.float32)
        hp[:, :r] = h
        Bv = np.array(c["B"], dtype=np.float32)
        yv = np.array(c["y"], dtype=np.float32)
        N = Bv.shape[0]
        Np = (N + 7) // 8 * 8                     # N % 8 == 0; extra columns of B are 0, of y are 0
        ldb = (r + 7) // 8 * 8
        Bb = np.zeros((Np, ldb), np.uint16)
        Bb[:N, :r] = (Bv.view(np.uint32) >> 16).astype(np.uint16)
        yb = np.zeros((h.shape[0], Np), np.uint16)
        yb[:, :N] = (yv.view(np.uint32) >> 16).astype(np.uint16)
        for fn, key in ((dsl.lora_expand_compensated, "compensated_out"), (dsl.lora_expand, "plain_out")):
            yg = bf16_to_gpu(yb)
            fn(f32_to_gpu(hp), bf16_to_gpu(Bb), yg, c["scale"], r=r)
            t.cuda.synchronize()
            got = oracle.bf16_to_f64(bf16_from_gpu(yg))[:, :N]
            assert np.array_equal(got, np.array(c[key])), (c["name"], key, got)


@pytest.mark.parametrize("M,r,N", [(1, 16, 4096), (37, 5, 1032), (64, 64, 520), (300, 33, 2048), (40, 128, 1032)])
def test_expand_compensated_parity(M, r, N):
    """Random fp32 h (full 24-bit significands): the compensated expand agrees
    with the oracle's compensated definition within 1 bf16 ulp (plus the fp32
    accumulation floor); it matches the correctly rounded product of the fp32
    h far more often than lora_expand does."""
    t = torch()
    rng = np.random.default_rng(300 + r)
    ldh = (r + 3) // 4 * 4
    h = np.zeros((M, ldh), np.float32)
    h[:, :r] = (rng.standard_normal((M, r)) * 0.5).astype(np.float32)
    Bm = normal_bf16((N, r), 0.05, r, "cpB")
    ldb = (r + 7) // 8 * 8
    Bp = np.zeros((N, ldb), np.uint16)
    Bp[:, :r] = Bm
    y = np.zeros((M, N), np.uint16)               # y = 0: the output is the product itself
    yc = bf16_to_gpu(y)
    dsl.lora_expand_compensated(f32_to_gpu(h), bf16_to_gpu(Bp), yc, 2.0, r=r)
    yp = bf16_to_gpu(y)
    dsl.lora_expand(f32_to_gpu(h), bf16_to_gpu(Bp), yp, 2.0, r=r)
    t.cuda.synchronize()
    gc, gp = bf16_from_gpu(yc), bf16_from_gpu(yp)
    yo, e, ab = oracle.expand_compensated(h[:, :r], Bm, y, 2.0)
    check_expand(gc, yo, e, ab, y, f"compensated M={M} r={r}", r=r)
    # correctly rounded product with the fp32 h itself (no conversion of h)
    exact = 2.0 * (h[:, :r].astype(np.float64) @ oracle.bf16_to_f64(Bm).T)
    want = oracle.bf16_rne(exact)
    match_c = float(np.mean(gc == want))
    match_p = float(np.mean(gp == want))
    assert match_c > 0.97 and match_c > match_p, (match_c, match_p)


@pytest.mark.parametrize("r", [16, 37, 64, 128])
def test_expand_compensated_large_m_tiles_bitwise(r):
    """At M x N large enough that lora_expand_compensated walks several tiles
    per workgroup (hi and lo halves of h staged in LDS), every row equals the
    one-tile-per-workgroup result of a small call on the same rows bit for
    bit, and sampled rows agree with the oracle's compensated expand."""
    M, N = 4100, 4104
    _say(f"large-M compensated expand r={r} M={M} N={N}")
    ldh = (r + 3) // 4 * 4
    ldb = (r + 7) // 8 * 8
    rng = np.random.default_rng(70 + r)
    h = np.zeros((M, ldh), np.float32)
    h[:, :r] = rng.normal(0, 0.5, (M, r)).astype(np.float32)
    h[:, r:] = np.nan                         # padding must never be read
    Bm = normal_bf16((N, r), 0.02, r, "cmB")
    Bp = np.zeros((N, ldb), np.uint16)
    Bp[:, :r] = Bm
    y = normal_bf16((M, N), 1.0, r, "cmy")
    hg, Bg = f32_to_gpu(h), bf16_to_gpu(Bp)
    yg = bf16_to_gpu(y)
    dsl.lora_expand_compensated(hg, Bg, yg, 2.0, r=r)
    got = bf16_from_gpu(yg)
    for r0 in (0, 1008, 4096 - 16, 4100 - 37):
        n = min(64, M - r0)
        ys = bf16_to_gpu(y[r0:r0 + n])
        dsl.lora_expand_compensated(hg[r0:r0 + n], Bg, ys, 2.0, r=r)
        assert np.array_equal(bf16_from_gpu(ys), got[r0:r0 + n]), f"rows {r0}.."
    rows = sorted(set([0, 15, 16, 2047, 4095, 4096, 4099] + rng.choice(M, 24, replace=False).tolist()))
    yo, e, ab = oracle.expand_compensated(h[rows, :r], Bm, y[rows], 2.0)
    check_expand(got[rows], yo, e, ab, y[rows], f"large-M compensated expand r={r}", r=r)


# ---------------------------------------------------------------------------
# multi-adapter shrink + expand in two launches (expand reads the workspace)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("case", ["qkv", "mixed", "decode", "large", "large_s16", "rank128"])
def test_sgmv_shrink_expand_bitwise(case):
    """lora_sgmv_shrink_expand gives the h and y bits of lora_sgmv_shrink
    (with the shrink scales) followed by lora_sgmv_expand (with the expand
    scales): tokens without an adapter keep y, ranks below r_max and not a
    multiple of 8 included.  The larger cases take the three-launch schedule
    (with h, and with h kept in the workspace); a third call, with h rows that
    are not a multiple of 16 bytes, keeps the tree in the expand, which walks
    several tiles per workgroup at large M.  Sampled rows agree with the
    oracle."""
    t = torch()
    if case == "qkv":
        c = sgmv_case(512, 4096, 6144, [64, 64, 64, 64], 1, 64, 8, seed=11, tag="se_q")
    elif case == "mixed":
        rng = np.random.default_rng(12)
        ids = rng.choice([-1, 0, 1, 2, 3, 7], 333).astype(np.int32)
        ids[40:140] = 1
        c = sgmv_case(333, 2048, 520, [5, 16, 37, 64], 0, 0, 16, seed=12, tag="se_m", ids=ids)
    elif case == "decode":
        c = sgmv_case(24, 8192, 1024, [64, 8, 32, 16] * 6, 0, 0, 8, seed=13, tag="se_d",
                      ids=np.arange(24, dtype=np.int32))
    elif case == "large":
        c = sgmv_case(4100, 1024, 4104, [8, 16, 32, 64, 5, 40], 16, 300, 4, seed=14, tag="se_l")
    elif case == "rank128":
        c = sgmv_case(1100, 1024, 2056, [128, 8, 65, 96], 1, 200, 8, seed=16, tag="se_r")
    else:                                          # 17 column blocks x 16 splits: tree kernel, then expand
        c = sgmv_case(4100, 1024, 4104, [8, 16, 32, 64, 5, 40], 16, 300, 16, seed=15, tag="se_l16")
    _say(f"sgmv shrink+expand {case} M={c.M} N={c.N}")
    n = len(c.ranks)
    As = [bf16_to_gpu(a) for a in c.As]
    Bs = []
    for b in c.Bs:
        r = b.shape[1]
        bp = np.zeros((c.N, (r + 7) // 8 * 8), np.uint16)
        bp[:, :r] = b
        Bs.append(bf16_to_gpu(bp))
    Ap = t.tensor([a.data_ptr() for a in As], dtype=t.int64, device="cuda")
    Bp = t.tensor([b.data_ptr() for b in Bs], dtype=t.int64, device="cuda")
    ranks = t.from_numpy(c.ranks).cuda()
    sh = np.array([0.5, 2.0, 1.0, 0.25] * ((n + 3) // 4), np.float32)[:n]
    ex = np.array([2.0, 1.0, 0.5, 3.0] * ((n + 3) // 4), np.float32)[:n]
    shg, exg = t.from_numpy(sh).cuda(), t.from_numpy(ex).cuda()
    idg, plan = _build_plan(c.ids, n)
    xg = bf16_to_gpu(c.x)
    ws = workspace(dsl.lora_sgmv_workspace_bytes(c.M, c.r_max, c.split_k))
    h1 = t.full((c.M, c.r_max), float("nan"), dtype=t.float32, device="cuda")
    dsl.lora_sgmv_shrink(xg, Ap, c.K, ranks, shg, idg, n, plan, h1, c.r_max, c.split_k, ws)
    y1 = bf16_to_gpu(c.y)
    dsl.lora_sgmv_expand(h1, Bp, ranks, exg, idg, n, y1, c.r_max)
    ws2 = workspace(dsl.lora_sgmv_workspace_bytes(c.M, c.r_max, c.split_k))
    h2 = t.full((c.M, c.r_max), float("nan"), dtype=t.float32, device="cuda")
    y2 = bf16_to_gpu(c.y)
    dsl.lora_sgmv_shrink_expand(xg, Ap, c.K, Bp, ranks, shg, exg, idg, n, plan, y2, c.r_max, c.split_k, ws2, h=h2)
    y3 = bf16_to_gpu(c.y)
    dsl.lora_sgmv_shrink_expand(xg, Ap, c.K, Bp, ranks, shg, exg, idg, n, plan, y3, c.r_max, c.split_k, ws2)
    # h rows that are not a multiple of 16 bytes: the tree always goes into the expand
    h4 = t.full((c.M, c.r_max + 1), float("nan"), dtype=t.float32, device="cuda")[:, :c.r_max]
    y4 = bf16_to_gpu(c.y)
    dsl.lora_sgmv_shrink_expand(xg, Ap, c.K, Bp, ranks, shg, exg, idg, n, plan, y4, c.r_max, c.split_k, ws2, h=h4)
    t.cuda.synchronize()
    assert np.array_equal(f32_bits(h1), f32_bits(h2)) and np.array_equal(f32_bits(h1), f32_bits(h4))
    g1 = bf16_from_gpu(y1)
    assert np.array_equal(g1, bf16_from_gpu(y2)) and np.array_equal(g1, bf16_from_gpu(y3))
    assert np.array_equal(g1, bf16_from_gpu(y4))
    hh = h2.cpu().numpy()
    rng = np.random.default_rng(5)
    for i in sorted(rng.choice(c.M, min(12, c.M), replace=False).tolist()):
        a = int(c.ids[i])
        if a < 0 or a >= n:
            assert np.all(hh[i] == 0.0) and np.array_equal(g1[i], c.y[i])
            continue
        r = int(c.ranks[a])
        check_shrink(hh[i:i + 1, :r], c.x[i:i + 1], c.As[a], float(sh[a]),
                     dsl.lora_shrink_plan(c.K, r, c.split_k), f"{case} h row {i}")
        yo, e, ab = oracle.expand(hh[i:i + 1, :r], c.Bs[a], c.y[i:i + 1], float(ex[a]))
        check_expand(g1[i:i + 1], yo, e, ab, c.y[i:i + 1], f"{case} y row {i}", r=r)

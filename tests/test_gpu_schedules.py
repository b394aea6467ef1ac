"""Batch invariance across every schedule switch, through the C-ABI library.

The entry points pick their launch schedule from the batch size: rank tiles
per shrink workgroup, row blocks per workgroup (one, two or four sharing A, or
the A-in-registers kernel with 4 to 16 row blocks per item), tiles per expand
workgroup, waves and XCD mapping of the tree + expand kernel, and one, two or
three launches.  None of these choices may change a bit: every variant runs
the same per-element chains, wave tree, Split-K tree and expand arithmetic,
and differs only in which workgroup computes which element.  The
batch-invariance experiment of the pages (the same row gives the same bits
whatever batch it is part of) is therefore run here at every row-block count
from 1 up to past the last switch for each workload shape: 16 probe rows at
fresh random positions among N(0,1) filler rows, every probe's h (fp32 bits)
and y (bf16 bits) compared with those of the probe rows computed alone - also
for the single-launch shrinks, whose tagged workspace and counters must be
back at zero after every batch size.  The
batch size M runs through 1..5, 64, 65 and one ragged M per row-block count
(M = 16 b - (7 b mod 16)), so every rule of the form "M below / at least a
bound" is seen from both sides.  The probe rows computed alone are checked
against the oracle.
"""
import numpy as np
import pytest

import deterministic_split_lora_amd as dsl
import oracle
from synth import normal_bf16
from tests.helpers import bf16_from_gpu, bf16_to_gpu, check_expand, check_shrink, f32_bits, gpu_available, torch

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

P = 16          # probe rows


def _say(*a):
    print(*a, flush=True)


def _batch_sizes(last_block):
    ms = {1, 2, 3, 4, 5, 64, 65}
    ms.update(16 * b - (7 * b) % 16 for b in range(1, last_block + 1))
    return sorted(m for m in ms if m <= 16 * last_block)


def _filler(gen, rows, cols):
    t = torch()
    return t.randn((rows, cols), generator=gen, device="cuda", dtype=t.float32).to(t.bfloat16)


# (label, K, r, N, split_k, last row-block count).  The last count lies past the
# final switch of the shape's rules: the A-in-registers kernel takes its 16th
# row block per item at 512 row blocks for split 8 (where it applies), the
# shrink's shared-A grouping switches at 2048 (row block, split) pairs, the
# expand's tiles per workgroup at 3072 one-tile workgroups, the tree's place
# at M r (column blocks) = 2^19.
SINGLE_SHAPES = [
    ("q_proj", 4096, 16, 4096, 8, 520),
    ("rank 64, N 6144", 4096, 64, 6144, 8, 520),
    ("MLP down", 14336, 32, 4096, 8, 264),
    ("small A, single launch up to 64 rows", 1024, 8, 1024, 8, 520),
]


@pytest.mark.parametrize("label,K,r,N,S,last", SINGLE_SHAPES)
def test_batch_invariance_every_row_block_count(label, K, r, N, S, last, record_property):
    t = torch()
    seed = K + r + N
    probe = normal_bf16((P, K), 1.0, seed, "sched_x")
    A = normal_bf16((r, K), 0.02, seed, "sched_A")
    B = normal_bf16((N, r), 0.02, seed, "sched_B")
    ybase = normal_bf16((P, N), 1.0, seed, "sched_y")
    Ag, Bg = bf16_to_gpu(A), bf16_to_gpu(B)
    xp, yp = bf16_to_gpu(probe), bf16_to_gpu(ybase)

    # the probe rows alone: shrink, then expand
    h0 = t.empty((P, r), dtype=t.float32, device="cuda")
    dsl.lora_shrink_splitk(xp, Ag, h0, t.empty(dsl.lora_shrink_workspace_bytes(P, r, S), dtype=t.uint8,
                                               device="cuda"), S, 1.0)
    y0 = yp.clone()
    dsl.lora_expand(h0, Bg, y0, 2.0)
    ref_h, ref_y = h0.view(t.int32).clone(), y0.view(t.int16).clone()

    Ms = _batch_sizes(last)
    Mmax = Ms[-1]
    _say(f"schedules {label}: K={K} r={r} N={N} S={S}, {len(Ms)} batch sizes up to {Mmax}")
    gen = t.Generator(device="cuda")
    gen.manual_seed(seed)
    X, Y = _filler(gen, Mmax, K), _filler(gen, Mmax, N)
    H = t.empty((Mmax, r), dtype=t.float32, device="cuda")
    ws = t.empty(max(dsl.lora_shrink_expand_workspace_bytes(Mmax, r, S),
                     dsl.lora_shrink_workspace_bytes(Mmax, r, S)), dtype=t.uint8, device="cuda")
    # the single-launch shrink's own buffers (tagged slots and counters, zero between calls)
    cws = t.zeros(dsl.lora_counted_workspace_bytes(Mmax, r, S), dtype=t.uint8, device="cuda")
    cnt = t.zeros(dsl.lora_shrink_counter_bytes(Mmax) // 4, dtype=t.int32, device="cuda")
    bad = t.zeros((len(Ms), 3), dtype=t.int64, device="cuda")
    rng = np.random.default_rng(seed)
    launches = {}
    for i, M in enumerate(Ms):
        n = min(P, M)
        pos = t.from_numpy(rng.choice(M, size=n, replace=False)).cuda()
        which = t.from_numpy(rng.choice(P, size=n, replace=False)).cuda()
        x, y, h = X[:M], Y[:M], H[:M]
        saved = x[pos].clone()
        x[pos] = xp[which]
        # lora_shrink_expand: one, two or three launches by M
        y[pos] = yp[which]
        dsl.lora_shrink_expand(x, Ag, Bg, y, ws, S, 1.0, 2.0, h=h)
        bad[i, 0] += (h[pos].view(t.int32) != ref_h[which]).sum() + (y[pos].view(t.int16) != ref_y[which]).sum()
        # lora_shrink_splitk + lora_expand: their own schedule rules
        y[pos] = yp[which]
        dsl.lora_shrink_splitk(x, Ag, h, ws, S, 1.0)
        dsl.lora_expand(h, Bg, y, 2.0)
        bad[i, 1] += (h[pos].view(t.int32) != ref_h[which]).sum() + (y[pos].view(t.int16) != ref_y[which]).sum()
        # lora_shrink_splitk_counted: one launch, the split that starts last combines
        h.fill_(float("nan"))
        dsl.lora_shrink_splitk_counted(x, Ag, h, cws, cnt, S, 1.0)
        bad[i, 2] += (h[pos].view(t.int32) != ref_h[which]).sum()
        x[pos] = saved
        nl = dsl.lora_shrink_expand_launches(M, K, r, N, S)
        launches[nl] = launches.get(nl, 0) + 1
    t.cuda.synchronize()
    b = bad.cpu().numpy()
    wrong = [(Ms[i], int(b[i, 0]), int(b[i, 1]), int(b[i, 2])) for i in range(len(Ms)) if b[i].any()]
    record_property("launch_counts_seen", launches)
    assert not wrong, f"{label}: probe bits changed at (M, shrink_expand, splitk+expand, counted) {wrong[:10]}"
    assert int(cnt.abs().sum()) == 0 and int(cws.count_nonzero()) == 0
    _say(f"  {len(Ms)} batch sizes identical; launches seen {launches}")

    # and the probe rows are right
    h_ref = ref_h.cpu().numpy().view(np.float32)
    check_shrink(h_ref, probe, A, 1.0, dsl.lora_shrink_plan(K, r, S), f"{label} probe h")
    yo, e, ab = oracle.expand(h_ref, B, ybase, 2.0)
    check_expand(bf16_from_gpu(y0), yo, e, ab, ybase, f"{label} probe y", r=r)


def _segment_ids(M, lo, hi, n, rng):
    ids = np.empty(M, np.int32)
    s = 0
    while s < M:
        ln = min(int(rng.integers(lo, hi + 1)), M - s)
        ids[s:s + ln] = int(rng.integers(0, n))
        s += ln
    return ids


# (label, K, N, ranks, split_k, segment lengths, last row-block count).  Past
# the last switch: the A-in-registers kernel reaches 16 row blocks per item
# near 510 (split 8) and 230 (split 16) row blocks; the multi-adapter expand
# walks up to 16 tiles per workgroup from 32768 one-tile workgroups (293 row
# blocks at N = 28672).
SGMV_SHAPES = [
    ("4 adapters of rank 64, N 6144", 4096, 6144, [64] * 4, 8, (1, 64), 520),
    ("32 adapters of ranks 8-64, N 28672", 8192, 28672, [8, 16, 32, 64] * 8, 16, (32, 512), 300),
]


@pytest.mark.parametrize("label,K,N,ranks,S,seg,last", SGMV_SHAPES)
def test_sgmv_batch_invariance_every_row_block_count(label, K, N, ranks, S, seg, last):
    t = torch()
    n = len(ranks)
    r_max = max(ranks)
    seed = K + N + n
    As = [normal_bf16((ranks[a], K), 0.02, seed, f"sched_sA{a}") for a in range(n)]
    Bs = [normal_bf16((N, ranks[a]), 0.02, seed, f"sched_sB{a}") for a in range(n)]
    Ag = [bf16_to_gpu(a) for a in As]
    Bg = []
    for b in Bs:
        bp = np.zeros((N, (b.shape[1] + 7) // 8 * 8), np.uint16)
        bp[:, :b.shape[1]] = b
        Bg.append(bf16_to_gpu(bp))
    Ap = t.tensor([a.data_ptr() for a in Ag], dtype=t.int64, device="cuda")
    Bp = t.tensor([b.data_ptr() for b in Bg], dtype=t.int64, device="cuda")
    rk = t.tensor(ranks, dtype=t.int32, device="cuda")
    sh_np = np.array([0.5, 2.0, 1.0, 0.25] * (n // 4), np.float32)
    ex_np = np.array([2.0, 1.0, 0.5, 3.0] * (n // 4), np.float32)
    sh, ex = t.from_numpy(sh_np).cuda(), t.from_numpy(ex_np).cuda()

    probe = normal_bf16((P, K), 1.0, seed, "sched_sx")
    ybase = normal_bf16((P, N), 1.0, seed, "sched_sy")
    pid_np = (np.arange(P) * 5 % n).astype(np.int32)          # the probes' adapters
    xp, yp, pid = bf16_to_gpu(probe), bf16_to_gpu(ybase), t.from_numpy(pid_np).cuda()

    # the probe rows alone: multi-adapter shrink, then expand
    plan0 = t.zeros(dsl.lora_sgmv_plan_bytes(P), dtype=t.uint8, device="cuda")
    dsl.lora_sgmv_plan(pid, n, plan0)
    h0 = t.zeros((P, r_max), dtype=t.float32, device="cuda")
    dsl.lora_sgmv_shrink(xp, Ap, K, rk, sh, pid, n, plan0, h0, r_max, S,
                         t.empty(dsl.lora_sgmv_workspace_bytes(P, r_max, S), dtype=t.uint8, device="cuda"))
    y0 = yp.clone()
    dsl.lora_sgmv_expand(h0, Bp, rk, ex, pid, n, y0, r_max)
    # columns at or past a probe's rank are not compared
    cols = t.arange(r_max, device="cuda")[None, :] < t.tensor([ranks[a] for a in pid_np], device="cuda")[:, None]
    ref_h, ref_y = t.where(cols, h0, 0.0).view(t.int32).clone(), y0.view(t.int16).clone()

    Ms = _batch_sizes(last)
    Mmax = Ms[-1]
    _say(f"sgmv schedules {label}: K={K} N={N} S={S}, {len(Ms)} batch sizes up to {Mmax}")
    gen = t.Generator(device="cuda")
    gen.manual_seed(seed)
    X, Y = _filler(gen, Mmax, K), _filler(gen, Mmax, N)
    rng = np.random.default_rng(seed)
    IDS = t.from_numpy(_segment_ids(Mmax, seg[0], seg[1], n, rng)).cuda()
    H = t.zeros((Mmax, r_max), dtype=t.float32, device="cuda")
    ws = t.empty(dsl.lora_sgmv_workspace_bytes(Mmax, r_max, S), dtype=t.uint8, device="cuda")
    plan = t.zeros(dsl.lora_sgmv_plan_bytes(Mmax), dtype=t.uint8, device="cuda")
    cws = t.zeros(dsl.lora_counted_workspace_bytes(Mmax, r_max, S), dtype=t.uint8, device="cuda")
    cnt = t.zeros(dsl.lora_sgmv_counter_bytes(Mmax) // 4, dtype=t.int32, device="cuda")
    bad = t.zeros((len(Ms), 3), dtype=t.int64, device="cuda")

    def differ(h, y, pos, which):
        hp = t.where(cols[which], h[pos], 0.0).view(t.int32)
        return (hp != ref_h[which]).sum() + (y[pos].view(t.int16) != ref_y[which]).sum()

    for i, M in enumerate(Ms):
        m = min(P, M)
        pos = t.from_numpy(rng.choice(M, size=m, replace=False)).cuda()
        which = t.from_numpy(rng.choice(P, size=m, replace=False)).cuda()
        x, y, h, ids = X[:M], Y[:M], H[:M], IDS[:M]
        saved_x, saved_id = x[pos].clone(), ids[pos].clone()
        x[pos] = xp[which]
        ids[pos] = pid[which]
        dsl.lora_sgmv_plan(ids, n, plan)
        # the pipeline: two or three launches by M
        y[pos] = yp[which]
        dsl.lora_sgmv_shrink_expand(x, Ap, K, Bp, rk, sh, ex, ids, n, plan, y, r_max, S, ws, h=h)
        bad[i, 0] += differ(h, y, pos, which)
        # lora_sgmv_shrink + lora_sgmv_expand
        y[pos] = yp[which]
        dsl.lora_sgmv_shrink(x, Ap, K, rk, sh, ids, n, plan, h, r_max, S, ws)
        dsl.lora_sgmv_expand(h, Bp, rk, ex, ids, n, y, r_max)
        bad[i, 1] += differ(h, y, pos, which)
        # lora_sgmv_shrink_counted: one launch (h only)
        h.fill_(float("nan"))
        dsl.lora_sgmv_shrink_counted(x, Ap, K, rk, sh, n, plan, h, r_max, S, cws, cnt)
        bad[i, 2] += (t.where(cols[which], h[pos], 0.0).view(t.int32) != ref_h[which]).sum()
        x[pos], ids[pos] = saved_x, saved_id
    t.cuda.synchronize()
    b = bad.cpu().numpy()
    wrong = [(Ms[i], int(b[i, 0]), int(b[i, 1]), int(b[i, 2])) for i in range(len(Ms)) if b[i].any()]
    assert not wrong, f"{label}: probe bits changed at (M, shrink_expand, shrink+expand, counted) {wrong[:10]}"
    assert int(cnt.abs().sum()) == 0 and int(cws.count_nonzero()) == 0
    _say(f"  {len(Ms)} batch sizes identical")

    # and the probe rows are right
    hh = h0.cpu().numpy()
    yy = bf16_from_gpu(y0)
    for j in range(P):
        a = int(pid_np[j])
        r = ranks[a]
        check_shrink(hh[j:j + 1, :r], probe[j:j + 1], As[a], float(sh_np[a]), dsl.lora_shrink_plan(K, r, S),
                     f"{label} probe {j} h")
        yo, e, ab = oracle.expand(hh[j:j + 1, :r], Bs[a], ybase[j:j + 1], float(ex_np[a]))
        check_expand(yy[j:j + 1], yo, e, ab, ybase[j:j + 1], f"{label} probe {j} y", r=r)


@pytest.mark.parametrize("multi", [False, True])
def test_offsets_beyond_32_bits(multi):
    """Batches whose x and y each hold more than 2^31 elements (524 293 tokens
    x 4096 in, x 4104 out): every element offset past 2^31 must be formed in
    64 bits.  Probe rows
    placed at the start, the middle and the last rows (past 2^31 / K) of the
    batch give the h and y bits of the probe rows computed alone, through the
    fused entry point and the separate calls (single adapter), or through the
    multi-adapter pipeline (two adapters in alternating segments of 4096
    tokens); the probe rows computed alone are checked against the oracle."""
    t = torch()
    M, K, r, N, S = (1 << 19) + 5, 4096, 16, 4104, 8
    assert M * K > 2 ** 31 and M * N > 2 ** 31
    probe = normal_bf16((P, K), 1.0, 7, "big_x")
    ybase = normal_bf16((P, N), 1.0, 7, "big_y")
    n = 2 if multi else 1
    As = [normal_bf16((r, K), 0.02, 7 + a, "big_A") for a in range(n)]
    Bs = [normal_bf16((N, r), 0.02, 7 + a, "big_B") for a in range(n)]
    Ag, Bg = [bf16_to_gpu(a) for a in As], [bf16_to_gpu(b) for b in Bs]
    xp, yp = bf16_to_gpu(probe), bf16_to_gpu(ybase)
    pos = np.array([0, 1, 2, 3, 4095, 4096, 262144, 262145, M // 2, M - 9, M - 8, M - 5, M - 4, M - 3, M - 2,
                    M - 1], dtype=np.int64)
    ids_np = ((np.arange(M) // 4096) % n).astype(np.int32)
    pid = ids_np[pos]
    _say(f"offsets past 2^31: M={M} K={K} multi={multi}")
    # the probe rows alone
    h0 = t.zeros((P, r), dtype=t.float32, device="cuda")
    y0 = yp.clone()
    for a in range(n):
        sel = np.nonzero(pid == a)[0]
        if len(sel) == 0:
            continue
        sg = t.from_numpy(sel).cuda()
        ha = t.empty((len(sel), r), dtype=t.float32, device="cuda")
        dsl.lora_shrink_splitk(xp[sg].contiguous(), Ag[a], ha,
                               t.empty(dsl.lora_shrink_workspace_bytes(len(sel), r, S), dtype=t.uint8,
                                       device="cuda"), S, 1.0)
        ya = yp[sg].contiguous()
        dsl.lora_expand(ha, Bg[a], ya, 2.0)
        h0[sg] = ha
        y0[sg] = ya
    ref_h, ref_y = h0.view(t.int32).clone(), y0.view(t.int16).clone()

    gen = t.Generator(device="cuda")
    gen.manual_seed(11)
    x = _filler(gen, M, K)
    y = _filler(gen, M, N)
    pg = t.from_numpy(pos).cuda()
    x[pg] = xp
    h = t.empty((M, r), dtype=t.float32, device="cuda")
    if multi:
        Ap = t.tensor([a.data_ptr() for a in Ag], dtype=t.int64, device="cuda")
        Bp = t.tensor([b.data_ptr() for b in Bg], dtype=t.int64, device="cuda")
        rk = t.full((n,), r, dtype=t.int32, device="cuda")
        ids = t.from_numpy(ids_np).cuda()
        plan = t.zeros(dsl.lora_sgmv_plan_bytes(M), dtype=t.uint8, device="cuda")
        dsl.lora_sgmv_plan(ids, n, plan)
        ws = t.empty(dsl.lora_sgmv_workspace_bytes(M, r, S), dtype=t.uint8, device="cuda")
        y[pg] = yp
        dsl.lora_sgmv_shrink_expand(x, Ap, K, Bp, rk, None, t.full((n,), 2.0, device="cuda"), ids, n, plan, y, r,
                                    S, ws, h=h)
        t.cuda.synchronize()
        assert t.equal(h[pg].view(t.int32), ref_h) and t.equal(y[pg].view(t.int16), ref_y), "pipeline"
    else:
        ws = t.empty(max(dsl.lora_shrink_expand_workspace_bytes(M, r, S), dsl.lora_shrink_workspace_bytes(M, r, S)),
                     dtype=t.uint8, device="cuda")
        y[pg] = yp
        dsl.lora_shrink_expand(x, Ag[0], Bg[0], y, ws, S, 1.0, 2.0, h=h)
        t.cuda.synchronize()
        assert t.equal(h[pg].view(t.int32), ref_h) and t.equal(y[pg].view(t.int16), ref_y), "shrink_expand"
        y[pg] = yp
        dsl.lora_shrink_splitk(x, Ag[0], h, ws, S, 1.0)
        dsl.lora_expand(h, Bg[0], y, 2.0)
        t.cuda.synchronize()
        assert t.equal(h[pg].view(t.int32), ref_h) and t.equal(y[pg].view(t.int16), ref_y), "separate calls"
    del x, y, h, ws
    t.cuda.empty_cache()
    h_ref = ref_h.cpu().numpy().view(np.float32)
    y_ref = bf16_from_gpu(y0)
    for a in range(n):
        sel = np.nonzero(pid == a)[0]
        check_shrink(h_ref[sel], probe[sel], As[a], 1.0, dsl.lora_shrink_plan(K, r, S), f"big probe h a={a}")
        yo, e, ab = oracle.expand(h_ref[sel], Bs[a], ybase[sel], 2.0)
        check_expand(y_ref[sel], yo, e, ab, ybase[sel], f"big probe y a={a}", r=r)

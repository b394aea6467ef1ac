"""Shared test plumbing: moving seeded inputs to the GPU and back, and the
tolerance checks that compare the GPU path with the CPU oracle."""
from __future__ import annotations

import numpy as np

import oracle


def torch():
    import torch as _t
    return _t


def gpu_available() -> bool:
    try:
        return torch().cuda.is_available()
    except Exception:
        return False


def bf16_to_gpu(bits: np.ndarray):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(t.bfloat16).cuda()


def bf16_from_gpu(t) -> np.ndarray:
    return t.detach().contiguous().view(torch().int16).cpu().numpy().view(np.uint16)


def f32_to_gpu(a: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def f32_bits(t) -> np.ndarray:
    return t.detach().contiguous().view(torch().int32).cpu().numpy()


def workspace(nbytes: int):
    t = torch()
    return t.empty(max(int(nbytes), 16), dtype=t.uint8, device="cuda")


def counted_workspace(M: int, r_max: int, split_k: int):
    """The single-launch shrinks' own workspace of tagged slots: zero before
    the first call (and left zero by every call)."""
    import deterministic_split_lora_amd as dsl
    t = torch()
    return t.zeros(max(int(dsl.lora_counted_workspace_bytes(M, r_max, split_k)), 16), dtype=t.uint8, device="cuda")


def check_shrink(h_gpu: np.ndarray, x, A, scale: float, plan: dict, what: str = "", atomic: bool = False):
    """Two bounds, both per element:
    * the stated tolerance: |h - ref| <= 1e-3 |scale| ||x_i|| ||A_j||;
    * a rounding bound from the arithmetic: every element is the result of
      one 32-product matrix-core step per step, k_steps accumulating steps, a
      log2(waves)-level and a log2(split_k)-level fp32 tree and one multiply,
      so |h - ref| <= (32 + k_steps + log2 W + log2 S + 2) 2^-24 |scale| sum|x A|;
      the atomic variant adds its S scaled partials one after another in any
      order, which takes S instead of log2 S + 1 in that count.
    Returns (max error / stated tolerance, max error / rounding bound)."""
    ref = oracle.shrink(x, A, scale)
    absum, xn, an = oracle.shrink_bounds(x, A)
    err = np.abs(h_gpu.astype(np.float64) - ref)
    tol = 1e-3 * abs(scale) * np.outer(xn, an)
    split_depth = plan["split_k"] if atomic else int(np.log2(plan["split_k"])) + 1
    depth = 32 + plan["k_steps"] + int(np.log2(plan["waves"])) + split_depth + 1
    rb = depth * 2.0 ** -24 * abs(scale) * absum + 1e-30
    assert np.all(err <= tol), f"{what}: shrink beyond stated tolerance, worst {np.max(err / tol):.3g}"
    assert np.all(err <= rb), f"{what}: shrink beyond rounding bound, worst {np.max(err / rb):.3g}"
    return float(np.max(err / tol)), float(np.max(err / rb))


def expand_floor(r):
    """Coefficient c of the fp32 cancellation floor c 2^-24 (|y| + |s| sum|hb B|).

    The GPU forms acc = sum_{j<r} bf16(h_j) B_jn in fp32 over one, two or four
    chained matrix-core steps: the products are exact and zero-padded slots add
    exactly, so with every fp32 addition rounded to nearest, in any order,
    |acc - sum| <= (r - 1) 2^-24 sum|hb B| to first order.  Then one fused
    multiply-add v = fl(s acc + y) adds 2^-24 |v|.  Together
    |v - e| <= r 2^-24 (|y| + |s| sum|hb B|) + O(2^-48); r + 2 keeps the
    second-order terms inside.  The last rounding, bf16(v), is within half the
    bf16 spacing at v, which is at most bf16_ulp(o) of the oracle's correctly
    rounded value o, so |y_gpu - e| <= bf16_ulp(o) + floor."""
    return np.asarray(r, dtype=np.float64) + 2.0


def check_expand(y_gpu: np.ndarray, yo: np.ndarray, e: np.ndarray, absum: np.ndarray, y_in: np.ndarray,
                 what: str, r: int):
    """|y_gpu - e| <= bf16_ulp(o) + (r + 2) 2^-24 (|y| + |s| sum|hb B|) per
    element (expand_floor); the floor matters only under cancellation.  r is
    the rank, or an array of per-row ranks broadcast against the rows.
    Returns the fraction of elements that differ from the oracle's correctly
    rounded value."""
    got = oracle.bf16_to_f64(y_gpu)
    ulp = oracle.bf16_ulp(yo)
    yv = np.abs(oracle.bf16_to_f64(y_in))
    floor = expand_floor(r) * 2.0 ** -24 * (yv + absum)
    err = np.abs(got - e)
    ok = err <= ulp + floor
    assert np.all(ok), f"{what}: expand beyond 1 bf16 ulp at {np.argwhere(~ok)[:5].tolist()}"
    return float(np.mean(y_gpu != yo))

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


def check_expand(y_gpu: np.ndarray, yo: np.ndarray, e: np.ndarray, absum: np.ndarray, y_in: np.ndarray,
                 what: str = "", r: int = 64):
    """|y_gpu - e| <= 1 bf16 ulp of the oracle's rounded value plus the fp32
    accumulation floor c 2^-24 (|y| + |s| sum|hb B|), c = max(100, r + 36),
    that matters only under cancellation: r products summed in fp32 over at
    most four chained matrix-core steps, one fused multiply-add.  Returns the
    fraction of elements that differ from the oracle's correctly rounded
    value."""
    got = oracle.bf16_to_f64(y_gpu)
    ulp = oracle.bf16_ulp(yo)
    yv = np.abs(oracle.bf16_to_f64(y_in))
    floor = max(100, r + 36) * 2.0 ** -24 * (yv + absum)
    err = np.abs(got - e)
    ok = err <= ulp + floor
    assert np.all(ok), f"{what}: expand beyond 1 bf16 ulp at {np.argwhere(~ok)[:5].tolist()}"
    return float(np.mean(y_gpu != yo))

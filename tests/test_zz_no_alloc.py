"""lora_shrink_expand_noalloc (the entry point that allocates nothing and
keeps its Split-K workspace in the library's fixed per-device buffer) against
lora_shrink_expand with a caller-owned workspace, through the C ABI: h and y
must be equal bit for bit, on consecutive calls of falling size (the buffer
then still holds the previous call's partials), with and without h, across
the one-, two- and three-launch schedules, up to the buffer's limit.  The
results are also checked against the CPU oracle."""
import numpy as np
import pytest

import deterministic_split_lora_amd as dsl
import oracle
from synth import single_adapter_case
from tests.helpers import bf16_from_gpu, bf16_to_gpu, check_expand, check_shrink, f32_bits, gpu_available, torch
from tests.helpers import workspace

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _pair(c, M, K, r, N, S, with_h, seed_tag):
    """(h, y) from lora_shrink_expand_noalloc and from lora_shrink_expand."""
    t = torch()
    xg, Ag, Bg = bf16_to_gpu(c.x), bf16_to_gpu(c.A), bf16_to_gpu(c.B)
    outs = []
    for which in ("noalloc", "workspace"):
        yg = bf16_to_gpu(c.y)
        h = t.full((M, r), float("nan"), dtype=t.float32, device="cuda") if with_h else None
        if which == "noalloc":
            dsl.lora_shrink_expand_noalloc(xg, Ag, Bg, yg, S, 1.0, 2.0, h=h)
        else:
            ws = workspace(dsl.lora_shrink_expand_workspace_bytes(M, r, S))
            dsl.lora_shrink_expand(xg, Ag, Bg, yg, ws, S, 1.0, 2.0, h=h)
        t.cuda.synchronize()
        outs.append((None if h is None else f32_bits(h), bf16_from_gpu(yg)))
    return outs


# (M, K, r, N, S): falling sizes, each call right after the previous one
CALLS = [
    (4096, 4096, 64, 1024, 8),   # the buffer's limit: 8 * 4096 * 64 * 4 = 8 MiB; three launches
    (300, 14336, 32, 4096, 8),   # smaller: partials then tree + expand
    (16, 4096, 16, 4096, 8),     # smaller still: the q_proj decode shape
    (1, 1024, 8, 520, 8),        # A of 16 KiB: the single-launch schedule
]


@pytest.mark.parametrize("with_h", [True, False])
def test_noalloc_matches_workspace_entry_point(with_h):
    t = torch()
    for n, (M, K, r, N, S) in enumerate(CALLS):
        print(f"  call {n}: M={M} K={K} r={r} N={N} S={S} h={'yes' if with_h else 'no'}", flush=True)
        assert S * M * r * 4 <= dsl.NOALLOC_SCRATCH_BYTES
        c = single_adapter_case(M, K, r, N, S, 2.0, seed=40 + n)
        (h_n, y_n), (h_w, y_w) = _pair(c, M, K, r, N, S, with_h, n)
        assert np.array_equal(y_n, y_w), f"call {n}: y differs from lora_shrink_expand"
        if with_h:
            assert np.array_equal(h_n, h_w), f"call {n}: h differs from lora_shrink_expand"
            rows = np.unique(np.linspace(0, M - 1, min(M, 24)).astype(int))
            hv = h_n.view(np.float32)
            check_shrink(hv[rows], c.x[rows], c.A, 1.0, dsl.lora_shrink_plan(K, r, S), f"noalloc call {n}")
            yo, e, ab = oracle.expand(hv[rows], c.B, c.y[rows], 2.0)
            check_expand(y_n[rows], yo, e, ab, c.y[rows], f"noalloc call {n}", r=r)
    t.cuda.synchronize()


def test_noalloc_repeats_and_refuses_oversize():
    """Repeated calls give identical bits; a call past the buffer raises
    before anything is enqueued and leaves y untouched."""
    t = torch()
    M, K, r, N, S = 64, 4096, 16, 4096, 8
    c = single_adapter_case(M, K, r, N, S, 2.0, seed=7)
    xg, Ag, Bg, y0 = bf16_to_gpu(c.x), bf16_to_gpu(c.A), bf16_to_gpu(c.B), bf16_to_gpu(c.y)
    first = None
    for _ in range(50):
        yg = y0.clone()
        dsl.lora_shrink_expand_noalloc(xg, Ag, Bg, yg, S, 1.0, 2.0)
        got = yg.view(t.int16).clone()
        if first is None:
            first = got
        assert t.equal(got, first)
    big = t.zeros((4097, K), dtype=t.bfloat16, device="cuda")
    A64 = t.zeros((64, K), dtype=t.bfloat16, device="cuda")
    B64 = t.zeros((N, 64), dtype=t.bfloat16, device="cuda")
    ybig = t.ones((4097, N), dtype=t.bfloat16, device="cuda")
    with pytest.raises(dsl.LoraError) as ei:
        dsl.lora_shrink_expand_noalloc(big, A64, B64, ybig, S, 1.0, 2.0)
    assert ei.value.status == 7
    t.cuda.synchronize()
    assert bool((ybig == 1).all())

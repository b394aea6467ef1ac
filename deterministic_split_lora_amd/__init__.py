"""Deterministic Split-K LoRA shrink / expand for AMD MI355X (gfx950).

The computation lives in liblora_det.so (hand-written HIP kernels behind the C
interface of include/lora_det.h); this package is its thin Python binding, with
one function per C entry point under the same name.  See the header for the
operand layouts, the determinism contract and the error codes.
"""
from ._binding import (  # noqa: F401
    EXPORTED, LIBRARY_PATH, LoraError, lib, lora_abi_version, lora_expand, lora_sgmv_expand,
    lora_sgmv_plan, lora_sgmv_plan_bytes, lora_sgmv_shrink, lora_sgmv_workspace_bytes, lora_shrink_plan,
    lora_shrink_splitk, lora_shrink_splitk_atomic, lora_shrink_workspace_bytes, lora_status_str,
    lora_shrink_expand, lora_shrink_expand_workspace_bytes, lora_shrink_partials, lora_expand_combine,
    lora_shrink_expand_fused, lora_shrink_expand_launches, lora_shrink_counter_bytes, lora_shrink_splitk_counted,
    lora_sgmv_counter_bytes, lora_sgmv_shrink_counted, lora_shrink_expand_counter_bytes, lora_shrink_expand_counted,
    lora_expand_compensated, lora_sgmv_shrink_expand, lora_shrink_expand_noalloc, NOALLOC_SCRATCH_BYTES,
    lora_sgmv_shrink_atomic, lora_counted_workspace_bytes,
)

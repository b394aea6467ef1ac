"""ctypes binding of liblora_det.so: argument marshalling only.

Each function has the name of the C entry point it calls (include/lora_det.h),
takes torch tensors that already live on the GPU, checks dtypes and that rows
are contiguous, passes raw pointers, row strides and sizes, and raises
``LoraError`` on a nonzero status.  Every step of the computation runs in the
HIP kernels; there is no fallback.  torch is used only for device memory and
the current stream.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY_PATH = os.path.join(_HERE, "liblora_det.so")

LORA_OK = 0
LORA_ERR_NULL = 1
LORA_ERR_SHAPE = 2
LORA_ERR_UNSUPPORTED = 3
LORA_ERR_ALIGN = 4
LORA_ERR_WORKSPACE = 5
LORA_ERR_LAUNCH = 6
LORA_ERR_SCRATCH = 7

EXPORTED = [
    "lora_abi_version", "lora_status_str", "lora_shrink_plan", "lora_shrink_workspace_bytes",
    "lora_shrink_splitk", "lora_shrink_splitk_atomic", "lora_expand", "lora_sgmv_plan_bytes",
    "lora_sgmv_plan", "lora_sgmv_workspace_bytes", "lora_sgmv_shrink", "lora_sgmv_expand",
    "lora_shrink_expand_workspace_bytes", "lora_shrink_expand", "lora_shrink_partials", "lora_expand_combine",
    "lora_shrink_expand_fused", "lora_shrink_expand_launches", "lora_shrink_counter_bytes",
    "lora_shrink_splitk_counted", "lora_sgmv_counter_bytes", "lora_sgmv_shrink_counted",
    "lora_shrink_expand_counter_bytes", "lora_shrink_expand_counted", "lora_expand_compensated",
    "lora_sgmv_shrink_expand", "lora_shrink_expand_noalloc",
    "lora_sgmv_shrink_atomic", "lora_counted_workspace_bytes",
]


class LoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class ShrinkPlan(ctypes.Structure):
    _fields_ = [("split_k", ctypes.c_int32), ("k_chunk", ctypes.c_int32), ("waves", ctypes.c_int32),
                ("k_steps", ctypes.c_int32), ("rank_tiles", ctypes.c_int32), ("row_block", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

# LORA_DET_ABI_VERSION of include/lora_det.h that these signatures follow.
ABI_VERSION = 6


def lib():
    """The loaded library; raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY_PATH):
            raise ImportError(f"{LIBRARY_PATH} is missing: build it with "
                              "`python -m deterministic_split_lora_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIBRARY_PATH)
        L.lora_abi_version.restype = ctypes.c_int
        L.lora_abi_version.argtypes = []
        if L.lora_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIBRARY_PATH} has ABI version {L.lora_abi_version()}, the binding "
                              f"expects {ABI_VERSION}: rebuild it")
        L.lora_status_str.restype = ctypes.c_char_p
        L.lora_status_str.argtypes = [ctypes.c_int]
        L.lora_shrink_plan.restype = ctypes.c_int
        L.lora_shrink_plan.argtypes = [_i64, _i32, _i32, ctypes.POINTER(ShrinkPlan)]
        L.lora_shrink_workspace_bytes.restype = _sz
        L.lora_shrink_workspace_bytes.argtypes = [_i64, _i32, _i32]
        L.lora_shrink_splitk.restype = ctypes.c_int
        L.lora_shrink_splitk.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _f32,
                                         _vp, _sz, _vp]
        L.lora_shrink_splitk_atomic.restype = ctypes.c_int
        L.lora_shrink_splitk_atomic.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _i32,
                                                _f32, _vp]
        L.lora_expand.restype = ctypes.c_int
        L.lora_expand.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i32, _i64, _f32, _vp]
        L.lora_expand_compensated.restype = ctypes.c_int
        L.lora_expand_compensated.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i32, _i64, _f32, _vp]
        L.lora_shrink_expand_workspace_bytes.restype = _sz
        L.lora_shrink_expand_workspace_bytes.argtypes = [_i64, _i32, _i32]
        L.lora_shrink_expand.restype = ctypes.c_int
        L.lora_shrink_expand.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32,
                                         _i64, _i32, _f32, _f32, _vp, _sz, _vp]
        L.lora_sgmv_shrink_atomic.restype = ctypes.c_int
        L.lora_sgmv_shrink_atomic.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _i32, _vp, _sz, _vp, _i64, _i64, _i64,
                                              _i32, _i32, _vp]
        L.lora_shrink_expand_noalloc.restype = ctypes.c_int
        L.lora_shrink_expand_noalloc.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64,
                                                 _i32, _i64, _i32, _f32, _f32, _vp]
        L.lora_shrink_expand_counter_bytes.restype = _sz
        L.lora_shrink_expand_counter_bytes.argtypes = [_i64]
        L.lora_shrink_expand_counted.restype = ctypes.c_int
        L.lora_shrink_expand_counted.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64,
                                                 _i32, _i64, _i32, _f32, _f32, _vp, _sz, _vp, _sz, _vp]
        L.lora_shrink_counter_bytes.restype = _sz
        L.lora_shrink_counter_bytes.argtypes = [_i64]
        L.lora_counted_workspace_bytes.restype = _sz
        L.lora_counted_workspace_bytes.argtypes = [_i64, _i32, _i32]
        L.lora_sgmv_counter_bytes.restype = _sz
        L.lora_sgmv_counter_bytes.argtypes = [_i64]
        L.lora_shrink_splitk_counted.restype = ctypes.c_int
        L.lora_shrink_splitk_counted.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _f32,
                                                 _vp, _sz, _vp, _sz, _vp]
        L.lora_sgmv_shrink_counted.restype = ctypes.c_int
        L.lora_sgmv_shrink_counted.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _i32, _vp, _sz, _vp, _i64, _i64,
                                               _i64, _i32, _i32, _vp, _sz, _vp, _sz, _vp]
        L.lora_shrink_expand_launches.restype = ctypes.c_int
        L.lora_shrink_expand_launches.argtypes = [_i64, _i64, _i32, _i64, _i32]
        L.lora_shrink_expand_fused.restype = ctypes.c_int
        L.lora_shrink_expand_fused.argtypes = [_vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64,
                                               _i32, _i64, _i32, _f32, _f32, _vp]
        L.lora_shrink_partials.restype = ctypes.c_int
        L.lora_shrink_partials.argtypes = [_vp, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _sz, _vp]
        L.lora_expand_combine.restype = ctypes.c_int
        L.lora_expand_combine.argtypes = [_vp, _sz, _i32, _f32, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i32, _i64,
                                          _f32, _vp]
        L.lora_sgmv_plan_bytes.restype = _sz
        L.lora_sgmv_plan_bytes.argtypes = [_i64]
        L.lora_sgmv_plan.restype = ctypes.c_int
        L.lora_sgmv_plan.argtypes = [_vp, _i64, _i32, _vp, _sz, _vp]
        L.lora_sgmv_workspace_bytes.restype = _sz
        L.lora_sgmv_workspace_bytes.argtypes = [_i64, _i32, _i32]
        L.lora_sgmv_shrink.restype = ctypes.c_int
        L.lora_sgmv_shrink.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _i32, _vp, _sz, _vp, _i64, _i64,
                                       _i64, _i32, _i32, _vp, _sz, _vp]
        L.lora_sgmv_expand.restype = ctypes.c_int
        L.lora_sgmv_expand.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, _i32, _vp, _i64, _i64, _i64, _i32, _vp]
        L.lora_sgmv_shrink_expand.restype = ctypes.c_int
        L.lora_sgmv_shrink_expand.argtypes = [_vp, _i64, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _sz, _vp,
                                              _i64, _vp, _i64, _i64, _i64, _i64, _i32, _i32, _vp, _sz, _vp]
        _lib = L
    return _lib


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------
def status_str(status: int) -> str:
    return lib().lora_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != LORA_OK:
        raise LoraError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _ld(t, name):
    import torch
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D")
    if t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous (stride(1) == 1)")
    return t.stride(0)


def _dtype(t, dt, name):
    if t.dtype != dt:
        raise TypeError(f"{name} must be {dt}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")


def _stream(stream, like):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream(like.device).cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


# ----------------------------------------------------------------------------
# entry points
# ----------------------------------------------------------------------------
def lora_abi_version() -> int:
    return int(lib().lora_abi_version())


def lora_status_str(status: int) -> str:
    return status_str(status)


def lora_shrink_plan(K: int, r: int, split_k: int) -> dict:
    p = ShrinkPlan()
    _check(lib().lora_shrink_plan(K, r, split_k, ctypes.byref(p)), "lora_shrink_plan")
    return p.as_dict()


def lora_shrink_workspace_bytes(M: int, r: int, split_k: int) -> int:
    return int(lib().lora_shrink_workspace_bytes(M, r, split_k))


def lora_sgmv_workspace_bytes(M: int, r_max: int, split_k: int) -> int:
    return int(lib().lora_sgmv_workspace_bytes(M, r_max, split_k))


def lora_sgmv_plan_bytes(M: int) -> int:
    return int(lib().lora_sgmv_plan_bytes(M))


def lora_shrink_splitk(x, A, h, workspace=None, split_k: int = 8, scale: float = 1.0, stream=None):
    """h[:M, :r] = scale * fixed_tree_s( x[:, chunk s] @ A[:, chunk s]^T )  (x [M,K] bf16, A [r,K] bf16,
    h fp32, workspace uint8/float tensor of lora_shrink_workspace_bytes)."""
    import torch
    _dtype(x, torch.bfloat16, "x"); _dtype(A, torch.bfloat16, "A"); _dtype(h, torch.float32, "h")
    M, K = x.shape
    r = A.shape[0]
    st = lib().lora_shrink_splitk(_ptr(x), _ld(x, "x"), _ptr(A), _ld(A, "A"), _ptr(h), _ld(h, "h"), M, K, r,
                                  split_k, scale, _ptr(workspace), _nbytes(workspace), _stream(stream, x))
    _check(st, "lora_shrink_splitk")
    return h


def lora_shrink_counter_bytes(M: int) -> int:
    return int(lib().lora_shrink_counter_bytes(M))


def lora_counted_workspace_bytes(M: int, r_max: int, split_k: int) -> int:
    return int(lib().lora_counted_workspace_bytes(M, r_max, split_k))


def lora_sgmv_counter_bytes(M: int) -> int:
    return int(lib().lora_sgmv_counter_bytes(M))


def lora_shrink_splitk_counted(x, A, h, workspace, counters, split_k: int = 8, scale: float = 1.0, stream=None):
    """Single-launch deterministic shrink.  workspace: zero-initialised GPU buffer of
    lora_counted_workspace_bytes(M, r, split_k) bytes, counters: zero-initialised
    int32 GPU tensor of lora_shrink_counter_bytes(M) / 4 elements (both left zero)."""
    import torch
    _dtype(x, torch.bfloat16, "x"); _dtype(A, torch.bfloat16, "A"); _dtype(h, torch.float32, "h")
    if counters is not None:
        _dtype(counters, torch.int32, "counters")
    M, K = x.shape
    r = A.shape[0]
    st = lib().lora_shrink_splitk_counted(_ptr(x), _ld(x, "x"), _ptr(A), _ld(A, "A"), _ptr(h), _ld(h, "h"), M, K,
                                          r, split_k, scale, _ptr(workspace), _nbytes(workspace), _ptr(counters),
                                          _nbytes(counters), _stream(stream, x))
    _check(st, "lora_shrink_splitk_counted")
    return h


def lora_shrink_splitk_atomic(x, A, h, split_k: int = 8, scale: float = 1.0, stream=None):
    import torch
    _dtype(x, torch.bfloat16, "x"); _dtype(A, torch.bfloat16, "A"); _dtype(h, torch.float32, "h")
    M, K = x.shape
    r = A.shape[0]
    st = lib().lora_shrink_splitk_atomic(_ptr(x), _ld(x, "x"), _ptr(A), _ld(A, "A"), _ptr(h), _ld(h, "h"),
                                         M, K, r, split_k, scale, _stream(stream, x))
    _check(st, "lora_shrink_splitk_atomic")
    return h


def lora_expand(h, B, y, scale: float, r: int | None = None, stream=None):
    """y[:M, :N] = bf16(fma(scale, bf16(h[:, :r]) @ B[:, :r]^T, y))  in place (B [N, r] bf16)."""
    import torch
    _dtype(h, torch.float32, "h"); _dtype(B, torch.bfloat16, "B"); _dtype(y, torch.bfloat16, "y")
    M, N = y.shape
    if r is None:
        r = B.shape[1]
    st = lib().lora_expand(_ptr(h), _ld(h, "h"), _ptr(B), _ld(B, "B"), _ptr(y), _ld(y, "y"), M, r, N, scale,
                           _stream(stream, y))
    _check(st, "lora_expand")
    return y


def lora_expand_compensated(h, B, y, scale: float, r: int | None = None, stream=None):
    """Like lora_expand, with h split into bf16 hi + bf16 lo (two matrix-core passes)."""
    import torch
    _dtype(h, torch.float32, "h"); _dtype(B, torch.bfloat16, "B"); _dtype(y, torch.bfloat16, "y")
    M, N = y.shape
    if r is None:
        r = B.shape[1]
    st = lib().lora_expand_compensated(_ptr(h), _ld(h, "h"), _ptr(B), _ld(B, "B"), _ptr(y), _ld(y, "y"), M, r, N,
                                       scale, _stream(stream, y))
    _check(st, "lora_expand_compensated")
    return y


def lora_shrink_expand_workspace_bytes(M: int, r: int, split_k: int) -> int:
    return int(lib().lora_shrink_expand_workspace_bytes(M, r, split_k))


def lora_shrink_expand(x, A, B, y, workspace, split_k: int = 8, shrink_scale: float = 1.0,
                       expand_scale: float = 1.0, h=None, stream=None):
    """Deterministic shrink then expand in two launches; y updated in place,
    h (optional, fp32 [M, >= r]) receives the shrink output."""
    import torch
    _dtype(x, torch.bfloat16, "x"); _dtype(A, torch.bfloat16, "A")
    _dtype(B, torch.bfloat16, "B"); _dtype(y, torch.bfloat16, "y")
    if h is not None:
        _dtype(h, torch.float32, "h")
    M, K = x.shape
    r = A.shape[0]
    N = y.shape[1]
    if y.shape[0] != M:
        raise ValueError("x and y must have the same number of rows")
    st = lib().lora_shrink_expand(_ptr(x), _ld(x, "x"), _ptr(A), _ld(A, "A"), _ptr(B), _ld(B, "B"), _ptr(h),
                                  _ld(h, "h") if h is not None else 0, _ptr(y), _ld(y, "y"), M, K, r, N, split_k,
                                  shrink_scale, expand_scale, _ptr(workspace), _nbytes(workspace),
                                  _stream(stream, x))
    _check(st, "lora_shrink_expand")
    return y


# LORA_NOALLOC_SCRATCH_BYTES of include/lora_det.h
NOALLOC_SCRATCH_BYTES = 8 << 20


def lora_shrink_expand_noalloc(x, A, B, y, split_k: int = 8, shrink_scale: float = 1.0, expand_scale: float = 1.0,
                               h=None, stream=None):
    """lora_shrink_expand with the library's fixed scratch buffer as the
    workspace (nothing allocated); split_k * M * r * 4 must not exceed
    NOALLOC_SCRATCH_BYTES.  Calls that may overlap on one device race on the
    buffer."""
    import torch
    _dtype(x, torch.bfloat16, "x"); _dtype(A, torch.bfloat16, "A")
    _dtype(B, torch.bfloat16, "B"); _dtype(y, torch.bfloat16, "y")
    if h is not None:
        _dtype(h, torch.float32, "h")
    M, K = x.shape
    r = A.shape[0]
    N = y.shape[1]
    if y.shape[0] != M:
        raise ValueError("x and y must have the same number of rows")
    st = lib().lora_shrink_expand_noalloc(_ptr(x), _ld(x, "x"), _ptr(A), _ld(A, "A"), _ptr(B), _ld(B, "B"),
                                          _ptr(h), _ld(h, "h") if h is not None else 0, _ptr(y), _ld(y, "y"), M, K,
                                          r, N, split_k, shrink_scale, expand_scale, _stream(stream, x))
    _check(st, "lora_shrink_expand_noalloc")
    return y


def lora_shrink_expand_counter_bytes(M: int) -> int:
    return int(lib().lora_shrink_expand_counter_bytes(M))


def lora_shrink_expand_counted(x, A, B, y, workspace, counters, split_k: int = 8, shrink_scale: float = 1.0,
                               expand_scale: float = 1.0, h=None, stream=None):
    """Deterministic shrink then expand in one launch; counters: zero-initialised
    int32 GPU tensor of lora_shrink_expand_counter_bytes(M) / 4 elements
    (element 0 is the status word, 0 after a complete call)."""
    import torch
    _dtype(x, torch.bfloat16, "x"); _dtype(A, torch.bfloat16, "A")
    _dtype(B, torch.bfloat16, "B"); _dtype(y, torch.bfloat16, "y")
    if h is not None:
        _dtype(h, torch.float32, "h")
    if counters is not None:
        _dtype(counters, torch.int32, "counters")
    M, K = x.shape
    r = A.shape[0]
    N = y.shape[1]
    if y.shape[0] != M:
        raise ValueError("x and y must have the same number of rows")
    st = lib().lora_shrink_expand_counted(_ptr(x), _ld(x, "x"), _ptr(A), _ld(A, "A"), _ptr(B), _ld(B, "B"),
                                          _ptr(h), _ld(h, "h") if h is not None else 0, _ptr(y), _ld(y, "y"), M, K,
                                          r, N, split_k, shrink_scale, expand_scale, _ptr(workspace),
                                          _nbytes(workspace), _ptr(counters), _nbytes(counters), _stream(stream, x))
    _check(st, "lora_shrink_expand_counted")
    return y


def lora_shrink_expand_launches(M: int, K: int, r: int, N: int, split_k: int) -> int:
    return int(lib().lora_shrink_expand_launches(M, K, r, N, split_k))


def lora_shrink_expand_fused(x, A, B, y, split_k: int = 8, shrink_scale: float = 1.0, expand_scale: float = 1.0,
                             h=None, stream=None):
    """Deterministic shrink then expand in one launch (no workspace); y in place."""
    import torch
    _dtype(x, torch.bfloat16, "x"); _dtype(A, torch.bfloat16, "A")
    _dtype(B, torch.bfloat16, "B"); _dtype(y, torch.bfloat16, "y")
    if h is not None:
        _dtype(h, torch.float32, "h")
    M, K = x.shape
    r = A.shape[0]
    N = y.shape[1]
    if y.shape[0] != M:
        raise ValueError("x and y must have the same number of rows")
    st = lib().lora_shrink_expand_fused(_ptr(x), _ld(x, "x"), _ptr(A), _ld(A, "A"), _ptr(B), _ld(B, "B"), _ptr(h),
                                        _ld(h, "h") if h is not None else 0, _ptr(y), _ld(y, "y"), M, K, r, N,
                                        split_k, shrink_scale, expand_scale, _stream(stream, x))
    _check(st, "lora_shrink_expand_fused")
    return y


def lora_shrink_partials(x, A, workspace, split_k: int = 8, stream=None):
    """workspace[s][i][j] = split s's fp32 partial of x @ A^T (one launch)."""
    import torch
    _dtype(x, torch.bfloat16, "x"); _dtype(A, torch.bfloat16, "A")
    M, K = x.shape
    r = A.shape[0]
    st = lib().lora_shrink_partials(_ptr(x), _ld(x, "x"), _ptr(A), _ld(A, "A"), M, K, r, split_k,
                                    _ptr(workspace), _nbytes(workspace), _stream(stream, x))
    _check(st, "lora_shrink_partials")
    return workspace


def lora_expand_combine(workspace, B, y, split_k: int = 8, shrink_scale: float = 1.0, expand_scale: float = 1.0,
                        h=None, r: int | None = None, stream=None):
    """Fixed-tree combine of the workspace, then the expand into y (one launch)."""
    import torch
    _dtype(B, torch.bfloat16, "B"); _dtype(y, torch.bfloat16, "y")
    if h is not None:
        _dtype(h, torch.float32, "h")
    M, N = y.shape
    if r is None:
        r = B.shape[1]
    st = lib().lora_expand_combine(_ptr(workspace), _nbytes(workspace), split_k, shrink_scale, _ptr(B), _ld(B, "B"),
                                   _ptr(h), _ld(h, "h") if h is not None else 0, _ptr(y), _ld(y, "y"), M, r, N,
                                   expand_scale, _stream(stream, y))
    _check(st, "lora_expand_combine")
    return y


def lora_sgmv_plan(token_adapter, n_adapters: int, plan, stream=None):
    import torch
    _dtype(token_adapter, torch.int32, "token_adapter")
    M = token_adapter.numel()
    st = lib().lora_sgmv_plan(_ptr(token_adapter), M, n_adapters, _ptr(plan), _nbytes(plan),
                              _stream(stream, token_adapter))
    _check(st, "lora_sgmv_plan")
    return plan


def lora_sgmv_shrink(x, A_ptrs, ld_a: int, ranks, scales, token_adapter, n_adapters: int, plan, h,
                     r_max: int, split_k: int, workspace, stream=None):
    """A_ptrs: int64 GPU tensor of adapter weight addresses ([r_a][ld_a] bf16 each)."""
    import torch
    _dtype(x, torch.bfloat16, "x"); _dtype(h, torch.float32, "h")
    _dtype(A_ptrs, torch.int64, "A_ptrs"); _dtype(ranks, torch.int32, "ranks")
    _dtype(token_adapter, torch.int32, "token_adapter")
    if scales is not None:
        _dtype(scales, torch.float32, "scales")
    M, K = x.shape
    st = lib().lora_sgmv_shrink(_ptr(x), _ld(x, "x"), _ptr(A_ptrs), ld_a, _ptr(ranks), _ptr(scales),
                                _ptr(token_adapter), n_adapters, _ptr(plan), _nbytes(plan), _ptr(h), _ld(h, "h"),
                                M, K, r_max, split_k, _ptr(workspace), _nbytes(workspace), _stream(stream, x))
    _check(st, "lora_sgmv_shrink")
    return h


def lora_sgmv_shrink_counted(x, A_ptrs, ld_a: int, ranks, scales, n_adapters: int, plan, h, r_max: int,
                             split_k: int, workspace, counters, stream=None):
    import torch
    _dtype(x, torch.bfloat16, "x"); _dtype(h, torch.float32, "h")
    _dtype(A_ptrs, torch.int64, "A_ptrs"); _dtype(ranks, torch.int32, "ranks")
    _dtype(counters, torch.int32, "counters")
    if scales is not None:
        _dtype(scales, torch.float32, "scales")
    M, K = x.shape
    st = lib().lora_sgmv_shrink_counted(_ptr(x), _ld(x, "x"), _ptr(A_ptrs), ld_a, _ptr(ranks), _ptr(scales),
                                        n_adapters, _ptr(plan), _nbytes(plan), _ptr(h), _ld(h, "h"), M, K, r_max,
                                        split_k, _ptr(workspace), _nbytes(workspace), _ptr(counters),
                                        _nbytes(counters), _stream(stream, x))
    _check(st, "lora_sgmv_shrink_counted")
    return h


def lora_sgmv_shrink_atomic(x, A_ptrs, ld_a: int, ranks, scales, n_adapters: int, plan, h, r_max: int,
                            split_k: int, stream=None):
    """The nondeterministic contrast: zero h, then the multi-adapter partial
    kernel adds every split's scaled partial into h with fp32 atomics."""
    import torch
    _dtype(x, torch.bfloat16, "x"); _dtype(h, torch.float32, "h")
    _dtype(A_ptrs, torch.int64, "A_ptrs"); _dtype(ranks, torch.int32, "ranks")
    if scales is not None:
        _dtype(scales, torch.float32, "scales")
    M, K = x.shape
    st = lib().lora_sgmv_shrink_atomic(_ptr(x), _ld(x, "x"), _ptr(A_ptrs), ld_a, _ptr(ranks), _ptr(scales),
                                       n_adapters, _ptr(plan), _nbytes(plan), _ptr(h), _ld(h, "h"), M, K, r_max,
                                       split_k, _stream(stream, x))
    _check(st, "lora_sgmv_shrink_atomic")
    return h


def lora_sgmv_shrink_expand(x, A_ptrs, ld_a: int, B_ptrs, ranks, shrink_scales, expand_scales, token_adapter,
                            n_adapters: int, plan, y, r_max: int, split_k: int, workspace, h=None, stream=None):
    """Multi-adapter shrink + expand in two launches (expand reads the Split-K
    workspace); y updated in place, h (optional) receives the shrink output."""
    import torch
    _dtype(x, torch.bfloat16, "x"); _dtype(y, torch.bfloat16, "y"); _dtype(token_adapter, torch.int32, "ids")
    if h is not None:
        _dtype(h, torch.float32, "h")
    M, K = x.shape
    N = y.shape[1]
    if y.shape[0] != M:
        raise ValueError("x and y must have the same number of rows")
    st = lib().lora_sgmv_shrink_expand(_ptr(x), _ld(x, "x"), _ptr(A_ptrs), ld_a, _ptr(B_ptrs), _ptr(ranks),
                                       _ptr(shrink_scales), _ptr(expand_scales), _ptr(token_adapter), n_adapters,
                                       _ptr(plan), _nbytes(plan), _ptr(h), _ld(h, "h") if h is not None else 0,
                                       _ptr(y), _ld(y, "y"), M, K, N, r_max, split_k, _ptr(workspace),
                                       _nbytes(workspace), _stream(stream, x))
    _check(st, "lora_sgmv_shrink_expand")
    return y


def lora_sgmv_expand(h, B_ptrs, ranks, scales, token_adapter, n_adapters: int, y, r_max: int, stream=None):
    """Multi-adapter expand, y updated in place for tokens with an adapter."""
    import torch
    _dtype(h, torch.float32, "h"); _dtype(y, torch.bfloat16, "y"); _dtype(token_adapter, torch.int32, "ids")
    M, N = y.shape
    st = lib().lora_sgmv_expand(_ptr(h), _ld(h, "h"), _ptr(B_ptrs), _ptr(ranks), _ptr(scales), _ptr(token_adapter),
                                n_adapters, _ptr(y), _ld(y, "y"), M, N, r_max, _stream(stream, y))
    _check(st, "lora_sgmv_expand")
    return y

"""Python binding of libmmrelu, the gfx950 library computing C = relu(A·B)
(and its fused-epilogue widening C = act(A·B + bias)).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libmmrelu.so`` (built from ``csrc/`` by ``build.py``). The C
entry points (``include/mmrelu.h``) are exposed under the same names and take
raw device pointers, sizes, leading dimensions (elements) and a HIP stream
handle. ``mmrelu(a, b, out=None)`` is a convenience wrapper for torch device
tensors (row-major, unit column stride) that launches on torch's current
stream; torch only provides device memory and streams.

There is no fallback: if the library is missing or cannot be loaded, every
call raises.
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmmrelu.so")

MMRELU_OK = 0
MMRELU_ERR_INVALID_VALUE = 1
MMRELU_ERR_NULL_POINTER = 2
MMRELU_ERR_MISALIGNED = 3
MMRELU_ERR_LAUNCH = 4
MMRELU_ERR_WORKSPACE_LIMIT = 5
STATIC_WORKSPACE_BYTES = 64 << 20
DTYPE_F32 = 0
DTYPE_BF16 = 1
ACT_RELU = 0
ACT_GELU_TANH = 1
ACT_NONE = 2
_ACTS = {"relu": ACT_RELU, "gelu_tanh": ACT_GELU_TANH, "none": ACT_NONE}

EXPORTED = (
    "mmrelu_f32", "mmrelu_bf16", "mmrelu_status_string", "mmrelu_version",
    "mmrelu_plan", "mmrelu_num_variants", "mmrelu_plan_variant",
    "mmrelu_wave_quantization", "mmrelu_f32_variant", "mmrelu_bf16_variant",
    "mmrelu_fused_f32", "mmrelu_fused_bf16", "mmrelu_fused_f32_variant", "mmrelu_fused_bf16_variant",
    "mmrelu_strided_workspace_size", "mmrelu_strided_f32", "mmrelu_strided_bf16", "mmrelu_strided_static",
    "mmrelu_softmax_rows_f32", "mmrelu_softmax_rows_bf16", "mmrelu_softmax_rows_f32_variant",
    "mmrelu_softmax_rows_bf16_variant", "mmrelu_softmax_rows_variant", "mmrelu_row_sum_f32", "mmrelu_row_sum_bf16",
)


class MmreluError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


class Plan(ctypes.Structure):
    _fields_ = [
        ("variant", ctypes.c_int32), ("block_m", ctypes.c_int32), ("block_n", ctypes.c_int32),
        ("block_k", ctypes.c_int32), ("threads", ctypes.c_int32), ("wg_per_cu", ctypes.c_int32),
        ("cus", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64), ("grid", ctypes.c_int64),
        ("waves", ctypes.c_int64), ("idle_slots_last", ctypes.c_int64), ("name", ctypes.c_char * 64),
    ]

    def as_dict(self) -> dict:
        d = {f: getattr(self, f) for f, _ in self._fields_ if f != "reserved"}
        d["name"] = self.name.decode()
        return d


_lib = None


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libmmrelu.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m tiled_matmul_relu_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    for name in ("mmrelu_f32", "mmrelu_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
        fn.restype = ctypes.c_int
    for name in ("mmrelu_f32_variant", "mmrelu_bf16_variant"):
        fn = getattr(lib, name)
        fn.argtypes = [i32, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
        fn.restype = ctypes.c_int
    for name in ("mmrelu_fused_f32", "mmrelu_fused_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
        fn.restype = ctypes.c_int
    for name in ("mmrelu_fused_f32_variant", "mmrelu_fused_bf16_variant"):
        fn = getattr(lib, name)
        fn.argtypes = [i32, ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
        fn.restype = ctypes.c_int
    for name in ("mmrelu_strided_f32", "mmrelu_strided_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i64, i64, i64, vp,
                       ctypes.c_size_t, vp]
        fn.restype = ctypes.c_int
    lib.mmrelu_strided_static.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                          i64, i64, i64, vp]
    lib.mmrelu_strided_static.restype = ctypes.c_int
    lib.mmrelu_strided_workspace_size.argtypes = [ctypes.c_int, ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i64,
                                                  i64, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.mmrelu_strided_workspace_size.restype = ctypes.c_int
    for name in ("mmrelu_softmax_rows_f32", "mmrelu_softmax_rows_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, i64, i64, i64, i64, vp]
        fn.restype = ctypes.c_int
    for name in ("mmrelu_softmax_rows_f32_variant", "mmrelu_softmax_rows_bf16_variant"):
        fn = getattr(lib, name)
        fn.argtypes = [i32, vp, vp, i64, i64, i64, i64, vp]
        fn.restype = ctypes.c_int
    lib.mmrelu_softmax_rows_variant.argtypes = [ctypes.c_int, i64, i64, i64, ctypes.POINTER(i32)]
    lib.mmrelu_softmax_rows_variant.restype = ctypes.c_int
    for name in ("mmrelu_row_sum_f32", "mmrelu_row_sum_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [vp, vp, i64, i64, i64, vp]
        fn.restype = ctypes.c_int
    lib.mmrelu_status_string.argtypes = [ctypes.c_int]
    lib.mmrelu_status_string.restype = ctypes.c_char_p
    lib.mmrelu_version.restype = ctypes.c_char_p
    lib.mmrelu_plan.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64, i32, ctypes.POINTER(Plan)]
    lib.mmrelu_plan.restype = ctypes.c_int
    lib.mmrelu_plan_variant.argtypes = [ctypes.c_int, i32, i64, i64, i64, i64, i64, i64, i32, ctypes.POINTER(Plan)]
    lib.mmrelu_plan_variant.restype = ctypes.c_int
    lib.mmrelu_num_variants.argtypes = [ctypes.c_int]
    lib.mmrelu_num_variants.restype = ctypes.c_int
    lib.mmrelu_wave_quantization.argtypes = [i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.mmrelu_wave_quantization.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().mmrelu_status_string(status).decode()


def version() -> str:
    return load_library().mmrelu_version().decode()


def _check(status: int, where: str) -> None:
    if status != MMRELU_OK:
        raise MmreluError(status, where)


# --- C entry points with the same names (raw pointers) -----------------------

def mmrelu_f32(A: int, B: int, C: int, M: int, N: int, K: int, lda: int, ldb: int, ldc: int,
               stream: int = 0) -> int:
    """Enqueue C = relu(A·B), fp32. Pointers are device addresses; returns the status."""
    return load_library().mmrelu_f32(A, B, C, M, N, K, lda, ldb, ldc, stream)


def mmrelu_bf16(A: int, B: int, C: int, M: int, N: int, K: int, lda: int, ldb: int, ldc: int,
                stream: int = 0) -> int:
    """Enqueue C = relu(A·B), bf16 in/out, fp32 accumulation; returns the status."""
    return load_library().mmrelu_bf16(A, B, C, M, N, K, lda, ldb, ldc, stream)


def mmrelu_f32_variant(variant: int, A: int, B: int, C: int, M: int, N: int, K: int, lda: int, ldb: int,
                       ldc: int, stream: int = 0) -> int:
    return load_library().mmrelu_f32_variant(variant, A, B, C, M, N, K, lda, ldb, ldc, stream)


def mmrelu_bf16_variant(variant: int, A: int, B: int, C: int, M: int, N: int, K: int, lda: int, ldb: int,
                        ldc: int, stream: int = 0) -> int:
    return load_library().mmrelu_bf16_variant(variant, A, B, C, M, N, K, lda, ldb, ldc, stream)


def mmrelu_fused_f32(act: int, A: int, B: int, bias: int, C: int, M: int, N: int, K: int, lda: int, ldb: int,
                     ldc: int, stream: int = 0) -> int:
    """Enqueue C = act(A·B + bias), fp32 (bias: device address of N floats, or 0 for none)."""
    return load_library().mmrelu_fused_f32(act, A, B, bias or None, C, M, N, K, lda, ldb, ldc, stream)


def mmrelu_fused_bf16(act: int, A: int, B: int, bias: int, C: int, M: int, N: int, K: int, lda: int, ldb: int,
                      ldc: int, stream: int = 0) -> int:
    """Enqueue C = act(A·B + bias), bf16 in/out (bias: N bf16 values, or 0), fp32 accumulation."""
    return load_library().mmrelu_fused_bf16(act, A, B, bias or None, C, M, N, K, lda, ldb, ldc, stream)


def mmrelu_fused_f32_variant(variant: int, act: int, A: int, B: int, bias: int, C: int, M: int, N: int, K: int,
                             lda: int, ldb: int, ldc: int, stream: int = 0) -> int:
    return load_library().mmrelu_fused_f32_variant(variant, act, A, B, bias or None, C, M, N, K, lda, ldb, ldc,
                                                   stream)


def mmrelu_fused_bf16_variant(variant: int, act: int, A: int, B: int, bias: int, C: int, M: int, N: int, K: int,
                              lda: int, ldb: int, ldc: int, stream: int = 0) -> int:
    return load_library().mmrelu_fused_bf16_variant(variant, act, A, B, bias or None, C, M, N, K, lda, ldb, ldc,
                                                    stream)


def mmrelu_strided_workspace_size(dtype: int, act: int, A: int, B: int, bias: int, C: int, M: int, N: int, K: int,
                                  sam: int, sak: int, sbk: int, sbn: int, scm: int, scn: int) -> int:
    """Workspace bytes a general-stride call with these arguments needs (raises on invalid arguments)."""
    n = ctypes.c_size_t()
    _check(load_library().mmrelu_strided_workspace_size(dtype, act, A or None, B or None, bias or None, C or None,
                                                        M, N, K, sam, sak, sbk, sbn, scm, scn, ctypes.byref(n)),
           "mmrelu_strided_workspace_size")
    return n.value


def mmrelu_strided_f32(act: int, A: int, B: int, bias: int, C: int, M: int, N: int, K: int, sam: int, sak: int,
                       sbk: int, sbn: int, scm: int, scn: int, workspace: int, workspace_bytes: int,
                       stream: int = 0) -> int:
    """Enqueue C = act(A·B + bias), fp32, with an element stride per dimension of A, B and C."""
    return load_library().mmrelu_strided_f32(act, A, B, bias or None, C, M, N, K, sam, sak, sbk, sbn, scm, scn,
                                             workspace or None, workspace_bytes, stream)


def mmrelu_strided_bf16(act: int, A: int, B: int, bias: int, C: int, M: int, N: int, K: int, sam: int, sak: int,
                        sbk: int, sbn: int, scm: int, scn: int, workspace: int, workspace_bytes: int,
                        stream: int = 0) -> int:
    """Enqueue C = act(A·B + bias), bf16 in/out, with an element stride per dimension of A, B and C."""
    return load_library().mmrelu_strided_bf16(act, A, B, bias or None, C, M, N, K, sam, sak, sbk, sbn, scm, scn,
                                              workspace or None, workspace_bytes, stream)


def mmrelu_strided_static(dtype: int, act: int, A: int, B: int, bias: int, C: int, M: int, N: int, K: int,
                          sam: int, sak: int, sbk: int, sbn: int, scm: int, scn: int, stream: int = 0) -> int:
    """Enqueue the general-stride call of `dtype` with its workspace taken
    from the library's fixed device array (no allocation); returns the
    status (MMRELU_ERR_WORKSPACE_LIMIT past STATIC_WORKSPACE_BYTES)."""
    return load_library().mmrelu_strided_static(dtype, act, A, B, bias or None, C, M, N, K, sam, sak, sbk, sbn,
                                                scm, scn, stream)


def mmrelu_softmax_rows_f32(X: int, Y: int, M: int, N: int, ldx: int, ldy: int, stream: int = 0) -> int:
    """Enqueue the row softmax of an fp32 M x N matrix; returns the status."""
    return load_library().mmrelu_softmax_rows_f32(X or None, Y or None, M, N, ldx, ldy, stream)


def mmrelu_softmax_rows_bf16(X: int, Y: int, M: int, N: int, ldx: int, ldy: int, stream: int = 0) -> int:
    """Enqueue the row softmax of a bf16 M x N matrix (fp32 inside); returns the status."""
    return load_library().mmrelu_softmax_rows_bf16(X or None, Y or None, M, N, ldx, ldy, stream)


def mmrelu_softmax_rows_f32_variant(variant: int, X: int, Y: int, M: int, N: int, ldx: int, ldy: int,
                                    stream: int = 0) -> int:
    return load_library().mmrelu_softmax_rows_f32_variant(variant, X or None, Y or None, M, N, ldx, ldy, stream)


def mmrelu_softmax_rows_bf16_variant(variant: int, X: int, Y: int, M: int, N: int, ldx: int, ldy: int,
                                     stream: int = 0) -> int:
    return load_library().mmrelu_softmax_rows_bf16_variant(variant, X or None, Y or None, M, N, ldx, ldy, stream)


def mmrelu_softmax_rows_variant(dtype: int, N: int, ldx: int, ldy: int) -> int:
    """The softmax kernel a call of this shape uses (16-byte aligned pointers)."""
    v = ctypes.c_int32()
    _check(load_library().mmrelu_softmax_rows_variant(dtype, N, ldx, ldy, ctypes.byref(v)),
           "mmrelu_softmax_rows_variant")
    return v.value


def mmrelu_row_sum_f32(X: int, out: int, M: int, N: int, ldx: int, stream: int = 0) -> int:
    """Enqueue out[i] = sum_j X[i][j] for an fp32 matrix (fp32 out); returns the status."""
    return load_library().mmrelu_row_sum_f32(X or None, out or None, M, N, ldx, stream)


def mmrelu_row_sum_bf16(X: int, out: int, M: int, N: int, ldx: int, stream: int = 0) -> int:
    """Enqueue out[i] = sum_j X[i][j] for a bf16 matrix (fp32 out); returns the status."""
    return load_library().mmrelu_row_sum_bf16(X or None, out or None, M, N, ldx, stream)


def mmrelu_plan(dtype: int, M: int, N: int, K: int, lda: int, ldb: int, ldc: int, cus: int = 0) -> dict:
    p = Plan()
    _check(load_library().mmrelu_plan(dtype, M, N, K, lda, ldb, ldc, cus, ctypes.byref(p)), "mmrelu_plan")
    return p.as_dict()


def mmrelu_plan_variant(dtype: int, variant: int, M: int, N: int, K: int, lda: int, ldb: int, ldc: int,
                        cus: int = 0) -> dict:
    p = Plan()
    _check(load_library().mmrelu_plan_variant(dtype, variant, M, N, K, lda, ldb, ldc, cus, ctypes.byref(p)),
           "mmrelu_plan_variant")
    return p.as_dict()


def mmrelu_num_variants(dtype: int) -> int:
    return load_library().mmrelu_num_variants(dtype)


def mmrelu_wave_quantization(blocks: int, slots: int) -> tuple[int, int]:
    w, idle = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().mmrelu_wave_quantization(blocks, slots, ctypes.byref(w), ctypes.byref(idle)),
           "mmrelu_wave_quantization")
    return w.value, idle.value


# --- torch convenience wrapper ----------------------------------------------

def _row_major(t) -> bool:
    """2-D with unit column stride and rows that do not overlap; a single
    column's stride is never used, so any value is accepted for it."""
    return t.dim() == 2 and (t.stride(1) == 1 or t.shape[1] <= 1) and t.stride(0) >= max(t.shape[1], 1)


def _ld(t) -> int:
    """Leading dimension (elements) of a tensor that _row_major accepts."""
    if not _row_major(t):
        raise ValueError("matrices must be 2-D, row-major with unit column stride")
    return max(t.stride(0), t.shape[1], 1)


def mmrelu(a, b, out=None, variant: int | None = None, stream=None, bias=None, act: str = "relu"):
    """act(a @ b + bias) for torch device tensors (float32 or bfloat16); the
    default is relu(a @ b).

    ``bias`` is an optional contiguous (N,) tensor of the same dtype and
    ``act`` one of "relu", "gelu_tanh", "none". ``out`` may be a preallocated
    (M, N) tensor. Row-major operands (unit column stride) go to the
    row-major entry points; any other strides (transposed or sliced views)
    go to the general-stride entry points with a workspace allocated here.
    Launches on ``stream`` (default: torch's current stream) and returns
    ``out`` without synchronising."""
    import torch
    if a.dtype != b.dtype or a.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("a and b must both be float32 or both bfloat16")
    if not (a.is_cuda and b.is_cuda):
        raise ValueError("a and b must be device tensors")
    M, K = a.shape
    K2, N = b.shape
    if K != K2:
        raise ValueError(f"inner dimensions differ: {K} vs {K2}")
    if out is None:
        out = torch.empty((M, N), dtype=a.dtype, device=a.device)
    elif out.shape != (M, N) or out.dtype != a.dtype or out.device != a.device:
        raise ValueError("out has the wrong shape, dtype or device")
    if act not in _ACTS:
        raise ValueError(f"act must be one of {sorted(_ACTS)}")
    if bias is not None and (bias.dtype != a.dtype or bias.device != a.device or bias.shape != (N,)
                             or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous (N,) tensor of the inputs' dtype and device")
    s = stream if stream is not None else torch.cuda.current_stream(a.device)
    if not (_row_major(a) and _row_major(b) and _row_major(out)):
        if variant is not None:
            raise ValueError("an explicit variant needs row-major a, b and out")
        kind = DTYPE_F32 if a.dtype == torch.float32 else DTYPE_BF16
        bp = bias.data_ptr() if bias is not None else 0
        strides = (a.stride(0), a.stride(1), b.stride(0), b.stride(1), out.stride(0), out.stride(1))
        need = mmrelu_strided_workspace_size(kind, _ACTS[act], a.data_ptr(), b.data_ptr(), bp, out.data_ptr(),
                                             M, N, K, *strides)
        ws = torch.empty(need + 256, dtype=torch.uint8, device=a.device) if need else None
        wp = 0
        if ws is not None:
            wp = (ws.data_ptr() + 255) // 256 * 256
            ws.record_stream(s)
        fn = mmrelu_strided_f32 if kind == DTYPE_F32 else mmrelu_strided_bf16
        _check(fn(_ACTS[act], a.data_ptr(), b.data_ptr(), bp, out.data_ptr(), M, N, K, *strides, wp, need,
                  s.cuda_stream), "mmrelu (strided)")
        return out
    args = (a.data_ptr(), b.data_ptr(), bias.data_ptr() if bias is not None else 0, out.data_ptr(), M, N, K,
            _ld(a), _ld(b), _ld(out), s.cuda_stream)
    if a.dtype == torch.float32:
        rc = (mmrelu_fused_f32(_ACTS[act], *args) if variant is None
              else mmrelu_fused_f32_variant(variant, _ACTS[act], *args))
    else:
        rc = (mmrelu_fused_bf16(_ACTS[act], *args) if variant is None
              else mmrelu_fused_bf16_variant(variant, _ACTS[act], *args))
    _check(rc, "mmrelu")
    return out


def softmax_rows(x, out=None, stream=None):
    """Row softmax of a 2-D float32 or bfloat16 device tensor (unit column
    stride); ``out`` may be ``x`` itself. Returns ``out`` without
    synchronising."""
    import torch
    if x.dim() != 2 or x.dtype not in (torch.float32, torch.bfloat16) or not x.is_cuda:
        raise ValueError("x must be a 2-D float32 or bfloat16 device tensor")
    M, N = x.shape
    out = torch.empty_like(x) if out is None else out
    if out.shape != x.shape or out.dtype != x.dtype:
        raise ValueError("out has the wrong shape or dtype")
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    fn = mmrelu_softmax_rows_f32 if x.dtype == torch.float32 else mmrelu_softmax_rows_bf16
    _check(fn(x.data_ptr(), out.data_ptr(), M, N, _ld(x), _ld(out), s.cuda_stream), "softmax_rows")
    return out


def row_sum(x, out=None, stream=None):
    """Sum of each row of a 2-D float32 or bfloat16 device tensor (unit
    column stride), as an (M,) float32 tensor. Returns without synchronising."""
    import torch
    if x.dim() != 2 or x.dtype not in (torch.float32, torch.bfloat16) or not x.is_cuda:
        raise ValueError("x must be a 2-D float32 or bfloat16 device tensor")
    M, N = x.shape
    out = torch.empty(M, dtype=torch.float32, device=x.device) if out is None else out
    if out.shape != (M,) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be a contiguous (M,) float32 tensor")
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    fn = mmrelu_row_sum_f32 if x.dtype == torch.float32 else mmrelu_row_sum_bf16
    _check(fn(x.data_ptr(), out.data_ptr(), M, N, _ld(x), s.cuda_stream), "row_sum")
    return out

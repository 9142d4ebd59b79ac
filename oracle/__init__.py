"""fp64 CPU oracle for C = relu(A·B): TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The gfx950 library never calls it and
shares no code with it; this package does not import the library either.

The arithmetic lives in ``mmrelu_oracle.c`` (plain C, OpenMP over rows),
built with gcc into ``liboracle.so`` next to it. Each routine is the plain
definition R[i][j] = max(0, sum_k A[i][k]·B[k][j]) in fp64 with ascending k,
its fused-epilogue form R[i][j] = act(sum_k A[i][k]·B[k][j] + bias[j])
with act one of ReLU, GeLU (tanh form) or none, and its general-stride form
(A[i][k] = a[i*sam + k*sak], B[k][j] = b[k*sbk + j*sbn]). It also holds the
two rungs before the matmul on the lecture's ladder: the row softmax and the
row sum. See the C file for the passages each follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "mmrelu_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile liboracle.so with gcc (no fast-math: IEEE double semantics)."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
           "-fno-fast-math", "-ffp-contract=off", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        build()
    lib = ctypes.CDLL(LIB)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    for name in ("oracle_mmrelu_f32", "oracle_mmrelu_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64]
        fn.restype = ctypes.c_int
    for name in ("oracle_mmrelu_f32_at", "oracle_mmrelu_bf16_at"):
        fn = getattr(lib, name)
        fn.argtypes = [p, p, i64, i64, i64, p, p, i64, p]
        fn.restype = None
    for name in ("oracle_fused_f32", "oracle_fused_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.c_int, p, p, p, p, i64, i64, i64, i64, i64, i64]
        fn.restype = ctypes.c_int
    for name in ("oracle_fused_f32_at", "oracle_fused_bf16_at"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.c_int, p, p, p, i64, i64, i64, p, p, i64, p]
        fn.restype = None
    for name in ("oracle_strided_f32", "oracle_strided_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.c_int, p, p, p, p, i64, i64, i64, i64, i64, i64, i64, i64]
        fn.restype = ctypes.c_int
    for name in ("oracle_strided_f32_at", "oracle_strided_bf16_at"):
        fn = getattr(lib, name)
        fn.argtypes = [ctypes.c_int, p, p, p, i64, i64, i64, i64, i64, p, p, i64, p]
        fn.restype = None
    for name in ("oracle_softmax_rows_f32", "oracle_softmax_rows_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [p, p, i64, i64, i64]
        fn.restype = ctypes.c_int
    for name in ("oracle_row_sum_f32", "oracle_row_sum_bf16"):
        fn = getattr(lib, name)
        fn.argtypes = [p, p, i64, i64, i64]
        fn.restype = None
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    return _load().oracle_num_threads()


def _check(a: np.ndarray, b: np.ndarray, M, N, K, lda, ldb, dtype):
    if a.dtype != dtype or b.dtype != dtype:
        raise TypeError(f"oracle inputs must be {dtype}")
    if not (a.flags.c_contiguous and b.flags.c_contiguous):
        raise ValueError("oracle inputs must be C-contiguous buffers")
    if min(M, N, K) < 0 or lda < max(1, K) or ldb < max(1, N):
        raise ValueError("bad sizes or leading dimensions")
    if M > 0 and K > 0 and a.size < (M - 1) * lda + K:
        raise ValueError("A buffer too small")
    if K > 0 and N > 0 and b.size < (K - 1) * ldb + N:
        raise ValueError("B buffer too small")


def _dtype_and_fns(a: np.ndarray):
    if a.dtype == np.float32:
        return np.float32, "oracle_mmrelu_f32", "oracle_mmrelu_f32_at"
    if a.dtype == np.uint16:
        return np.uint16, "oracle_mmrelu_bf16", "oracle_mmrelu_bf16_at"
    raise TypeError("oracle inputs are float32 or uint16 (bf16 bit patterns)")


def mmrelu(a: np.ndarray, b: np.ndarray, M=None, N=None, K=None, lda=None, ldb=None) -> np.ndarray:
    """relu(A·B) as an M x N float64 array. ``a``/``b`` are float32 (fp32) or
    uint16 (bf16 bit patterns) row-major buffers with leading dimensions lda/ldb
    (defaults: the arrays' 2-D shapes)."""
    dtype, full, _ = _dtype_and_fns(a)
    if M is None:
        M, lda = a.shape[0], a.shape[1]
        K = K if K is not None else a.shape[1]
        ldb = b.shape[1]
        N = N if N is not None else b.shape[1]
    lda = lda if lda is not None else K
    ldb = ldb if ldb is not None else N
    _check(a, b, M, N, K, lda, ldb, dtype)
    r = np.empty((M, N), dtype=np.float64)
    if M == 0 or N == 0:
        return r
    rc = getattr(_load(), full)(a.ctypes.data, b.ctypes.data, r.ctypes.data, M, N, K, lda, ldb, N)
    if rc != 0:
        raise MemoryError("oracle could not allocate its row accumulator")
    return r


def mmrelu_at(a: np.ndarray, b: np.ndarray, rows, cols, K: int, lda: int, ldb: int) -> np.ndarray:
    """relu(A·B)[rows[t], cols[t]] for each t, as float64 (one dot product each)."""
    dtype, _, at = _dtype_and_fns(a)
    ii = np.ascontiguousarray(rows, dtype=np.int64)
    jj = np.ascontiguousarray(cols, dtype=np.int64)
    if ii.shape != jj.shape:
        raise ValueError("rows and cols differ in length")
    if ii.size and (ii.min() < 0 or jj.min() < 0):
        raise ValueError("negative index")
    if ii.size and K > 0:
        if a.size < ii.max() * lda + K or b.size < (K - 1) * ldb + jj.max() + 1:
            raise ValueError("index beyond the buffers")
    out = np.empty(ii.size, dtype=np.float64)
    if ii.size:
        getattr(_load(), at)(a.ctypes.data, b.ctypes.data, K, lda, ldb,
                             ii.ctypes.data, jj.ctypes.data, ii.size, out.ctypes.data)
    return out


ACTS = {"relu": 0, "gelu_tanh": 1, "none": 2}


def _bias_ptr(bias, dtype, N):
    if bias is None:
        return None
    if bias.dtype != dtype or not bias.flags.c_contiguous or bias.size < N:
        raise ValueError("bias must be a C-contiguous array of N elements of the inputs' dtype")
    return bias.ctypes.data


def fused(act: str, a: np.ndarray, b: np.ndarray, bias=None, M=None, N=None, K=None, lda=None,
          ldb=None) -> np.ndarray:
    """act(A·B + bias) as an M x N float64 array; ``act`` in ACTS, ``bias``
    None or N values of the inputs' dtype (float32 or uint16 bf16 patterns)."""
    dtype, _, _ = _dtype_and_fns(a)
    if M is None:
        M, lda = a.shape[0], a.shape[1]
        K = K if K is not None else a.shape[1]
        ldb = b.shape[1]
        N = N if N is not None else b.shape[1]
    lda = lda if lda is not None else K
    ldb = ldb if ldb is not None else N
    _check(a, b, M, N, K, lda, ldb, dtype)
    bp = _bias_ptr(bias, dtype, N)
    r = np.empty((M, N), dtype=np.float64)
    if M == 0 or N == 0:
        return r
    fn = "oracle_fused_f32" if dtype == np.float32 else "oracle_fused_bf16"
    rc = getattr(_load(), fn)(ACTS[act], a.ctypes.data, b.ctypes.data, bp, r.ctypes.data, M, N, K, lda, ldb, N)
    if rc != 0:
        raise MemoryError("oracle could not allocate its row accumulator")
    return r


def fused_at(act: str, a: np.ndarray, b: np.ndarray, bias, rows, cols, K: int, lda: int, ldb: int) -> np.ndarray:
    """act(A·B + bias)[rows[t], cols[t]] for each t, as float64."""
    dtype, _, _ = _dtype_and_fns(a)
    ii = np.ascontiguousarray(rows, dtype=np.int64)
    jj = np.ascontiguousarray(cols, dtype=np.int64)
    if ii.shape != jj.shape:
        raise ValueError("rows and cols differ in length")
    if ii.size and (ii.min() < 0 or jj.min() < 0):
        raise ValueError("negative index")
    if ii.size and K > 0:
        if a.size < ii.max() * lda + K or b.size < (K - 1) * ldb + jj.max() + 1:
            raise ValueError("index beyond the buffers")
    bp = _bias_ptr(bias, dtype, int(jj.max()) + 1 if jj.size else 0)
    out = np.empty(ii.size, dtype=np.float64)
    if ii.size:
        fn = "oracle_fused_f32_at" if dtype == np.float32 else "oracle_fused_bf16_at"
        getattr(_load(), fn)(ACTS[act], a.ctypes.data, b.ctypes.data, bp, K, lda, ldb,
                             ii.ctypes.data, jj.ctypes.data, ii.size, out.ctypes.data)
    return out


def _check_strided(a, b, M, N, K, sam, sak, sbk, sbn):
    dtype, _, _ = _dtype_and_fns(a)
    if b.dtype != dtype:
        raise TypeError("a and b differ in dtype")
    if not (a.flags.c_contiguous and b.flags.c_contiguous):
        raise ValueError("oracle inputs must be C-contiguous buffers")
    if min(M, N, K) < 0 or min(sam, sak, sbk, sbn) < 0:
        raise ValueError("negative size or stride")
    if M > 0 and K > 0 and a.size <= (M - 1) * sam + (K - 1) * sak:
        raise ValueError("A buffer too small for its strides")
    if K > 0 and N > 0 and b.size <= (K - 1) * sbk + (N - 1) * sbn:
        raise ValueError("B buffer too small for its strides")
    return dtype


def strided(act: str, a: np.ndarray, b: np.ndarray, bias, M: int, N: int, K: int,
            sam: int, sak: int, sbk: int, sbn: int) -> np.ndarray:
    """act(A·B + bias) as an M x N float64 array, with A[i][k] = a.flat[i*sam +
    k*sak] and B[k][j] = b.flat[k*sbk + j*sbn] (non-negative strides, in
    elements); ``a``/``b`` are C-contiguous float32 or uint16 (bf16) buffers."""
    dtype = _check_strided(a, b, M, N, K, sam, sak, sbk, sbn)
    bp = _bias_ptr(bias, dtype, N)
    r = np.empty((M, N), dtype=np.float64)
    if M == 0 or N == 0:
        return r
    fn = "oracle_strided_f32" if dtype == np.float32 else "oracle_strided_bf16"
    rc = getattr(_load(), fn)(ACTS[act], a.ctypes.data, b.ctypes.data, bp, r.ctypes.data, M, N, K,
                              sam, sak, sbk, sbn, N)
    if rc != 0:
        raise MemoryError("oracle could not allocate its row accumulator")
    return r


def strided_at(act: str, a: np.ndarray, b: np.ndarray, bias, rows, cols, M: int, N: int, K: int,
               sam: int, sak: int, sbk: int, sbn: int) -> np.ndarray:
    """act(A·B + bias)[rows[t], cols[t]] for each t with general strides, as float64."""
    dtype = _check_strided(a, b, M, N, K, sam, sak, sbk, sbn)
    ii = np.ascontiguousarray(rows, dtype=np.int64)
    jj = np.ascontiguousarray(cols, dtype=np.int64)
    if ii.shape != jj.shape:
        raise ValueError("rows and cols differ in length")
    if ii.size and (ii.min() < 0 or jj.min() < 0 or ii.max() >= M or jj.max() >= N):
        raise ValueError("index outside the M x N result")
    bp = _bias_ptr(bias, dtype, N)
    out = np.empty(ii.size, dtype=np.float64)
    if ii.size:
        fn = "oracle_strided_f32_at" if dtype == np.float32 else "oracle_strided_bf16_at"
        getattr(_load(), fn)(ACTS[act], a.ctypes.data, b.ctypes.data, bp, K, sam, sak, sbk, sbn,
                             ii.ctypes.data, jj.ctypes.data, ii.size, out.ctypes.data)
    return out


def _rows(x: np.ndarray, M, N, ldx):
    dtype, _, _ = _dtype_and_fns(x)
    if not x.flags.c_contiguous:
        raise ValueError("oracle inputs must be C-contiguous buffers")
    if M is None:
        M, N = x.shape
        ldx = max(N, 1)
    ldx = ldx if ldx is not None else max(N, 1)
    if min(M, N) < 0 or ldx < max(1, N):
        raise ValueError("bad sizes or leading dimension")
    if M > 0 and N > 0 and x.size < (M - 1) * ldx + N:
        raise ValueError("X buffer too small")
    return dtype, M, N, ldx


def softmax_rows(x: np.ndarray, M=None, N=None, ldx=None) -> np.ndarray:
    """Softmax of each row of X (M x N, leading dimension ldx) as an M x N
    float64 array: exp(x - rowmax) / sum(exp(x - rowmax))."""
    dtype, M, N, ldx = _rows(x, M, N, ldx)
    r = np.empty((M, N), dtype=np.float64)
    if M == 0 or N == 0:
        return r
    fn = "oracle_softmax_rows_f32" if dtype == np.float32 else "oracle_softmax_rows_bf16"
    if getattr(_load(), fn)(x.ctypes.data, r.ctypes.data, M, N, ldx) != 0:
        raise MemoryError("oracle could not allocate its row buffer")
    return r


def row_sum(x: np.ndarray, M=None, N=None, ldx=None) -> np.ndarray:
    """Sum of each row of X (M x N, leading dimension ldx) as M float64 values."""
    dtype, M, N, ldx = _rows(x, M, N, ldx)
    r = np.zeros(M, dtype=np.float64)
    if M == 0:
        return r
    fn = "oracle_row_sum_f32" if dtype == np.float32 else "oracle_row_sum_bf16"
    getattr(_load(), fn)(x.ctypes.data, r.ctypes.data, M, N, ldx)
    return r

"""The oracle: a plain, slow, obviously correct CPU GEMM in binary64.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with
the GPU path and imports nothing from it.

``gemm`` computes C[i][j] = sum_k A(i,k) * B(k,j) in binary64 with k ascending,
from operands stored as fp32 (``numpy.float32``) or as raw 16-bit patterns of
fp16 / bf16 (``numpy.uint16``), with row- or column-major A and B and arbitrary
leading dimensions.  The definition is the element formula of the product
("CUDA tile", 2.1 walk-through; "Tiling 策略与内存层次优化", roofline section).
The arithmetic lives in ``gemm_oracle.c``; this module only checks extents (so
the C code never reads out of bounds) and marshals arrays.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
CODES = {"f32": 0, "f16": 1, "bf16": 2}
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, vp, dp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double), ctypes.c_int
    lib.oracle_gemm_rows.argtypes = [i64, i64, i64, vp, i64, i32, vp, i64, i32, i32, i64, i64, dp]
    lib.oracle_gemm_rows.restype = i32
    lib.oracle_gemm_elements.argtypes = [i64, vp, i64, i32, vp, i64, i32, i32, vp, vp, i64, dp]
    lib.oracle_gemm_elements.restype = None
    lib.oracle_encode_array.argtypes = [dp, vp, i64, i32]
    lib.oracle_decode_array.argtypes = [vp, dp, i64, i32]
    lib.oracle_decode_f16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_f16.restype = ctypes.c_double
    lib.oracle_decode_bf16.argtypes = [ctypes.c_uint16]
    lib.oracle_decode_bf16.restype = ctypes.c_double
    lib.oracle_encode_f16.argtypes = [ctypes.c_double]
    lib.oracle_encode_f16.restype = ctypes.c_uint16
    lib.oracle_encode_bf16.argtypes = [ctypes.c_double]
    lib.oracle_encode_bf16.restype = ctypes.c_uint16
    lib.oracle_max_threads.restype = i32
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_set_threads.restype = None
    _lib = lib
    return lib


def _storage(x, dtype):
    want = np.float32 if dtype == "f32" else np.uint16
    x = np.ascontiguousarray(x).reshape(-1)
    if x.dtype != want:
        raise TypeError(f"oracle expects {np.dtype(want).name} storage for {dtype}, got {x.dtype}")
    return x


def _need(rows, cols, ld):
    """Elements a (rows x cols) operand with leading dimension ld occupies."""
    if rows == 0 or cols == 0:
        return 0
    return (rows - 1) * ld + cols


def _check_operands(M, N, K, A, lda, a_col, B, ldb, b_col):
    if min(M, N, K) < 0:
        raise ValueError("negative extent")
    a_rows, a_cols = (K, M) if a_col else (M, K)
    b_rows, b_cols = (N, K) if b_col else (K, N)
    if a_rows and a_cols and lda < a_cols:
        raise ValueError("lda smaller than the contiguous extent of A")
    if b_rows and b_cols and ldb < b_cols:
        raise ValueError("ldb smaller than the contiguous extent of B")
    if A.size < _need(a_rows, a_cols, lda):
        raise ValueError("A storage too small")
    if B.size < _need(b_rows, b_cols, ldb):
        raise ValueError("B storage too small")


def gemm(M, N, K, A, lda, B, ldb, dtype, a_col=False, b_col=False, rows=None):
    """Rows ``rows = (r0, r1)`` (default all) of C as a float64 (r1-r0) x N array."""
    lib = _load()
    A = _storage(A, dtype)
    B = _storage(B, dtype)
    _check_operands(M, N, K, A, lda, a_col, B, ldb, b_col)
    r0, r1 = (0, M) if rows is None else rows
    if not (0 <= r0 <= r1 <= M):
        raise ValueError("row range out of bounds")
    C = np.zeros((r1 - r0, N), dtype=np.float64)
    if r1 > r0 and N > 0:
        rc = lib.oracle_gemm_rows(M, N, K, A.ctypes.data, lda, int(a_col), B.ctypes.data, ldb,
                                  int(b_col), CODES[dtype], r0, r1,
                                  C.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
        if rc != 0:
            raise MemoryError("oracle could not allocate its decoded operands")
    return C


def elements(M, N, K, A, lda, B, ldb, dtype, ii, jj, a_col=False, b_col=False):
    """C[ii[t], jj[t]] for each t, one binary64 dot product per element."""
    lib = _load()
    A = _storage(A, dtype)
    B = _storage(B, dtype)
    _check_operands(M, N, K, A, lda, a_col, B, ldb, b_col)
    ii = np.ascontiguousarray(ii, dtype=np.int64)
    jj = np.ascontiguousarray(jj, dtype=np.int64)
    if ii.shape != jj.shape:
        raise ValueError("index arrays differ in shape")
    if ii.size and (ii.min() < 0 or ii.max() >= M or jj.min() < 0 or jj.max() >= N):
        raise ValueError("sample index out of range")
    out = np.zeros(ii.shape, dtype=np.float64)
    if ii.size:
        lib.oracle_gemm_elements(K, A.ctypes.data, lda, int(a_col), B.ctypes.data, ldb, int(b_col),
                                 CODES[dtype], ii.ctypes.data, jj.ctypes.data, ii.size,
                                 out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out


def encode(x, dtype):
    """binary64 -> fp16 / bf16 bit patterns, round to nearest, ties to even."""
    lib = _load()
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    lib.oracle_encode_array(x.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), out.ctypes.data,
                            x.size, CODES[dtype])
    return out


def decode(bits, dtype):
    """Storage (fp32 values or 16-bit patterns) -> exact binary64 values."""
    lib = _load()
    bits = _storage(bits, dtype) if dtype == "f32" else np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    lib.oracle_decode_array(bits.ctypes.data, out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
                            bits.size, CODES[dtype])
    return out


def max_threads():
    return int(_load().oracle_max_threads())


def set_threads(n):
    """Threads of the oracle's parallel loops from now on (results do not depend on it)."""
    _load().oracle_set_threads(int(n))


def epilogue(S, alpha=1.0, beta=0.0, C_prior=None, bias=None, activation="none"):
    """The fused epilogue on an exact product S (binary64, M x N): element-wise work on
    the GEMM tile's output before it is written back ("Tiling 策略与内存层次优化",
    fusion stage: bias add and ReLU fused into the tile's output end), with the usual
    scaling of the product and of the prior C:

        T[i][j] = act(alpha * S[i][j] + beta * C_prior[i][j] + bias[j]),

    act = ReLU (everything not above zero, NaN included, becomes +0) or the identity.
    alpha and beta are taken as the fp32 values a caller passes; C_prior is the
    decoded prior C (binary64, exact), bias N fp32 values.  beta == 0 ignores C_prior.
    Computed in binary64: T is exact whenever its terms are small integers."""
    S = np.asarray(S, dtype=np.float64)
    T = np.float64(np.float32(alpha)) * S
    if np.float32(beta) != 0:
        T = T + np.float64(np.float32(beta)) * np.asarray(C_prior, dtype=np.float64)
    if bias is not None:
        T = T + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    if activation == "relu":
        T = np.where(T > 0, T, 0.0)
    elif activation != "none":
        raise ValueError(f"unknown activation {activation}")
    return T


def transpose(x, rows, cols, ld_in, ld_out=None):
    """The transpose as defined: out[c][r] = in[r][c] ("CUDA tile", applications section,
    the tiled transpose), element by element over a flat row-major storage of any
    element type (the values are moved, not interpreted).  Returns the flat output
    storage (cols x ld_out, padding columns zero)."""
    x = np.ascontiguousarray(x).reshape(-1)
    ld_out = rows if ld_out is None else ld_out
    if ld_in < cols or ld_out < rows:
        raise ValueError("leading dimension smaller than the row length")
    if rows and cols and x.size < (rows - 1) * ld_in + cols:
        raise ValueError("input storage too short")
    out = np.zeros(cols * ld_out, dtype=x.dtype)
    r = np.arange(rows, dtype=np.int64)
    for c in range(cols):
        out[c * ld_out + r] = x[r * ld_in + c]
    return out


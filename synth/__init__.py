"""Seeded synthetic operands for the GEMM workloads.

This module only draws and lays out input matrices; it holds none of the
product's arithmetic.  Both the GPU-side tests/benchmark and the oracle take
their operands from here, so the exact bytes fed to the GPU are the oracle's input.

Recipe (one CPU ``torch.Generator`` per call, seeded; A is drawn before B):
  uniform     torch.rand(shape) * 2 - 1, i.e. uniform on [-1, 1), then rounded
              to the element type with round-to-nearest-even (``Tensor.to``)
  normal_half torch.randn(shape) * 0.5, then rounded the same way
  ones        every entry 1
  identity    square identity (requires M == K for A, K == N for B)
  perm        permutation matrix from ``torch.randperm``
  int         integers drawn uniformly from [-r, r]
  sparse_pm1  entries in {-1, 0, +1}; B column j is nonzero only at rows k with
              (k + j) % period == 0, so every output is a sum of at most
              ceil(K / period) terms of magnitude 1 and every K slab contributes

Storage: row-major A is (M, lda), column-major A is (K, lda) holding A^T rows;
row-major B is (K, ldb), column-major B is (N, ldb).  Padding columns beyond the
logical extent (ld > extent) are filled with ``pad`` (NaN by default) so that a
kernel which reads them by mistake produces NaN in its output.
"""
from dataclasses import dataclass, field

import numpy as np
import torch

TORCH_DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    dtype: str          # input element type
    out: str            # output element type
    a_col: bool = False
    b_col: bool = False
    dist: str = "uniform"
    seed: int = 0
    note: str = field(default="", compare=False)


# The five workloads (and the ragged variant of the second) the path is measured on.
WORKLOADS = {
    "f32_64": Workload("f32_64", 64, 64, 64, "f32", "f32",
                       note="fp32 64^3, the 64x64 matrix cut into 2x2 tiles of 32"),
    "f16_1024": Workload("f16_1024", 1024, 1024, 1024, "f16", "f16",
                         note="fp16 1024^3 row-major, fp16 out"),
    "f16_1000": Workload("f16_1000", 1000, 1000, 1000, "f16", "f16",
                         note="fp16 1000^3 ragged edge tiles, fp16 out"),
    "f16_2048_nt": Workload("f16_2048_nt", 2048, 2048, 2048, "f16", "f32", b_col=True,
                            dist="normal_half",
                            note="fp16 2048^3, A row-major, B column-major, fp32 out"),
    "bf16_4096": Workload("bf16_4096", 4096, 4096, 4096, "bf16", "bf16",
                          note="bf16 4096^3 row-major, bf16 out (compute-bound)"),
    "bf16_skinny": Workload("bf16_skinny", 16, 8192, 8192, "bf16", "f32",
                            note="bf16 16x8192x8192 row-major, fp32 out (bandwidth-bound)"),
}


def _draw(gen, shape, dist, dtype, r=4):
    if dist == "uniform":
        x = torch.rand(shape, generator=gen, dtype=torch.float32) * 2 - 1
    elif dist == "normal_half":
        x = torch.randn(shape, generator=gen, dtype=torch.float32) * 0.5
    elif dist == "ones":
        x = torch.ones(shape, dtype=torch.float32)
    elif dist == "int":
        x = torch.randint(-r, r + 1, shape, generator=gen).to(torch.float32)
    else:
        raise ValueError(f"unknown distribution {dist}")
    return x.to(TORCH_DTYPES[dtype])


def _special(gen, rows, cols, dist, dtype, period, is_b):
    if dist == "identity":
        if rows != cols:
            raise ValueError("identity operand must be square")
        return torch.eye(rows, dtype=torch.float32).to(TORCH_DTYPES[dtype])
    if dist == "perm":
        if rows != cols:
            raise ValueError("permutation operand must be square")
        p = torch.randperm(rows, generator=gen)
        x = torch.zeros((rows, cols), dtype=torch.float32)
        x[torch.arange(rows), p] = 1.0
        return x.to(TORCH_DTYPES[dtype])
    if dist == "sparse_pm1":
        signs = torch.randint(0, 2, (rows, cols), generator=gen).to(torch.float32) * 2 - 1
        if is_b:  # rows = k, cols = j
            k = torch.arange(rows).view(-1, 1)
            j = torch.arange(cols).view(1, -1)
            mask = ((k + j) % period == 0).to(torch.float32)
            return (signs * mask).to(TORCH_DTYPES[dtype])
        zeros = torch.randint(0, 4, (rows, cols), generator=gen) == 0
        return (signs * (~zeros).to(torch.float32)).to(TORCH_DTYPES[dtype])
    return None


def logical(M, N, K, dtype, dist="uniform", seed=0, dist_b=None, r=4, period=1):
    """Logical A (M x K) and B (K x N) as CPU tensors of the element type."""
    gen = torch.Generator().manual_seed(seed)
    dist_b = dist if dist_b is None else dist_b
    A = _special(gen, M, K, dist, dtype, period, False)
    if A is None:
        A = _draw(gen, (M, K), dist, dtype, r=r)
    B = _special(gen, K, N, dist_b, dtype, period, True)
    if B is None:
        B = _draw(gen, (K, N), dist_b, dtype, r=r)
    return A, B


def lay_out(X, col_major, ld=None, pad=float("nan")):
    """Store logical X (rows x cols) row- or column-major with leading dimension ld."""
    S = X.t() if col_major else X
    rows, cols = S.shape
    ld = cols if ld is None else ld
    if ld < cols:
        raise ValueError("leading dimension smaller than the contiguous extent")
    out = torch.full((rows, ld), pad, dtype=X.dtype) if ld > cols else torch.empty((rows, ld), dtype=X.dtype)
    out[:, :cols] = S
    return out.contiguous(), ld


def operands(M, N, K, dtype, a_col=False, b_col=False, lda=None, ldb=None, dist="uniform",
             seed=0, dist_b=None, r=4, period=1, pad=float("nan")):
    """Stored operands: (A_storage, lda, B_storage, ldb, A_logical, B_logical)."""
    A, B = logical(M, N, K, dtype, dist=dist, seed=seed, dist_b=dist_b, r=r, period=period)
    As, lda = lay_out(A, a_col, lda, pad)
    Bs, ldb = lay_out(B, b_col, ldb, pad)
    return As, lda, Bs, ldb, A, B


def workload_operands(w: Workload, seed=None):
    return operands(w.M, w.N, w.K, w.dtype, a_col=w.a_col, b_col=w.b_col, dist=w.dist,
                    seed=w.seed if seed is None else seed)


def to_storage_numpy(t):
    """CPU tensor -> numpy storage the oracle reads: float32, or raw uint16 patterns."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def from_storage_numpy(x, dtype):
    """Inverse of ``to_storage_numpy`` for 16-bit types (raw patterns -> tensor)."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint16).view(np.int16))
    return t.view(TORCH_DTYPES[dtype])


def epilogue_inputs(M, N, out_t, ldc=None, dist="uniform", seed=1, r=4):
    """Prior C (M x ldc storage of the output type, padding columns NaN) and an fp32
    bias of N values for the fused-epilogue tests, from one seeded generator (C first).
    dist "uniform": both uniform on [-1, 1); "int": integers in [-r, r]."""
    gen = torch.Generator().manual_seed(seed)
    ldc = N if ldc is None else ldc
    C = _draw(gen, (M, N), dist, out_t, r=r)
    bias = _draw(gen, (N,), dist, "f32", r=r)
    Cs, _ = lay_out(C, False, ldc)
    return Cs, bias


def raw_matrix(rows, ld, elem_bytes, seed=0, pad=0):
    """rows x ld matrix of random bit patterns of 2- or 4-byte elements (every pattern,
    NaNs included: a transpose moves bytes), as a CPU tensor of int16 / int32; columns
    are all drawn, the caller decides how many of them are logical."""
    gen = torch.Generator().manual_seed(seed)
    dt = {2: torch.int16, 4: torch.int32}[elem_bytes]
    lo, hi = (-(1 << 15), 1 << 15) if elem_bytes == 2 else (-(1 << 31), 1 << 31)
    return torch.randint(lo, hi, (rows, ld), generator=gen, dtype=torch.int64).to(dt)


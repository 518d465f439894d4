"""The fp32 matrix-core kernel (v_mfma_f32_32x32x2_f32, 128 x 128 tiles) against the
oracle: bit-exact on small-integer products in every layout, ragged extents whose
contiguous dimension is not a multiple of four (element-wise loads), misaligned
pointers and padded leading dimensions, and the planner's choice at 4096^3 fp32 on
sampled elements."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from gemm_cases import check_exact, check_tolerance, oracle_ref, run_gpu

pytestmark = pytest.mark.gpu

CFG = (2, 128, 128, 16, 2, 2, 2, 1)
LAYOUTS = list(itertools.product((False, True), repeat=2))


@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
def test_exact_integer_products(a_col, b_col):
    M, N, K = 384, 256, 512
    print(f"[mfma32 exact] a_col={a_col} b_col={b_col}", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "f32", a_col, b_col, dist="int", r=3, seed=21)
    _, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, "f32", "f32", a_col, b_col, cfg=CFG)
    assert (desc["kind"], desc["bm"], desc["bk"]) == (2, 128, 16)
    check_exact(raw, oracle_ref(As, lda, Bs, ldb, M, N, K, "f32", a_col, b_col), "f32")


@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
@pytest.mark.parametrize("M,N,K", [(130, 257, 203), (1, 129, 17), (129, 1, 33), (200, 200, 1)])
def test_ragged_extents(M, N, K, a_col, b_col):
    print(f"[mfma32 ragged] {M}x{N}x{K} a_col={a_col} b_col={b_col}", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "f32", a_col, b_col, seed=22)
    vals, _, _ = run_gpu(As, lda, Bs, ldb, M, N, K, "f32", "f32", a_col, b_col, cfg=CFG)
    check_tolerance(vals, oracle_ref(As, lda, Bs, ldb, M, N, K, "f32", a_col, b_col), "f32")


@pytest.mark.parametrize("offsets,pads", [((1, 0, 0), (0, 0, 0)), ((0, 3, 0), (0, 0, 0)), ((0, 0, 1), (0, 0, 5)),
                                          ((0, 0, 0), (4, 8, 4)), ((2, 2, 2), (3, 1, 2))])
def test_misaligned_and_padded(offsets, pads):
    M, N, K = 264, 200, 136
    print(f"[mfma32 offsets {offsets} pads {pads}]", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "f32", lda=K + pads[0], ldb=N + pads[1], seed=23)
    vals, _, _ = run_gpu(As, lda, Bs, ldb, M, N, K, "f32", "f32", ldc=N + pads[2], cfg=CFG,
                         offset_a=offsets[0], offset_b=offsets[1], offset_c=offsets[2])
    check_tolerance(vals, oracle_ref(As, lda, Bs, ldb, M, N, K, "f32"), "f32")


def test_4096_fp32_sampled():
    M = N = K = 4096
    print("[mfma32 4096^3 fp32]", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "f32", seed=24)
    vals, _, desc = run_gpu(As, lda, Bs, ldb, M, N, K, "f32", "f32")
    assert (desc["kind"], desc["bm"], desc["bk"]) == (2, 128, 16)      # the planner's choice
    rng = np.random.default_rng(0)
    ii = np.concatenate([rng.integers(0, M, 4000), [0, 127, 128, M - 1]])
    jj = np.concatenate([rng.integers(0, N, 4000), [0, 128, 127, N - 1]])
    ref = oracle.elements(M, N, K, synth.to_storage_numpy(As), lda, synth.to_storage_numpy(Bs), ldb, "f32", ii, jj)
    check_tolerance(vals[ii, jj], ref, "f32", "sampled")

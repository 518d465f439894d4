"""Split-K of the eight-wave kernels (K chunks as separate workgroups, fp32 partials
added in chunk order by a second kernel) against the oracle: every split factor of
both tile shapes, every layout, bit-exact integer products, chunks that do not divide
K, the fused epilogue applied by the reduction, the planner's choice at 512 x 512 x
8192, and bit-identical results run after run."""
import itertools

import numpy as np
import pytest

import memory_hierarchy_optimisation_amd as mh
import oracle
import synth
from gemm_cases import check_exact, check_tolerance, oracle_ref, run_gpu

pytestmark = pytest.mark.gpu

SPLITS = [(2, 64, 64, 128, 2, 4, 5, s) for s in (2, 4, 8)] + [(2, 128, 128, 64, 2, 4, 5, s) for s in (2, 4, 8)]
LAYOUTS = list(itertools.product((False, True), repeat=2))


@pytest.mark.parametrize("cfg", SPLITS)
@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
def test_exact_integer_products(cfg, a_col, b_col):
    M, N, K = 256, 384, 2048
    print(f"[split-K exact] cfg={cfg} a_col={a_col} b_col={b_col}", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "bf16", a_col, b_col, dist="int", r=3, seed=31)
    _, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, "bf16", "f32", a_col, b_col, cfg=cfg)
    assert desc["split_k"] == cfg[7]
    check_exact(raw, oracle_ref(As, lda, Bs, ldb, M, N, K, "bf16", a_col, b_col), "f32")


@pytest.mark.parametrize("cfg", SPLITS)
@pytest.mark.parametrize("in_t,out_t", [("f16", "f16"), ("bf16", "bf16"), ("f16", "f32")])
def test_ragged_and_uneven_chunks(cfg, in_t, out_t):
    M, N, K = 200, 264, 2 * cfg[7] * cfg[3] + 40      # two slabs a chunk, the last chunk shorter
    print(f"[split-K ragged] cfg={cfg} {in_t}->{out_t} {M}x{N}x{K}", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, seed=32)
    vals, _, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, cfg=cfg)
    check_tolerance(vals, oracle_ref(As, lda, Bs, ldb, M, N, K, in_t), out_t)


@pytest.mark.parametrize("cfg", [SPLITS[1], SPLITS[4]])
def test_epilogue_through_the_reduction(cfg):
    M, N, K = 256, 512, 4096
    print(f"[split-K epilogue] cfg={cfg}", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "bf16", dist="int", r=3, seed=33)
    Cs, bias = synth.epilogue_inputs(M, N, "bf16", dist="int", r=4, seed=34)
    epi = dict(alpha=2.0, beta=-1.0, bias=bias, activation=mh.GEMM_ACT_RELU)
    _, raw, _ = run_gpu(As, lda, Bs, ldb, M, N, K, "bf16", "bf16", cfg=cfg, c_init=Cs, epi=epi)
    S = oracle_ref(As, lda, Bs, ldb, M, N, K, "bf16")
    prior = oracle.decode(synth.to_storage_numpy(Cs), "bf16")
    check_exact(raw, oracle.epilogue(S, 2.0, -1.0, prior, bias.numpy(), "relu"), "bf16")


def test_planner_choice_and_reproducibility():
    M, N, K = 512, 512, 8192
    print("[split-K 512x512x8192]", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "bf16", seed=35)
    v1, raw1, desc = run_gpu(As, lda, Bs, ldb, M, N, K, "bf16", "f32")
    assert desc["split_k"] == 4 and desc["bm"] == 64
    _, raw2, _ = run_gpu(As, lda, Bs, ldb, M, N, K, "bf16", "f32")
    assert np.array_equal(raw1, raw2)
    check_tolerance(v1, oracle_ref(As, lda, Bs, ldb, M, N, K, "bf16"), "f32")

"""gemm_run_noalloc, the entry point that allocates no device memory, against
gemm_plan + gemm_run_epilogue: the same kernels with the split-K workspace in the
library's per-GPU scratch array instead of the plan's.  Each case makes two calls in
a row, the second on a smaller problem (another split and another workspace layout
in the same array), and compares every output bit for bit with the planned path and
with the oracle at the tolerance of the output type."""
import numpy as np
import pytest
import torch

import memory_hierarchy_optimisation_amd as mh
import synth
from gemm_cases import check_tolerance, oracle_ref

pytestmark = pytest.mark.gpu

CASES = {
    "skinny_split": ("bf16", "f32", [(16, 8192, 8192), (16, 2048, 4096)]),
    "eight_wave_split": ("bf16", "bf16", [(512, 512, 8192), (256, 256, 4096)]),
    "eight_wave_split_f16": ("f16", "f32", [(512, 768, 4096), (128, 256, 2048)]),
}


def _run_both(M, N, K, in_t, out_t, seed, epi):
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, seed=seed)
    A, B = As.cuda(), Bs.cuda()
    tdt = synth.TORCH_DTYPES[out_t]
    prior = (torch.rand((M, N), generator=torch.Generator().manual_seed(seed + 1)) * 2 - 1).to(tdt)
    bias = torch.linspace(-0.5, 0.5, N, device="cuda") if epi else None
    code = mh.DTYPE_OF[(in_t, out_t)]
    kw = dict(alpha=0.75, beta=0.5, bias=bias, activation=mh.GEMM_ACT_RELU) if epi else {}
    C_plan = prior.cuda()
    plan = mh.gemm_plan(M, N, K, lda, ldb, N, code, 0)
    try:
        desc = mh.gemm_plan_describe(plan)
        if epi:
            mh.gemm_run_epilogue(plan, A, B, C_plan, **kw)
        else:
            mh.gemm_run(plan, A, B, C_plan)
    finally:
        torch.cuda.synchronize()
        mh.gemm_destroy(plan)
    C_free = prior.cuda()
    mh.gemm_run_noalloc(M, N, K, lda, ldb, N, code, 0, A, B, C_free, epilogue=epi, **kw)
    torch.cuda.synchronize()
    return As, lda, Bs, ldb, prior, bias, C_plan.cpu(), C_free.cpu(), desc


@pytest.mark.parametrize("epi", [False, True])
@pytest.mark.parametrize("case", sorted(CASES))
def test_noalloc_matches_planned_run(case, epi):
    in_t, out_t, shapes = CASES[case]
    for n, (M, N, K) in enumerate(shapes):
        print(f"[noalloc] {case} epi={epi} call {n + 1}: M={M} N={N} K={K} {in_t}->{out_t}", flush=True)
        As, lda, Bs, ldb, prior, bias, C_plan, C_free, desc = _run_both(M, N, K, in_t, out_t, 50 + n, epi)
        assert desc["split_k"] > 1 and desc["workspace_bytes"] > 0, desc
        assert torch.equal(C_plan.view(torch.int16 if out_t != "f32" else torch.int32),
                           C_free.view(torch.int16 if out_t != "f32" else torch.int32)), f"call {n + 1}"
        S = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t)
        if epi:
            import oracle
            ref = oracle.epilogue(S, 0.75, 0.5, prior.to(torch.float64).numpy(), bias.cpu().numpy(), "relu")
        else:
            ref = S
        check_tolerance(C_free.to(torch.float64).numpy(), ref, out_t, f"{case} call {n + 1}")


def test_noalloc_plain_products_and_degenerate_extents():
    """Plans without a workspace run as gemm_run does; K = 0 fills zeros; M = 0 is a no-op."""
    M, N, K = 300, 200, 100
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "f16", seed=3)
    A, B = As.cuda(), Bs.cuda()
    C = torch.full((M, N), float("nan"), device="cuda")
    mh.gemm_run_noalloc(M, N, K, lda, ldb, N, mh.GEMM_F16_F32, 0, A, B, C)
    torch.cuda.synchronize()
    check_tolerance(C.cpu().double().numpy(), oracle_ref(As, lda, Bs, ldb, M, N, K, "f16"), "f32", "plain")
    mh.gemm_run_noalloc(M, N, 0, 1, N, N, mh.GEMM_F16_F32, 0, A, B, C)
    torch.cuda.synchronize()
    assert np.all(C.cpu().numpy() == 0.0)
    mh.gemm_run_noalloc(0, N, K, lda, ldb, N, mh.GEMM_F16_F32, 0, A, B, C)
    torch.cuda.synchronize()

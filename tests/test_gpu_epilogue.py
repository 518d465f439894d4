"""Parity of the fused epilogue (gemm_run_epilogue) with the oracle, on the GPU.

C = act(alpha * A x B + beta * C_prior + bias[j]) through every compiled variant on a
ragged shape, bit-exact on small-integer suites (every kernel family, every output
type), beta == 0 never reading C, the identity epilogue equal to gemm_run bit for
bit, K == 0, and the measured workloads at full size (sampled where the oracle would
be slow).
"""
import numpy as np
import pytest
import torch

import memory_hierarchy_optimisation_amd as mh
import oracle
import synth
from gemm_cases import check_exact, check_tolerance, oracle_ref, run_gpu

pytestmark = pytest.mark.gpu

ACT = {mh.GEMM_ACT_NONE: "none", mh.GEMM_ACT_RELU: "relu"}


def _prior(Cs, out_t):
    st = synth.to_storage_numpy(Cs)
    return st.astype(np.float64) if out_t == "f32" else oracle.decode(st, out_t)


def _reference(S, Cs, bias, out_t, epi, N):
    return oracle.epilogue(S, epi["alpha"], epi["beta"], _prior(Cs, out_t)[:, :N], bias.numpy()[:N],
                           ACT[epi["activation"]])


def _fits(M, N, K, in_t, out_t, cfg):
    try:
        p = mh.gemm_plan_config(M, N, K, K, N, N, mh.DTYPE_OF[(in_t, out_t)], 0, cfg)
    except mh.GemmError:
        return False
    mh.gemm_destroy(p)
    return True


def _accepts(cfg, in_t):
    M = 16 if cfg[0] == mh.GEMM_KIND_SKINNY else 512
    try:
        p = mh.gemm_plan_config(M, 512, 512, 512, 512, 512, mh.DTYPE_OF[(in_t, "f32")], 0, cfg)
    except mh.GemmError:
        return False
    mh.gemm_destroy(p)
    return True


def _configs():
    out = []
    for c in mh.gemm_catalogue():
        if _accepts(c, "f32"):
            out.append((c, "f32", "f32"))
        if _accepts(c, "bf16"):
            out += [(c, "bf16", "f32")] if c[0] == mh.GEMM_KIND_SKINNY else [(c, "bf16", "bf16"), (c, "f16", "f32")]
    return out


@pytest.mark.parametrize("cfg,in_t,out_t", _configs())
def test_every_variant_with_bias_relu_alpha_beta(cfg, in_t, out_t):
    if cfg[0] == mh.GEMM_KIND_SKINNY:
        M, N, K = 16, 1096, 1032
    elif cfg[7] > 1:     # eight-wave split-K: two K slabs a chunk at least
        M, N, K = 304, 272, 2 * cfg[7] * cfg[3] + 40
    else:
        M, N, K = (300, 270, 200) if _fits(300, 270, 200, in_t, out_t, cfg) else (304, 272, 200)
    print(f"[epilogue variant {cfg} {in_t}->{out_t}] M={M} N={N} K={K}", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, seed=5)
    Cs, bias = synth.epilogue_inputs(M, N, out_t, seed=6)
    epi = dict(alpha=0.75, beta=-0.5, bias=bias, activation=mh.GEMM_ACT_RELU)
    vals, _, desc = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, cfg=cfg, c_init=Cs, epi=epi)
    assert tuple(desc[k] for k in ("kind", "bm", "bn", "bk")) == cfg[:4]
    S = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t)
    check_tolerance(vals, _reference(S, Cs, bias, out_t, epi, N), out_t, f"{cfg}")


EXACT_CFGS = [None, (2, 256, 256, 32, 2, 4, 5, 1), (2, 128, 128, 64, 2, 4, 5, 1), (2, 64, 64, 128, 2, 4, 5, 1),
              (2, 128, 128, 64, 2, 2, 2, 1)]


@pytest.mark.parametrize("in_t,out_t", [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")])
@pytest.mark.parametrize("cfg", EXACT_CFGS)
@pytest.mark.parametrize("layout", [(False, False), (True, True)])
def test_exact_integer_epilogue(in_t, out_t, cfg, layout):
    a_col, b_col = layout
    M = N = K = 512
    print(f"[epilogue exact {in_t}->{out_t} cfg={cfg} layout={layout}]", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, a_col=a_col, b_col=b_col, dist="int", r=3, seed=7)
    Cs, bias = synth.epilogue_inputs(M, N, out_t, dist="int", r=4, seed=8)
    epi = dict(alpha=2.0, beta=-1.0, bias=bias, activation=mh.GEMM_ACT_RELU)
    _, raw, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, a_col, b_col, cfg=cfg, c_init=Cs, epi=epi)
    S = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, a_col, b_col)
    check_exact(raw, _reference(S, Cs, bias, out_t, epi, N), out_t, f"cfg {cfg}")


@pytest.mark.parametrize("in_t,out_t,M,N,K,cfg", [
    ("f32", "f32", 64, 64, 64, None), ("f32", "f32", 100, 130, 70, (1, 128, 128, 16, 4, 1, 2, 1)),
    ("bf16", "f32", 16, 1024, 2048, (3, 16, 128, 32, 1, 4, 2, 4)),
    ("bf16", "f32", 16, 1024, 2048, (3, 16, 128, 32, 1, 4, 2, 16)),
    ("f16", "f16", 12, 1000, 504, None),
])
def test_exact_integer_epilogue_other_kernels(in_t, out_t, M, N, K, cfg):
    print(f"[epilogue exact {in_t}->{out_t} {M}x{N}x{K} cfg={cfg}]", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, dist="int", r=3, seed=9)
    Cs, bias = synth.epilogue_inputs(M, N, out_t, dist="int", r=4, seed=10)
    epi = dict(alpha=3.0, beta=2.0, bias=bias, activation=mh.GEMM_ACT_NONE)
    _, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, cfg=cfg, c_init=Cs, epi=epi)
    S = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t)
    check_exact(raw, _reference(S, Cs, bias, out_t, epi, N), out_t, f"{desc['kind']} {desc['bm']}")


@pytest.mark.parametrize("in_t,out_t,M,N,K", [("bf16", "bf16", 512, 512, 256), ("f32", "f32", 96, 80, 64),
                                               ("bf16", "f32", 16, 2048, 2048), ("f16", "f16", 1000, 1000, 136)])
def test_beta_zero_never_reads_c(in_t, out_t, M, N, K):
    print(f"[epilogue beta 0 {in_t}->{out_t} {M}x{N}x{K}]", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, seed=11)
    _, bias = synth.epilogue_inputs(M, N, out_t, seed=12)
    nan = torch.full((M, N), float("nan"), dtype=synth.TORCH_DTYPES[out_t])
    epi = dict(alpha=-1.5, beta=0.0, bias=bias, activation=mh.GEMM_ACT_NONE)
    vals, _, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, c_init=nan, epi=epi)
    assert np.isfinite(vals).all()
    S = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t)
    check_tolerance(vals, oracle.epilogue(S, -1.5, 0.0, None, bias.numpy()), out_t, "beta 0")


@pytest.mark.parametrize("in_t,out_t,M,N,K", [("bf16", "bf16", 4096, 512, 512), ("f16", "f32", 1000, 1000, 1000),
                                               ("f32", "f32", 64, 64, 64), ("bf16", "f32", 16, 8192, 1024)])
def test_identity_epilogue_is_gemm_run(in_t, out_t, M, N, K):
    print(f"[epilogue identity {in_t}->{out_t} {M}x{N}x{K}]", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, seed=13)
    _, raw0, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t)
    epi = dict(alpha=1.0, beta=0.0, bias=None, activation=mh.GEMM_ACT_NONE)
    _, raw1, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, epi=epi)
    assert np.array_equal(raw0, raw1)


@pytest.mark.parametrize("out_t", ["f32", "bf16"])
def test_k_zero_with_epilogue(out_t):
    M, N = 33, 70
    in_t = "f32" if out_t == "f32" else "bf16"
    print(f"[epilogue K=0 {out_t}]", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, 0, in_t, seed=14)
    Cs, bias = synth.epilogue_inputs(M, N, out_t, dist="int", r=4, seed=15)
    epi = dict(alpha=5.0, beta=-2.0, bias=bias, activation=mh.GEMM_ACT_RELU)
    _, raw, _ = run_gpu(As, max(lda, 1), Bs, ldb, M, N, 0, in_t, out_t, c_init=Cs, epi=epi)
    check_exact(raw, _reference(np.zeros((M, N)), Cs, bias, out_t, epi, N), out_t, "K=0")


def test_bad_epilogue_arguments():
    p = mh.gemm_plan(64, 64, 64, 64, 64, 64, mh.GEMM_F32_F32, 0)
    try:
        A = torch.zeros(64, 64, device="cuda")
        with pytest.raises(mh.GemmError, match="activation"):
            mh.gemm_run_epilogue(p, A, A, A, activation=7)
        bias = torch.zeros(65, device="cuda")
        with pytest.raises(mh.GemmError, match="aligned"):
            mh.gemm_run_epilogue(p, A, A, A, bias=bias.data_ptr() + 2)
    finally:
        mh.gemm_destroy(p)


@pytest.mark.parametrize("name", ["f16_1024", "f16_1000", "bf16_skinny", "f16_2048_nt", "bf16_4096"])
def test_workloads_with_epilogue(name):
    w = synth.WORKLOADS[name]
    As, lda, Bs, ldb, _, _ = synth.workload_operands(w)
    print(f"[epilogue workload {name}]", flush=True)
    Cs, bias = synth.epilogue_inputs(w.M, w.N, w.out, seed=16)
    epi = dict(alpha=0.5, beta=0.25, bias=bias, activation=mh.GEMM_ACT_RELU)
    vals, _, desc = run_gpu(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.out, w.a_col, w.b_col,
                            c_init=Cs, epi=epi)
    Cp = _prior(Cs, w.out)
    S = oracle_ref(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.a_col, w.b_col)
    check_tolerance(vals, oracle.epilogue(S, 0.5, 0.25, Cp, bias.numpy(), "relu"), w.out, name)


# The 256 x 256 eight-wave tile brings a 16-bit prior C into LDS with the loads of the
# four slabs past K (in the prologue when K has fewer than four slabs); these cases
# cover every slab count up to nine, ragged tiles, a padded C and the launches that
# fall back to the staged path (C misaligned, N not a multiple of 8).
CFG256 = (2, 256, 256, 32, 2, 4, 5, 1)


@pytest.mark.parametrize("K", [32, 64, 96, 128, 160, 200, 224, 288])
@pytest.mark.parametrize("in_t", ["f16", "bf16"])
def test_256_tile_prior_c_every_slab_count(K, in_t):
    M, N = 264, 520
    a_col = b_col = K % 64 == 0
    print(f"[epilogue 256 prior {in_t} K={K} layout={a_col}]", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, a_col=a_col, b_col=b_col, dist="int", r=3, seed=K)
    Cs, bias = synth.epilogue_inputs(M, N, in_t, dist="int", r=4, seed=K + 1)
    epi = dict(alpha=2.0, beta=-1.0, bias=bias, activation=mh.GEMM_ACT_RELU)
    _, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, in_t, a_col, b_col, cfg=CFG256, c_init=Cs, epi=epi)
    assert (desc["bm"], desc["bn"]) == (256, 256)
    S = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, a_col, b_col)
    check_exact(raw, _reference(S, Cs, bias, in_t, epi, N), in_t, f"K={K}")


@pytest.mark.parametrize("case", ["padded_ldc", "misaligned_c", "n_not_multiple_of_8", "no_bias_beta_only"])
def test_256_tile_prior_c_layouts_and_fallbacks(case):
    in_t = "bf16"
    M, N, K, ldc, off_c, b_col = 300, 264, 136, None, 0, False
    epi_kw = dict(alpha=0.5, beta=1.5, activation=mh.GEMM_ACT_NONE)
    if case == "padded_ldc":
        ldc = N + 24
    elif case == "misaligned_c":
        off_c = 1
    elif case == "n_not_multiple_of_8":
        N, b_col = 262, True
    print(f"[epilogue 256 prior {case}] M={M} N={N} K={K} ldc={ldc} off_c={off_c}", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, b_col=b_col, dist="int", r=3, seed=21)
    Cs, bias = synth.epilogue_inputs(M, N, in_t, dist="int", r=4, seed=22)
    epi = dict(epi_kw, bias=None if case == "no_bias_beta_only" else bias)
    _, raw, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, in_t, False, b_col, ldc=ldc, offset_c=off_c, cfg=CFG256,
                        c_init=Cs, epi=epi)
    S = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, False, b_col)
    ref_bias = np.zeros(N, np.float32) if epi["bias"] is None else bias.numpy()[:N]
    ref = oracle.epilogue(S, epi["alpha"], epi["beta"], _prior(Cs, in_t)[:, :N], ref_bias, "none")
    check_exact(raw, ref, in_t, case)


@pytest.mark.parametrize("in_t", ["f16", "bf16"])
@pytest.mark.parametrize("a_col,b_col", [(False, False), (False, True), (True, False), (True, True)])
def test_256_tile_prior_c_every_layout(in_t, a_col, b_col):
    M, N, K = 520, 264, 136
    print(f"[epilogue 256 prior layout {in_t} a_col={a_col} b_col={b_col}]", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, a_col=a_col, b_col=b_col, dist="int", r=3, seed=41)
    Cs, bias = synth.epilogue_inputs(M, N, in_t, dist="int", r=4, seed=42)
    epi = dict(alpha=-1.0, beta=0.5, bias=bias, activation=mh.GEMM_ACT_RELU)
    _, raw, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, in_t, a_col, b_col, cfg=CFG256, c_init=Cs, epi=epi)
    S = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, a_col, b_col)
    check_exact(raw, _reference(S, Cs, bias, in_t, epi, N), in_t, f"layout {a_col},{b_col}")

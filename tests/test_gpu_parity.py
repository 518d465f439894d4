"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Workload tests run each measured shape at full size in the configuration the planner
picks (the one the benchmark times) and compare every output with the oracle.  Then: ragged extents that leave partial tiles in every
dimension, every compiled variant forced on a ragged shape, every layout, padded
leading dimensions, misaligned pointers (narrow-load path), bit-exact small-integer
suites (one pins the round-to-nearest-even epilogue), closed forms, degenerate
extents and guard bands around C.
"""
import itertools

import numpy as np
import pytest
import torch

import memory_hierarchy_optimisation_amd as mh
import oracle
import synth
from gemm_cases import SENTINEL16, SENTINEL32, check_exact, check_tolerance, oracle_ref, run_gpu

pytestmark = pytest.mark.gpu

HALF_DTYPES = [("f16", "f16"), ("f16", "f32"), ("bf16", "bf16"), ("bf16", "f32")]
ALL_DTYPES = [("f32", "f32")] + HALF_DTYPES
LAYOUTS = list(itertools.product((False, True), repeat=2))


def _accepts(cfg, in_t):
    """Whether gemm_plan_config takes this configuration for this input type (asked of
    the library on an aligned 512^3 product, so that only the type decides)."""
    try:
        p = mh.gemm_plan_config(512, 512, 512, 512, 512, 512, mh.DTYPE_OF[(in_t, "f32")], 0, cfg)
    except mh.GemmError:
        return False
    mh.gemm_destroy(p)
    return True


def _catalogue_for(in_t):
    """Every compiled tile configuration for an input type (the library's catalogue,
    without the split-K variants, which have tests of their own)."""
    return [c for c in mh.gemm_catalogue() if c[0] != mh.GEMM_KIND_SKINNY and c[7] == 1 and _accepts(c, in_t)]


# ---- the measured workloads at full size ---------------------------------------------------

def _workload(name):
    w = synth.WORKLOADS[name]
    As, lda, Bs, ldb, _, _ = synth.workload_operands(w)
    print(f"[workload {name}] M={w.M} N={w.N} K={w.K} {w.dtype}->{w.out} a_col={w.a_col} "
          f"b_col={w.b_col}", flush=True)
    return w, As, lda, Bs, ldb


@pytest.mark.parametrize("name", ["f32_64", "f16_1024", "f16_1000", "bf16_skinny"])
def test_workload_whole(name):
    w, As, lda, Bs, ldb = _workload(name)
    C, raw, desc = run_gpu(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.out, w.a_col, w.b_col)
    Cref = oracle_ref(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.a_col, w.b_col)
    check_tolerance(C, Cref, w.out, name)


def test_workload_2048_nt_whole():
    w, As, lda, Bs, ldb = _workload("f16_2048_nt")
    C, raw, desc = run_gpu(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.out, w.a_col, w.b_col)
    Cref = oracle_ref(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.a_col, w.b_col)
    check_tolerance(C, Cref, w.out, "f16_2048_nt")
    # the elementwise bar as well, on every output (the normwise one could hide a few)
    err = np.abs(C - Cref)
    assert np.all(err <= 1e-3 * (np.abs(Cref) + 1.0)), float(err.max())


def test_workload_4096_whole():
    w, As, lda, Bs, ldb = _workload("bf16_4096")
    C, raw, desc = run_gpu(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.out, w.a_col, w.b_col)
    Cref = oracle_ref(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.a_col, w.b_col)
    check_tolerance(C, Cref, w.out, "bf16_4096")
    # Where |C_ref| >= 1 a bf16 step (>= 2^-7) is far above the fp32 sums' error, so the
    # result is the nearest bf16 of C_ref or a neighbour of it.
    big = np.abs(Cref) >= 1.0
    near = oracle.encode(Cref[big], "bf16").astype(np.int32)
    assert np.all(np.abs(raw[big].astype(np.int32) - near) <= 1)
    # All-ones closed form over the whole output at the same shape: C_ij = K exactly.
    ones = torch.ones((w.M, w.K), dtype=synth.TORCH_DTYPES[w.dtype])
    onesb = torch.ones((w.K, w.N), dtype=synth.TORCH_DTYPES[w.dtype])
    C1, raw1, _ = run_gpu(ones, w.K, onesb, w.N, w.M, w.N, w.K, w.dtype, w.out)
    assert np.all(C1 == w.K)


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 4096), (2048, 1024, 8192)])
def test_256_tile_both_k_contiguous_whole(M, N, K):
    """The 256 x 256 tile with row-major A and column-major B (A in pairs of slabs, B
    refilled in the phase of its last reads), forced, on random data at a deep K, every
    output against the oracle."""
    print(f"[256 tile NT whole] M={M} N={N} K={K}", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "bf16", b_col=True, seed=7)
    C, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, "bf16", "f32", False, True, cfg=(2, 256, 256, 32, 2, 4, 5, 1))
    assert (desc["bm"], desc["bn"]) == (256, 256)
    Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, "bf16", False, True)
    check_tolerance(C, Cref, "f32", "256 tile NT")
    err = np.abs(C - Cref)
    assert np.all(err <= 1e-3 * (np.abs(Cref) + 1.0)), float(err.max())


def test_workload_64_as_two_by_two_tiles():
    """The 64x64 product as 2 x 2 tiles of 32 x 32 ("CUDA tile", 2.1)."""
    w, As, lda, Bs, ldb = _workload("f32_64")
    cfg = (1, 32, 32, 32, 4, 1, 2, 1)
    C, raw, desc = run_gpu(As, lda, Bs, ldb, 64, 64, 64, "f32", "f32", cfg=cfg)
    assert (desc["grid_x"], desc["grid_y"]) == (2, 2)
    check_tolerance(C, oracle_ref(As, lda, Bs, ldb, 64, 64, 64, "f32"), "f32")


# ---- ragged extents ------------------------------------------------------------------------

EDGES = [1, 15, 16, 17, 31, 33, 63, 65, 127, 129]


@pytest.mark.parametrize("in_t,out_t", ALL_DTYPES)
def test_ragged_extents(in_t, out_t):
    rng = np.random.default_rng(5)
    cases = [(m, n, k) for m in EDGES for n in EDGES for k in (1, 17, 65, 129)]
    picks = rng.choice(len(cases), 60, replace=False)
    for idx in picks:
        M, N, K = cases[idx]
        for a_col, b_col in LAYOUTS:
            As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, a_col, b_col, seed=int(idx))
            C, raw, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, a_col, b_col)
            Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, a_col, b_col)
            check_tolerance(C, Cref, out_t, f"M={M} N={N} K={K} a_col={a_col} b_col={b_col}")


ALIGNED_ONLY = {(2, 256, 256, 32, 2, 4, 5, 1), (2, 128, 128, 64, 2, 4, 5, 1), (2, 64, 64, 128, 2, 4, 5, 1)}


@pytest.mark.parametrize("in_t,out_t", ALL_DTYPES)
def test_every_variant_every_layout_ragged(in_t, out_t):
    """Every compiled variant forced on a shape that leaves partial tiles and a partial
    K slab; the variants with direct 16-byte staging get extents that are multiples of 8."""
    for cfg in _catalogue_for(in_t):
        M, N, K = (304, 272, 200) if cfg in ALIGNED_ONLY else (300, 270, 200)
        for a_col, b_col in LAYOUTS:
            As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, a_col, b_col, seed=3)
            C, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, a_col, b_col, cfg=cfg)
            assert (desc["bm"], desc["bn"]) == (cfg[1], cfg[2])
            Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, a_col, b_col)
            check_tolerance(C, Cref, out_t, f"cfg={cfg} a_col={a_col} b_col={b_col}")


def test_aligned_variants_refuse_extents_that_are_not_multiples_of_8():
    for cfg in ALIGNED_ONLY:
        As, lda, Bs, ldb, _, _ = synth.operands(300, 270, 200, "bf16", seed=3)
        with pytest.raises(mh.GemmError, match="multiples of 8"):
            run_gpu(As, lda, Bs, ldb, 300, 270, 200, "bf16", "bf16", cfg=cfg)


@pytest.mark.parametrize("cfg", sorted(ALIGNED_ONLY))
@pytest.mark.parametrize("b_col", [False, True])
def test_aligned_variants_fall_back_on_misaligned_pointers(cfg, b_col):
    """Run-time fallback to the register-staged kernel when a base pointer is not
    16-byte aligned: same plan, still correct."""
    M, N, K = 264, 520, 136
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "bf16", False, b_col, seed=6)
    C, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, "bf16", "f32", False, b_col, cfg=cfg,
                           offset_a=1, offset_b=0)
    check_tolerance(C, oracle_ref(As, lda, Bs, ldb, M, N, K, "bf16", False, b_col), "f32")


W8_256 = (2, 256, 256, 32, 2, 4, 5, 1)
W8_128 = (2, 128, 128, 64, 2, 4, 5, 1)
W8_64 = (2, 64, 64, 128, 2, 4, 5, 1)


@pytest.mark.parametrize("in_t,out_t", [("bf16", "bf16"), ("f16", "f32"), ("bf16", "f32"), ("f16", "f16")])
@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
@pytest.mark.parametrize("cfg", [W8_256, W8_128, W8_64], ids=["256", "128", "64"])
def test_eight_wave_kernels_every_slab_count(in_t, out_t, a_col, b_col, cfg):
    """The eight-wave kernels keep a ring of five slabs (32 deep at 256 x 256, 64 deep at
    128 x 128) with four requested ahead; K from one partial slab to more than two trips
    round the ring, on a ragged grid, in every layout (K-contiguous operands read 16
    bytes a lane, M/N-contiguous ones through LDS transpose reads)."""
    M, N = 264, 520
    bk = cfg[3]
    for K in (8, bk, bk + 8, 3 * bk, 5 * bk, 5 * bk + 8, 10 * bk + 8):
        As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, a_col, b_col, seed=K)
        C, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, a_col, b_col, cfg=cfg)
        assert (desc["bm"], desc["bn"], desc["threads"]) == (cfg[1], cfg[2], 512)
        Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, a_col, b_col)
        check_tolerance(C, Cref, out_t, f"K={K} a_col={a_col} b_col={b_col}")


@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
@pytest.mark.parametrize("cfg", [W8_256, W8_128, W8_64], ids=["256", "128", "64"])
@pytest.mark.parametrize("out_t", ["f32", "bf16"])
def test_eight_wave_kernels_exact_integer_sums(a_col, b_col, cfg, out_t):
    """Dense integers in [-3, 3] over two full tiles in each direction (four at 128, eight at 64):
    every fp32 partial sum is exact, so the output must be the oracle's rounding bit
    for bit (for bf16 output: the oracle's round-to-nearest-even of the exact sum); a
    misplaced fragment, slab, wave block, K half or staged store changes it."""
    M, N, K = 512, 512, 512
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "bf16", a_col, b_col, dist="int", r=3, seed=21)
    C, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, "bf16", out_t, a_col, b_col, cfg=cfg)
    Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, "bf16", a_col, b_col)
    check_exact(raw, Cref, out_t, f"a_col={a_col} b_col={b_col}")


@pytest.mark.parametrize("cfg", [W8_256, W8_128, W8_64], ids=["256", "128", "64"])
@pytest.mark.parametrize("out_t", ["f32", "bf16"])
def test_eight_wave_kernels_unaligned_c(cfg, out_t):
    """C whose base or leading dimension is not 16-byte aligned takes the direct stores
    instead of the LDS-staged ones; guard bands check both paths write nothing else."""
    M, N, K = 264, 520, 136
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "bf16", seed=12)
    Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, "bf16")
    for offset_c, ldc in ((0, N), (1, N), (0, N + 4)):
        C, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, "bf16", out_t, ldc=ldc, cfg=cfg, offset_c=offset_c)
        check_tolerance(C, Cref, out_t, f"offset_c={offset_c} ldc={ldc}")


@pytest.mark.parametrize("out_t,ldc", [("f32", 4194304 - 64), ("f32", 4194304 + 8), ("bf16", 8388608 + 8)],
                         ids=["f32-below", "f32-above", "bf16-above"])
def test_staged_stores_long_rows_of_c(out_t, ldc):
    """The 256 x 256 tile's staged stores go through a buffer resource based at the
    wave's block of C, whose offsets must stay below 2^31 bytes; a C whose 128 rows of a
    block span more than that takes streaming global stores instead.  Just below the
    limit (offsets near 2^31) and above it (4.4 GB of C), both output types; the padding
    columns, checked on the device, must keep their sentinel."""
    M, N, K = 264, 264, 136
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "bf16", seed=31)
    Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, "bf16")
    eb = 4 if out_t == "f32" else 2
    print(f"[long rows] out={out_t} ldc={ldc} C bytes={M * ldc * eb}", flush=True)
    sent = SENTINEL32 if out_t == "f32" else SENTINEL16
    cbuf = torch.full((M, ldc), sent, dtype=torch.int32 if out_t == "f32" else torch.int16, device="cuda")
    A, B = As.cuda(), Bs.cuda()
    plan = mh.gemm_plan_config(M, N, K, lda, ldb, ldc, mh.DTYPE_OF[("bf16", out_t)], 0, W8_256)
    try:
        mh.gemm_run(plan, A, B, cbuf)
        torch.cuda.synchronize()
    finally:
        mh.gemm_destroy(plan)
    assert not bool((cbuf[:, N:] != sent).any()), "write into the padding columns of C"
    body = cbuf[:, :N].cpu().numpy()
    del cbuf
    torch.cuda.empty_cache()
    vals = body.view(np.float32).astype(np.float64) if out_t == "f32" else oracle.decode(body.view(np.uint16), out_t)
    check_tolerance(vals, Cref, out_t, f"ldc={ldc}")


def SKINNY(split):
    return (3, 16, 128, 32, 1, 4, 2, split)


@pytest.mark.parametrize("in_t,out_t", HALF_DTYPES)
def test_skinny_every_split_ragged(in_t, out_t):
    """At most 16 rows: K split across 1..16 workgroup chunks (the last ones partly or
    wholly past K), rows below 16, a last column block narrower than 128."""
    for M, N, K in [(1, 136, 200), (5, 1000, 1032), (16, 264, 4104), (16, 4096, 64)]:
        As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, seed=M + K)
        Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t)
        for split in (1, 2, 4, 8, 16):
            C, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, cfg=SKINNY(split))
            assert (desc["kind"], desc["split_k"]) == (mh.GEMM_KIND_SKINNY, split)
            check_tolerance(C, Cref, out_t, f"M={M} N={N} K={K} split={split}")


@pytest.mark.parametrize("out_t", ["bf16", "f32"])
def test_skinny_exact_integer_sums(out_t):
    """Integer inputs: every partial sum (per wave, per workgroup, across chunks) is exact,
    so the output is the oracle's rounding of the exact sum, bit for bit."""
    M, N, K = 16, 1024, 8192
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "bf16", dist="int", r=2, seed=4)
    Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, "bf16")
    for split in (1, 8):
        C, raw, _ = run_gpu(As, lda, Bs, ldb, M, N, K, "bf16", out_t, cfg=SKINNY(split))
        check_exact(raw, Cref, out_t)


def test_skinny_split_k_repeats_bit_for_bit():
    """The last workgroup of a column block adds the chunks' partials in chunk order,
    so repeated runs of one plan (which also re-arm the arrival counters) give the
    same bits; a second plan with its own workspace agrees."""
    w = synth.WORKLOADS["bf16_skinny"]
    As, lda, Bs, ldb, _, _ = synth.workload_operands(w)
    A, B = As.cuda(), Bs.cuda()
    code = mh.DTYPE_OF[(w.dtype, w.out)]
    outs = []
    for _ in range(2):
        plan = mh.gemm_plan(w.M, w.N, w.K, lda, ldb, w.N, code, 0)
        try:
            d = mh.gemm_plan_describe(plan)
            assert d["kind"] == mh.GEMM_KIND_SKINNY and d["split_k"] > 1 and d["workspace_bytes"] > 0
            for _ in range(3):
                C = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
                mh.gemm_run(plan, A, B, C)
                torch.cuda.synchronize()
                outs.append(C.cpu())
        finally:
            mh.gemm_destroy(plan)
    for o in outs[1:]:
        assert torch.equal(o.view(torch.int32), outs[0].view(torch.int32))
    rows = (0, 3)
    Cref = oracle_ref(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, rows=rows)
    check_tolerance(outs[0][rows[0]:rows[1]].double().numpy(), Cref, "f32", "skinny rows")


def test_skinny_falls_back_on_misaligned_pointers():
    M, N, K = 16, 1024, 2048
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "f16", seed=12)
    Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, "f16")
    for oa, ob in [(1, 0), (0, 3)]:
        C, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, "f16", "f32", cfg=SKINNY(4), offset_a=oa, offset_b=ob)
        check_tolerance(C, Cref, "f32", f"offsets {oa} {ob}")


@pytest.mark.parametrize("in_t,out_t", [("bf16", "bf16"), ("f16", "f32"), ("f32", "f32")])
def test_thousand_cubed_every_layout(in_t, out_t):
    M = N = K = 1000
    for a_col, b_col in LAYOUTS:
        As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, a_col, b_col, seed=1)
        C, raw, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, a_col, b_col)
        rows = (0, 70)
        Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, a_col, b_col, rows=rows)
        check_tolerance(C[rows[0]:rows[1]], Cref, out_t, f"a_col={a_col} b_col={b_col}")
        Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, a_col, b_col, rows=(M - 40, M))
        check_tolerance(C[M - 40:], Cref, out_t, f"last rows a_col={a_col} b_col={b_col}")


# ---- leading dimensions and alignment ------------------------------------------------------------

@pytest.mark.parametrize("in_t,out_t", ALL_DTYPES)
def test_padded_leading_dimensions(in_t, out_t):
    M, N, K = 200, 136, 264
    for a_col, b_col in LAYOUTS:
        lda = (M if a_col else K) + 24
        ldb = (K if b_col else N) + 8
        As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, a_col, b_col, lda=lda, ldb=ldb, seed=2)
        C, raw, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, a_col, b_col, ldc=N + 40)
        Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, a_col, b_col)
        check_tolerance(C, Cref, out_t, f"a_col={a_col} b_col={b_col}")


@pytest.mark.parametrize("in_t,out_t", ALL_DTYPES)
def test_misaligned_pointers_and_odd_leading_dimensions(in_t, out_t):
    M, N, K = 130, 97, 211
    for a_col, b_col in LAYOUTS:
        lda = (M if a_col else K) + 3
        ldb = (K if b_col else N) + 5
        As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, a_col, b_col, lda=lda, ldb=ldb, seed=4)
        C, raw, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, a_col, b_col, ldc=N + 1,
                            offset_a=1, offset_b=3, offset_c=1)
        Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, a_col, b_col)
        check_tolerance(C, Cref, out_t, f"a_col={a_col} b_col={b_col}")


# ---- bit-exact integer suites --------------------------------------------------------------------

@pytest.mark.parametrize("in_t,out_t", HALF_DTYPES)
@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
def test_exact_sparse_sums(in_t, out_t, a_col, b_col):
    """Entries in {-1, 0, 1}; B column j nonzero only where (k + j) % period == 0, so
    |C| <= ceil(K / period) is exact in the output type and every slab contributes."""
    M, N, K = 257, 190, 1000
    limit = 256 if out_t == "bf16" else 2048
    period = -(-K // limit)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, a_col, b_col, dist="sparse_pm1",
                                            period=period, seed=8)
    C, raw, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, a_col, b_col)
    Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, a_col, b_col)
    check_exact(raw, Cref, out_t)


@pytest.mark.parametrize("in_t,out_t", ALL_DTYPES)
def test_exact_dense_small_integers_rounded_once(in_t, out_t):
    """Dense integers in [-4, 4]: every fp32 partial sum is exact (|sum| <= 16K < 2^24),
    so the only rounding is the final cast: the output must equal the oracle's
    round-to-nearest-even of the exact sum, bit for bit."""
    for (M, N, K), cfg in [((320, 260, 1024), None), ((64, 64, 4096), None)]:
        for a_col, b_col in [(False, False), (False, True)]:
            As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, a_col, b_col, dist="int", r=4, seed=9)
            C, raw, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t, a_col, b_col, cfg=cfg)
            Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, in_t, a_col, b_col)
            check_exact(raw, Cref, out_t)


# ---- closed forms ------------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["f32_64", "f16_1024", "f16_1000", "f16_2048_nt", "bf16_skinny"])
def test_closed_forms_at_workload_shapes(name):
    w = synth.WORKLOADS[name]
    # all ones: C_ij = K exactly in every output type used
    As, lda, Bs, ldb, _, _ = synth.operands(w.M, w.N, w.K, w.dtype, w.a_col, w.b_col, dist="ones")
    C, raw, _ = run_gpu(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.out, w.a_col, w.b_col)
    assert np.all(C == w.K)
    # identity on the right (B = I when K == N): C = A exactly
    if w.K == w.N:
        As, lda, Bs, ldb, A, _ = synth.operands(w.M, w.N, w.K, w.dtype, w.a_col, w.b_col,
                                                dist="uniform", dist_b="identity", seed=1)
        C, raw, _ = run_gpu(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.out, w.a_col, w.b_col)
        assert np.array_equal(C, A.to(torch.float64).numpy())
    # permutation on the left (A = P when M == K): rows of B permuted exactly
    if w.M == w.K:
        As, lda, Bs, ldb, P, B = synth.operands(w.M, w.N, w.K, w.dtype, w.a_col, w.b_col,
                                                dist="perm", dist_b="uniform", seed=2)
        C, raw, _ = run_gpu(As, lda, Bs, ldb, w.M, w.N, w.K, w.dtype, w.out, w.a_col, w.b_col)
        p = P.to(torch.float64).numpy().argmax(axis=1)
        assert np.array_equal(C, B.to(torch.float64).numpy()[p])


# ---- degenerate extents ------------------------------------------------------------------------

@pytest.mark.parametrize("in_t,out_t", ALL_DTYPES)
def test_degenerate_extents(in_t, out_t):
    # M = 0 or N = 0: nothing is written (the guard bands check that)
    for M, N, K in [(0, 5, 7), (6, 0, 7), (0, 0, 0)]:
        As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t)
        C, raw, desc = run_gpu(As, max(lda, 1), Bs, max(ldb, 1), M, N, K, in_t, out_t, ldc=max(N, 1))
        assert desc["kind"] == mh.GEMM_KIND_NONE
    # K = 0: C is the empty sum, zero everywhere
    M, N = 33, 45
    empty = torch.zeros((0,), dtype=synth.TORCH_DTYPES[in_t])
    C, raw, desc = run_gpu(empty, 1, empty, N, M, N, 0, in_t, out_t, ldc=N + 3)
    assert np.all(C == 0)


def test_single_element_and_single_row():
    for in_t, out_t in ALL_DTYPES:
        for M, N, K in [(1, 1, 1), (1, 1, 4096), (1, 4096, 1), (4096, 1, 8), (1, 300, 700)]:
            As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, in_t, seed=M + N + K)
            C, raw, _ = run_gpu(As, lda, Bs, ldb, M, N, K, in_t, out_t)
            check_tolerance(C, oracle_ref(As, lda, Bs, ldb, M, N, K, in_t), out_t, f"{M}x{N}x{K}")


# ---- operands at addresses whose low 32 bits have bit 31 set --------------------------------
# The eight-wave kernels read their load origins through the first lane, 32 bits at a
# time; a low half with bit 31 set must not spill into the high half.  A is placed so
# that it starts 512 KiB below a 4 GiB boundary (low word 0xFFF80000, bit 31 set, and
# the operand crosses into the next 4 GiB), B at low word 0x80000100.

def _place(storage, low_word, keep):
    """Copy a CPU storage tensor into a fresh device buffer at the first address whose
    low 32 bits equal `low_word`; returns that address (the buffer is kept alive in
    `keep`)."""
    flat = storage.reshape(-1)
    nbytes = flat.numel() * flat.element_size()
    buf = torch.empty((1 << 32) + nbytes + 4096, dtype=torch.uint8, device="cuda")
    keep.append(buf)
    base = buf.data_ptr()
    off = (low_word - (base & 0xFFFFFFFF)) % (1 << 32)
    assert off + nbytes <= buf.numel()
    addr = base + off
    assert addr & 0xFFFFFFFF == low_word and addr % 16 == 0
    buf[off:off + nbytes].copy_(flat.contiguous().view(torch.uint8).to("cuda"))
    return addr


W8_CONFIGS = [(2, 256, 256, 32, 2, 4, 5, 1), (2, 128, 128, 64, 2, 4, 5, 1), (2, 64, 64, 128, 2, 4, 5, 1),
              (2, 128, 128, 64, 2, 4, 5, 2)]


@pytest.mark.parametrize("cfg", W8_CONFIGS)
@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
def test_operands_at_high_low_word(cfg, a_col, b_col):
    M, N, K = 512, 512, 1024
    print(f"[high low word] cfg={cfg} a_col={a_col} b_col={b_col}", flush=True)
    As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "bf16", a_col, b_col, dist="int", r=3, seed=31)
    keep = []
    try:
        a_addr = _place(As, 0xFFF80000, keep)
        b_addr = _place(Bs, 0x80000100, keep)
        C = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        layout = (mh.GEMM_A_COL if a_col else 0) | (mh.GEMM_B_COL if b_col else 0)
        plan = mh.gemm_plan_config(M, N, K, lda, ldb, N, mh.GEMM_BF16_F32, layout, cfg)
        try:
            mh.gemm_run(plan, a_addr, b_addr, C)
            torch.cuda.synchronize()
        finally:
            mh.gemm_destroy(plan)
        got = C.cpu().numpy()
    finally:
        del keep
        torch.cuda.empty_cache()
    Cref = oracle_ref(As, lda, Bs, ldb, M, N, K, "bf16", a_col, b_col)
    check_exact(got, Cref, "f32", f"cfg={cfg}")


def test_clock_probe_reads_a_plausible_clock():
    """The one-wave clock probe (a measurement helper): shader cycles over a 2 ms window
    of the 100 MHz real-time counter give a clock between 100 MHz and 3 GHz, and the
    window it reports is at least the one asked for."""
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    mh.gemm_clock_probe(out.data_ptr(), 200_000)
    torch.cuda.synchronize()
    cycles, ticks = (int(v) for v in out.cpu().tolist())
    assert ticks >= 200_000
    assert 100.0 <= 100.0 * cycles / ticks <= 3000.0, (cycles, ticks)


@pytest.mark.parametrize("a_col,b_col", LAYOUTS)
def test_fp32_vector_loads_at_edges(a_col, b_col):
    """The fp32 FMA tiles with 16-byte loads: extents that leave partial 4-element chunks
    at every edge (ld a multiple of 4, so the vector path is taken), exact integer
    products, each FMA tile forced."""
    for cfg in [(1, 32, 32, 32, 4, 1, 2, 1), (1, 64, 64, 16, 4, 1, 2, 1), (1, 128, 128, 16, 4, 1, 2, 1)]:
        for M, N, K in [(33, 35, 37), (130, 66, 18), (5, 7, 3)]:
            lda = ((M if a_col else K) + 3) // 4 * 4
            ldb = ((K if b_col else N) + 3) // 4 * 4
            As, lda, Bs, ldb, _, _ = synth.operands(M, N, K, "f32", a_col, b_col, lda=lda, ldb=ldb, dist="int", seed=M)
            C, raw, desc = run_gpu(As, lda, Bs, ldb, M, N, K, "f32", "f32", a_col, b_col, cfg=cfg)
            assert (desc["bm"], desc["kind"]) == (cfg[1], 1)
            check_exact(raw, oracle_ref(As, lda, Bs, ldb, M, N, K, "f32", a_col, b_col), "f32",
                        f"cfg={cfg} M={M} N={N} K={K}")

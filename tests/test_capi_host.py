"""Host-side checks of the C ABI that need no GPU: the library loads and exports every
function the header declares, arguments are validated, and the planner's choices
follow the pages' rules (LDS budget, grid geometry, per-shape regimes).  No kernel
is launched here."""
import ctypes
import os
import re

import pytest

import memory_hierarchy_optimisation_amd as mh
from oracle import formulas as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhgemm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("gemm_plan", "gemm_run", "gemm_destroy", "gemm_last_error",
                     "gemm_plan_describe", "gemm_plan_config"):
        assert required in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mh.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(lib, name), name
    assert set(_declared_functions()) == set(mh.EXPORTS)


def _plan(M, N, K, dtype, layout=0, lda=None, ldb=None, ldc=None, cfg=None):
    a_col, b_col = layout & 1, layout & 2
    lda = (M if a_col else K) if lda is None else lda
    ldb = (K if b_col else N) if ldb is None else ldb
    ldc = N if ldc is None else ldc
    p = mh.gemm_plan(M, N, K, lda, ldb, ldc, dtype, layout) if cfg is None else \
        mh.gemm_plan_config(M, N, K, lda, ldb, ldc, dtype, layout, cfg)
    try:
        return mh.gemm_plan_describe(p)
    finally:
        mh.gemm_destroy(p)


@pytest.mark.parametrize("args,msg", [
    ((4, 4, 4, 3, 4, 4, 0, 0), "lda"),
    ((4, 4, 4, 4, 3, 4, 0, 0), "ldb"),
    ((4, 4, 4, 4, 4, 3, 0, 0), "ldc"),
    ((4, 4, 4, 3, 4, 4, 0, 1), "lda"),          # column-major A needs lda >= M
    ((4, 4, 8, 8, 7, 4, 1, 2), "ldb"),          # column-major B needs ldb >= K
    ((-1, 4, 4, 4, 4, 4, 0, 0), "negative"),
    ((4, 4, 4, 4, 4, 4, 9, 0), "dtype"),
    ((4, 4, 4, 4, 4, 4, 0, 4), "layout"),
    ((1 << 31, 4, 4, 4, 4, 4, 0, 0), "2^31"),
])
def test_plan_rejects_invalid_arguments(args, msg):
    with pytest.raises(mh.GemmError) as e:
        mh.gemm_plan(*args)
    assert msg in str(e.value)


def test_run_rejects_null_plan_and_describe_null():
    lib = ctypes.CDLL(mh.LIB_PATH)
    lib.gemm_run.argtypes = [ctypes.c_void_p] * 5
    assert lib.gemm_run(None, None, None, None, None) == mh.GEMM_ERR_INVALID_ARG
    lib.gemm_plan_describe.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    assert lib.gemm_plan_describe(None, None) == mh.GEMM_ERR_INVALID_ARG
    lib.gemm_destroy.argtypes = [ctypes.c_void_p]
    lib.gemm_destroy(None)  # NULL is ignored


def test_empty_extents_plan_to_no_kernel():
    for M, N, K in [(0, 3, 3), (3, 0, 3), (3, 3, 0), (0, 0, 0)]:
        d = _plan(M, N, K, mh.GEMM_BF16_BF16, lda=max(K, 1), ldb=max(N, 1), ldc=max(N, 1))
        assert d["kind"] == mh.GEMM_KIND_NONE


def test_leading_dimension_only_checked_when_operand_has_elements():
    d = _plan(5, 5, 0, mh.GEMM_F16_F16, lda=0, ldb=0, ldc=5)
    assert d["kind"] == mh.GEMM_KIND_NONE


def test_the_pages_two_by_two_example():
    """64 x 64 as tiles of 32 x 32 -> a 2 x 2 grid ("CUDA tile", 2.1)."""
    d = _plan(64, 64, 64, mh.GEMM_F32_F32)
    assert (d["kind"], d["bm"], d["bn"]) == (mh.GEMM_KIND_FMA, 32, 32)
    assert (d["grid_x"], d["grid_y"]) == F.launch_grid(64, 64, 32, 32) == (2, 2)


@pytest.mark.parametrize("M,N,K,dtype,layout", [
    (1024, 1024, 1024, mh.GEMM_F16_F16, 0),
    (1000, 1000, 1000, mh.GEMM_F16_F16, 0),
    (2048, 2048, 2048, mh.GEMM_F16_F32, 2),
    (4096, 4096, 4096, mh.GEMM_BF16_BF16, 0),
    (16, 8192, 8192, mh.GEMM_BF16_F32, 0),
    (333, 777, 5, mh.GEMM_F32_F32, 3),
])
def test_grid_and_lds_follow_the_formulas(M, N, K, dtype, layout):
    d = _plan(M, N, K, dtype, layout)
    assert (d["grid_x"], d["grid_y"]) == F.launch_grid(M, N, d["bm"], d["bn"])
    elem = 4 if dtype == mh.GEMM_F32_F32 else 2
    formula = F.smem_bytes(d["bm"], d["bn"], d["bk"], elem, d["stages"])
    if d["kind"] == mh.GEMM_KIND_MFMA:
        assert d["lds_bytes"] == formula          # swizzled, no padding
    elif d["kind"] == mh.GEMM_KIND_SKINNY:
        # no staged slabs: LDS holds the four waves' 16 x BN fp32 partials and a flag
        assert d["lds_bytes"] == 4 * 16 * d["bn"] * 4 + 16
        assert d["grid_z"] == d["split_k"]
    else:
        assert formula <= d["lds_bytes"] <= formula * 1.2   # k-rows padded by 4 floats
    assert d["lds_bytes"] <= 160 * 1024
    assert d["cus"] > 0


def test_per_shape_regimes():
    """Small grids take small tiles to fill the compute units; the largest square
    shape takes the largest tile ("GPU Kernel 的 Tile、Grid、Wave 与 Launch Overhead",
    per-shape choices: fewer, bigger workers once there are enough of them)."""
    small = _plan(1024, 1024, 1024, mh.GEMM_F16_F16)
    mid = _plan(2048, 2048, 2048, mh.GEMM_F16_F32, 2)
    big = _plan(4096, 4096, 4096, mh.GEMM_BF16_BF16)
    assert small["bm"] * small["bn"] < mid["bm"] * mid["bn"] < big["bm"] * big["bn"]
    for d in (small, mid, big):
        assert d["grid_x"] * d["grid_y"] >= 256


def test_forced_configuration_checks():
    d = _plan(300, 300, 300, mh.GEMM_BF16_BF16, cfg=(2, 128, 128, 64, 2, 2, 2, 1))
    assert (d["bm"], d["bn"], d["bk"]) == (128, 128, 64)
    with pytest.raises(mh.GemmError, match="no compiled variant"):
        _plan(300, 300, 300, mh.GEMM_BF16_BF16, cfg=(2, 96, 96, 64, 2, 2, 2, 1))
    with pytest.raises(mh.GemmError, match="input type"):
        _plan(300, 300, 300, mh.GEMM_F32_F32, cfg=(2, 128, 128, 64, 2, 2, 2, 1))
    with pytest.raises(mh.GemmError, match="input type"):
        _plan(300, 300, 300, mh.GEMM_BF16_F32, cfg=(1, 64, 64, 16, 4, 1, 2, 1))


SKINNY_WS = lambda gn, split: (0 if split == 1 else (gn * 4 + 255) // 256 * 256 + split * gn * 16 * 128 * 4)


@pytest.mark.parametrize("M,N,K,split", [
    (16, 8192, 8192, 4),     # 64 column blocks x 4 chunks = one workgroup per compute unit
    (4, 256, 8192, 16),      # two column blocks: the largest split
    (16, 8192, 1024, 2),     # K chunks stop at 512
    (1, 32768, 4096, 1),     # 256 column blocks already fill the chip
])
def test_skinny_products_split_k_across_workgroups(M, N, K, split):
    d = _plan(M, N, K, mh.GEMM_BF16_F32)
    gn = (N + 127) // 128
    assert d["kind"] == mh.GEMM_KIND_SKINNY
    assert (d["bm"], d["bn"], d["split_k"]) == (16, 128, split)
    assert (d["grid_x"], d["grid_y"], d["grid_z"]) == (1, gn, split)
    assert d["workspace_bytes"] == SKINNY_WS(gn, split)


@pytest.mark.parametrize("M,N,K,dtype,layout,lda,ldb", [
    (17, 8192, 8192, mh.GEMM_BF16_F32, 0, None, None),   # more than 16 rows
    (16, 8192, 8196, mh.GEMM_BF16_F32, 0, 8200, None),   # K not a multiple of 8
    (16, 8190, 8192, mh.GEMM_BF16_F32, 0, None, None),   # N not a multiple of 8
    (16, 8192, 8192, mh.GEMM_BF16_F32, 1, 16, None),     # column-major A
    (16, 8192, 8192, mh.GEMM_BF16_F32, 2, None, 8192),   # column-major B
    (16, 8192, 8192, mh.GEMM_F32_F32, 0, None, None),    # fp32 inputs
])
def test_skinny_variant_only_where_it_applies(M, N, K, dtype, layout, lda, ldb):
    kw = {}
    if lda is not None:
        kw["lda"] = lda
    if ldb is not None:
        kw["ldb"] = ldb
    d = _plan(M, N, K, dtype, layout, **kw)
    assert d["kind"] != mh.GEMM_KIND_SKINNY


def test_forced_skinny_configurations():
    for split in (1, 2, 4, 8, 16):
        d = _plan(8, 1024, 4096, mh.GEMM_F16_F16, cfg=(3, 16, 128, 32, 1, 4, 2, split))
        assert (d["kind"], d["split_k"], d["grid_z"]) == (mh.GEMM_KIND_SKINNY, split, split)
        assert d["workspace_bytes"] == SKINNY_WS(8, split)
    with pytest.raises(mh.GemmError, match="at most 16 rows"):
        _plan(17, 1024, 4096, mh.GEMM_F16_F16, cfg=(3, 16, 128, 32, 1, 4, 2, 2))
    with pytest.raises(mh.GemmError, match="multiples of 8"):
        _plan(8, 1024, 4092, mh.GEMM_F16_F16, cfg=(3, 16, 128, 32, 1, 4, 2, 2))
    with pytest.raises(mh.GemmError, match="no compiled variant"):
        _plan(8, 1024, 4096, mh.GEMM_F16_F16, cfg=(3, 16, 128, 32, 1, 4, 2, 3))


def test_last_error_clears_on_success():
    with pytest.raises(mh.GemmError):
        mh.gemm_plan(4, 4, 4, 1, 4, 4, 0, 0)
    assert "lda" in mh.gemm_last_error()
    p = mh.gemm_plan(4, 4, 4, 4, 4, 4, 0, 0)
    mh.gemm_destroy(p)
    assert mh.gemm_last_error() == ""


def test_one_hip_runtime_in_the_process():
    """The library shares torch's HIP runtime instead of mapping a second one."""
    assert len(mh.hip_runtimes_mapped()) == 1


def test_transpose_argument_checks():
    """gemm_transpose validates before touching a device; empty extents are a no-op."""
    mh.gemm_transpose(0, 0, 0, 5, 5, 1, 4, stream=0)
    mh.gemm_transpose(0, 0, 4, 0, 1, 4, 2, stream=0)
    for args, msg in [((16, 16, 2, 2, 2, 2, 8), "elem_bytes"), ((16, 16, 2, 4, 3, 2, 4), "ld_in"),
                      ((16, 16, 2, 4, 4, 1, 4), "ld_out"), ((18, 16, 2, 2, 2, 2, 4), "misaligned"),
                      ((0, 16, 2, 2, 2, 2, 4), "NULL"), ((16, 16, -1, 2, 2, 2, 4), "negative"),
                      ((16, 16, 1 << 32, 2, 2, 1 << 32, 4), r"2\^31")]:
        with pytest.raises(mh.GemmError, match=msg):
            mh.gemm_transpose(*args, stream=0)


@pytest.mark.parametrize("M,N,K,split", [(512, 512, 8192, 4), (256, 256, 16384, 8), (768, 512, 4096, 2),
                                         (512, 512, 512, 1), (1024, 1024, 1024, 1), (4096, 4096, 4096, 1)])
def test_eight_wave_split_k_for_small_grids(M, N, K, split):
    """Too few workers: a grid of eight-wave tiles that covers at most half of the 256
    compute units gets K split by the smallest power of two (at most 8) that covers
    three quarters of them, with at least four K slabs per chunk; the plan then owns
    split x M x N fp32 partials."""
    d = _plan(M, N, K, mh.GEMM_BF16_BF16)
    assert d["split_k"] == split and d["grid_z"] == split
    assert d["workspace_bytes"] == (split * M * N * 4 if split > 1 else 0)


def test_forced_eight_wave_split_needs_two_slabs_per_chunk():
    with pytest.raises(mh.GemmError, match="two K slabs"):
        _plan(512, 512, 1024, mh.GEMM_BF16_BF16, cfg=(2, 64, 64, 128, 2, 4, 5, 8))
    d = _plan(512, 512, 2048, mh.GEMM_BF16_BF16, cfg=(2, 64, 64, 128, 2, 4, 5, 8))
    assert d["split_k"] == 8


def test_clock_probe_argument_checks():
    """gemm_clock_probe validates before touching a device."""
    for out, ticks, msg in ((0, 100, "NULL"), (12, 100, "misaligned"), (16, 0, "ticks"),
                            (16, 10 ** 9 + 1, "ticks")):
        with pytest.raises(mh.GemmError, match=msg):
            mh.gemm_clock_probe(out, ticks, stream=0)


def test_noalloc_rejects_a_workspace_beyond_its_scratch(tmp_path):
    """A plan whose split-K workspace exceeds the 16 MiB scratch array is refused with a
    message before anything reaches a device (the tuned table forces such a plan:
    2048 x 2048 partials of fp32 in 8 chunks are 128 MiB)."""
    table = tmp_path / "tune.txt"
    table.write_text("2048 2048 8192 8192 2048 2048 4 0 | 2 128 128 64 2 4 5 8 | 1.0\n")
    assert mh.gemm_tune_load(str(table)) == 1
    try:
        with pytest.raises(mh.GemmError, match="exceeds the scratch array"):
            mh.gemm_run_noalloc(2048, 2048, 8192, 8192, 2048, 2048, mh.GEMM_BF16_F32, 0, 256, 256, 256, stream=0)
        with pytest.raises(mh.GemmError, match="lda"):
            mh.gemm_run_noalloc(16, 16, 16, 8, 16, 16, mh.GEMM_BF16_F32, 0, 256, 256, 256, stream=0)
    finally:
        mh.gemm_tune_clear()


def _report_registers():
    """Registers per lane of every kernel in the build's resource report, keyed by name:
    architected VGPRs in 4-register granules, then AGPRs, the total in 8-register
    allocation granules."""
    path = os.path.join(ROOT, "_build", "resource_usage.txt")
    out = {}
    for line in open(path):
        name, *kv = line.split()
        f = dict(x.split("=", 1) for x in kv)
        v, a = int(f["vgpr"]), int(f["agpr"])
        out[name] = ((v + 3) // 4 * 4 + a + 7) // 8 * 8
    return out


def _family(cfg):
    """Pattern of the mangled kernel names that implement a catalogue entry."""
    kind, bm, bn, bk, _, _, stages, split = cfg
    if kind == mh.GEMM_KIND_FMA:
        return rf"fma_gemmILi{bm}E"
    if kind == mh.GEMM_KIND_SKINNY:
        return r"skinny_gemm"
    if bk == 16:
        return r"mfma32_gemm"
    if stages == 5:
        return rf"w8_gemm.*Tile{bm}E"
    return rf"mfma_gemmINS_\d+Half\w+ELi{bm}ELi{bn}E"


def test_occupancy_filter_uses_the_build_report():
    """The planner's register counts are the largest of each kernel family in the
    compiler's resource report of this build (not constants)."""
    report = _report_registers()
    regs = mh.gemm_catalogue_registers()
    cat = mh.gemm_catalogue()
    assert len(regs) == len(cat)
    for cfg, r in zip(cat, regs):
        family = [v for k, v in report.items() if re.search(_family(cfg), k)]
        assert family, cfg
        assert r == max(family), (cfg, r, max(family))

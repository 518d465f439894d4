"""The pages' formulas against the numbers the pages print, and against brute-force counts."""
import ast
import itertools
import os

import pytest

from oracle import formulas as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.txt")


def _rows():
    rows = []
    with open(GOLDEN, encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            fn, args, expected, tol, source = [p.strip() for p in line.split("|", 4)]
            rows.append((fn, args, expected, float(tol), source))
    return rows


@pytest.mark.parametrize("fn,args,expected,tol,source", _rows())
def test_printed_numbers(fn, args, expected, tol, source):
    got = getattr(F, fn)(*eval(args, {"__builtins__": {}}, {}))
    want = ast.literal_eval(expected)
    if isinstance(want, tuple):
        assert tuple(got) == want, source
    elif tol == 0:
        assert got == want, source
    else:
        assert abs(got - want) <= tol, (got, want, source)


def test_golden_file_is_not_empty():
    assert len(_rows()) >= 20


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (8, 8, 8), (4, 9, 2)])
def test_naive_load_count_is_two_per_multiply_add(M, N, K):
    loads = F.count_naive_loads(M, N, K)
    assert loads == 2 * M * N * K
    # fp16: FLOPs over bytes of those loads is the naive 0.5 FLOP/B
    assert F.gemm_flops(M, N, K) / (loads * 2) == F.naive_intensity(2)


@pytest.mark.parametrize("m,n,k,b,bk", [(16, 16, 16, 4, 4), (32, 32, 24, 8, 8), (24, 16, 12, 8, 3),
                                        (64, 64, 64, 32, 32)])
def test_tiled_traffic_matches_two_mnk_over_b(m, n, k, b, bk):
    """Counting loads of the block-tiled loop nest reproduces 2mnk/b (qian.cx)
    for any K slab depth: the K split does not change the total."""
    assert F.count_tiled_loads(m, n, k, b, b, bk) == F.tiled_traffic_elements(m, n, k, b)


def test_k_split_leaves_traffic_unchanged():
    base = F.count_tiled_loads(32, 32, 48, 8, 8, 48)
    for bk in (1, 2, 3, 4, 6, 8, 12, 16, 24):
        assert F.count_tiled_loads(32, 32, 48, 8, 8, bk) == base


@pytest.mark.parametrize("TM,TN", [(4, 4), (8, 4), (4, 16), (16, 16)])
def test_tiled_intensity_matches_counted_traffic(TM, TN):
    """One output tile over full K: 2*TM*TN*K FLOP over (TM+TN)*K loaded elements."""
    M, N, K = TM, TN, 12
    loads = F.count_tiled_loads(M, N, K, TM, TN, 4)
    assert F.gemm_flops(M, N, K) / (loads * 2) == pytest.approx(F.tiled_intensity(TM, TN, 2), rel=1e-12)


def test_ragged_tiles_count_only_in_range_elements():
    # 10x10x10 with 4x4 tiles and BK=3: each in-range element of A is loaded once per column
    # tile and each in-range element of B once per row tile.
    M = N = K = 10
    gm, gn = F.launch_grid(M, N, 4, 4)
    assert (gm, gn) == (3, 3)
    assert F.count_tiled_loads(M, N, K, 4, 4, 3) == M * K * gn + K * N * gm


def test_compulsory_intensity_matches_square_limit():
    # With M = N = K = n and elem e, 2n^3 / (3 n^2 e) = 2n / (3e).
    for n, e in itertools.product((64, 1024, 4096), (2, 4)):
        assert F.compulsory_intensity(n, n, n, e) == pytest.approx(2 * n / (3 * e))
    # bf16 4096^3 with a bf16 output: 1365.33 FLOP/B
    assert F.compulsory_intensity(4096, 4096, 4096, 2) == pytest.approx(1365.333, rel=1e-5)


def test_algorithmic_bytes_of_each_workload():
    assert F.algorithmic_bytes(64, 64, 64, 4, 4, 4) == 49152
    assert F.algorithmic_bytes(1024, 1024, 1024, 2, 2, 2) == 6291456
    assert F.algorithmic_bytes(2048, 2048, 2048, 2, 2, 4) == 33554432
    assert F.algorithmic_bytes(4096, 4096, 4096, 2, 2, 2) == 100663296
    assert F.algorithmic_bytes(16, 8192, 8192, 2, 2, 4) == 135004160


def test_roofline_is_min_of_roofs():
    assert F.roofline(2.5e15, 8e12, 15.9) == pytest.approx(15.9 * 8e12)
    assert F.roofline(2.5e15, 8e12, 1365) == 2.5e15
    assert F.ridge_point(2.5e15, 8e12) == pytest.approx(312.5)


def test_square_tile_intensity_is_the_tiled_intensity_of_a_square_tile():
    """The qian.cx note's 0.5*b (b x b output tile, fp16) and the T_M x T_N formula of
    "Tiling 策略与内存层次优化" are the same quantity for square tiles; both equal the
    FLOPs over the counted loads of the tiled loop nest."""
    for b in (1, 2, 4, 8, 16, 32, 64, 128, 256):
        for e in (2, 4):
            assert F.tiled_intensity_square(b, e) == pytest.approx(F.tiled_intensity(b, b, e), rel=1e-15)
    for b in (2, 4, 8):
        M = N = 2 * b
        K = 6
        loads = F.count_tiled_loads(M, N, K, b, b, 3)
        assert F.gemm_flops(M, N, K) / (loads * 2) == pytest.approx(F.tiled_intensity_square(b, 2), rel=1e-12)


def test_square_tile_scales_naive_intensity_by_b():
    # qian.cx: tiling with b x b output tiles divides the loads by b, so the intensity
    # is b times the naive one.
    for b in (1, 3, 16, 249):
        assert F.tiled_intensity_square(b, 2) == pytest.approx(b * F.naive_intensity(2))


def test_compute_intensity_of_counted_loop_nests():
    """FLOPs over counted bytes: the naive nest gives 1/elem, the tiled one the tile formula."""
    M, N, K = 3, 5, 7
    assert F.compute_intensity(F.gemm_flops(M, N, K), F.count_naive_loads(M, N, K) * 2) == 0.5
    loads = F.count_tiled_loads(8, 8, 12, 8, 8, 4)
    assert F.compute_intensity(F.gemm_flops(8, 8, 12), loads * 4) == pytest.approx(F.tiled_intensity(8, 8, 4))


def test_roofline_switches_roofs_at_the_printed_ridge():
    """Below the ridge the bandwidth roof binds, at and above it the compute roof.
    A100: ridge 156 FLOP/B ("Tiling 策略与内存层次优化"); V100-class: b = 249 reaches the
    compute roof and b = 248 does not (qian.cx: b >= 2P/B)."""
    assert F.roofline(312e12, 2e12, 155) == pytest.approx(155 * 2e12)
    assert F.roofline(312e12, 2e12, 155) < 312e12
    assert F.roofline(312e12, 2e12, F.ridge_point(312e12, 2e12)) == 312e12
    assert F.roofline(112e12, 900e9, F.tiled_intensity_square(248)) < 112e12
    assert F.roofline(112e12, 900e9, F.tiled_intensity_square(249)) == 112e12
    b_min = F.tile_needed_for_ridge(112e12, 900e9, 2)
    assert F.roofline(112e12, 900e9, F.tiled_intensity_square(b_min)) == pytest.approx(112e12)
    # monotone in intensity, flat above the ridge
    vals = [F.roofline(2.5e15, 8e12, ai) for ai in (1, 10, 100, 312.5, 1000, 1365)]
    assert vals == sorted(vals) and vals[-1] == vals[-2] == vals[-3] == 2.5e15

"""The pages' traffic, intensity and resource formulas, plus brute-force counters.

TEST INFRASTRUCTURE ONLY (same import rule as the rest of ``oracle/``).

Each closed form below restates a formula from the pages; each ``count_*``
function walks the corresponding loop nest and counts element loads one by one,
so the closed forms are checked by enumeration rather than by retyping them.

Sources (page title, section):
  [T] "Tiling 策略与内存层次优化": roofline review; how tiling raises intensity;
      constraint 1 (shared memory), constraint 2 (registers), constraint 3
      (occupancy); launch configuration in the scheduling stage; the GEMM
      walk-through (naive step).
  [Q] qian.cx note on tiled vs naive matrix multiply: naive 0.5 FLOP/B, tiled
      traffic 2mnk/b and intensity 0.5*b, the K split l, the V100-class example.
  [W] "GPU Kernel 的 Tile、Grid、Wave 与 Launch Overhead": register-limited CTAs
      per SM, wave count, the 1024^2 wide-tile intensity example.
  [C] "CUDA tile": 2.1 block tiling (64x64 matrix cut into 2x2 tiles of 32).
"""
from math import ceil, floor


# ---- roofline [T roofline review; Q roofline paragraph] ---------------------------

def compute_intensity(flops, nbytes):
    return flops / nbytes


def ridge_point(peak_flops, bandwidth):
    """FLOP per byte a kernel needs to leave the bandwidth roof [T]."""
    return peak_flops / bandwidth


def roofline(peak_flops, bandwidth, intensity):
    """Attainable FLOP/s: min(peak, intensity * bandwidth)."""
    return min(peak_flops, intensity * bandwidth)


# ---- GEMM traffic and intensity --------------------------------------------------

def gemm_flops(M, N, K):
    """One multiply and one add per (i, j, k)."""
    return 2 * M * N * K


def naive_element_flops(K):
    """[T, walk-through step 1]: one output element costs 2K FLOP."""
    return 2 * K


def naive_element_bytes(K, elem):
    """[T, step 1]: it reads a row of A and a column of B, 2K elements."""
    return 2 * K * elem


def naive_intensity(elem):
    """[T step 1; Q]: 2K FLOP over 2K*elem bytes -> 1/elem (0.5 for fp16)."""
    return 1.0 / elem


def compulsory_intensity(M, N, K, elem_in, elem_out=None):
    """2MNK over the bytes of A, B and C each moved once.

    [T, "how tiling raises intensity"] prints 2MNK / ((MK+KN+MN)*elem) under the
    label "naive"; numerically it is the every-operand-once (compulsory) traffic,
    which is how it is used here: the algorithmic bytes of one GEMM call.
    """
    elem_out = elem_in if elem_out is None else elem_out
    return gemm_flops(M, N, K) / ((M * K + K * N) * elem_in + M * N * elem_out)


def algorithmic_bytes(M, N, K, elem_a, elem_b, elem_c):
    return M * K * elem_a + K * N * elem_b + M * N * elem_c


def tiled_intensity(TM, TN, elem):
    """[T]: 2*TM*TN / ((TM+TN)*elem) for one TM x TN output tile."""
    return 2.0 * TM * TN / ((TM + TN) * elem)


def tiled_traffic_elements(m, n, k, b):
    """[Q]: (m/b)(n/b) tiles each reading 2*b*k elements -> 2mnk/b."""
    return 2 * m * n * k / b


def tiled_intensity_square(b, elem=2):
    """[Q]: the naive 1/elem scaled by b (0.5*b for fp16)."""
    return b / elem


def tile_needed_for_ridge(peak_flops, bandwidth, elem=2):
    """[Q]: 0.5*b >= P/B  <=>  b >= 2P/B (fp16)."""
    return elem * peak_flops / bandwidth


# ---- resources [T constraints 1-3; W] ---------------------------------------------

def smem_bytes(BM, BN, BK, elem, stages):
    """[T constraint 1]: (BM*BK + BK*BN) * elem * stages."""
    return (BM * BK + BK * BN) * elem * stages


def blocks_per_sm_by_smem(capacity_bytes, tile_bytes):
    return floor(capacity_bytes / tile_bytes)


def ctas_per_sm_by_regs(regs_per_thread, warps_per_cta, threads_per_warp, regs_per_sm):
    """[W, SM section]: floor(regs_per_SM / (regs * warps * threads))."""
    return regs_per_sm // (regs_per_thread * warps_per_cta * threads_per_warp)


def waves(ctas, sms, ctas_per_sm):
    """[W, wave section]: CTAs / (SMs * CTAs per SM)."""
    return ctas / (sms * ctas_per_sm)


def launch_grid(M, N, BM, BN):
    """[T, scheduling stage]: (ceil(M/BM), ceil(N/BN))."""
    return (ceil(M / BM), ceil(N / BN))


# ---- brute-force counters (walk the loop nests, count loads) ----------------------

def count_naive_loads(M, N, K):
    """One thread per output element, each multiply-add loads one A and one B element."""
    loads = 0
    for _i in range(M):
        for _j in range(N):
            for _k in range(K):
                loads += 2
    return loads


def count_tiled_loads(M, N, K, BM, BN, BK):
    """Elements copied from global memory by the block-tiled loop nest.

    For every output tile and every K slab, the in-range part of the A tile
    (BM x BK) and of the B tile (BK x BN) is loaded once; out-of-range positions
    are zero-filled and cost no load ("CUDA tile", 4, boundary checks).
    """
    loads = 0
    gm, gn = launch_grid(M, N, BM, BN)
    for bm in range(gm):
        for bn in range(gn):
            for k0 in range(0, K, BK):
                for r in range(BM):
                    for c in range(BK):
                        if bm * BM + r < M and k0 + c < K:
                            loads += 1
                for r in range(BK):
                    for c in range(BN):
                        if k0 + r < K and bn * BN + c < N:
                            loads += 1
    return loads

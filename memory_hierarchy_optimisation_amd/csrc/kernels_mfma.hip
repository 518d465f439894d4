// kernels_mfma.hip -- fp16 / bf16 tiled GEMM on gfx950 matrix cores (fp32 accumulation).
//
// Three tiling levels ("Tiling 策略与内存层次优化", multi-level tiling: block tile ->
// warp tile -> MMA instruction; "寄存器Tiling", 1.1 and 3.1 for the AMD wave64 form):
//   * a workgroup owns a BM x BN tile of C and walks K in slabs of BK = 64;
//   * each slab of A (BM x 64) and B (64 x BN) is staged in LDS, double-buffered:
//     the global loads of slab t+1 are issued before the matrix instructions of
//     slab t and written to the other LDS buffer afterwards, so one barrier per slab
//     suffices (same page, double buffering; the single-buffer form needs two);
//   * each wave owns a (BM/WM) x (BN/WN) register tile of 16 x 16 fp32 accumulator
//     blocks fed by v_mfma_f32_16x16x32_{bf16,f16}.
//
// Operands keep their storage orientation in LDS.  A K-contiguous operand (row-major
// A, column-major B) is stored as rows of 64 k-values; a fragment is one 16-byte LDS
// read per lane.  An M- or N-contiguous operand (column-major A, row-major B) is
// stored as 64 k-rows of BM (or BN) values and its fragments come from two LDS
// transpose reads per lane, so no operand is transposed in registers.
//
// Global loads are 16 bytes per lane along the contiguous dimension ("Tiling 策略与
// 内存层次优化", memory coalescing and the 128-bit vector loads of the walk-through).
// Loads that would leave the matrix are replaced by zeros ("CUDA tile", 4: zero
// padding is the identity of the sum); a chunk that straddles the edge is read
// element by element.  LDS chunk positions are XOR-swizzled by row (same page, bank
// conflicts and swizzling: bank index = (row XOR column) mod banks).
#include "device.h"

namespace mhg {
namespace {

constexpr int BK = 64;

// Byte offset of 16-byte chunk `chunk` (0..7) of row `row` in a K-contiguous tile
// (rows of 64 two-byte elements = 128 bytes).
__device__ __forceinline__ int kc_off(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7)) << 4);
}

// Byte offset of chunk `chunk` of k-row `krow` in an M/N-contiguous tile with NCH
// chunks per row.  A transpose read touches 4 consecutive k-rows at the same
// columns; the XOR spreads those rows over distinct 32-byte bank groups.
template <int NCH>
__device__ __forceinline__ int mn_off(int krow, int chunk) {
  return krow * (NCH * 16) + ((chunk ^ (((krow & 3) << 1) & (NCH - 1))) << 4);
}

// One operand's share of a K slab: R rows of C-tile extent (BM for A, BN for B),
// K-contiguous (KC) or not, staged by NT threads.
template <int R, bool KC, int NT>
struct OperandTile {
  static constexpr int CHUNKS = R * BK / 8;
  static constexpr int PER = CHUNKS / NT;
  static constexpr int NCH = R / 8;
  static_assert(CHUNKS % NT == 0, "tile chunks must divide evenly over the threads");
  static_assert(KC || (NCH & (NCH - 1)) == 0, "chunks per row must be a power of two");

  u32x4 reg[PER];

  // Issue the global loads of the slab starting at k0 into registers.
  //   g: storage; ld: leading dimension; mn_lim: M (A) or N (B); base: m0 or n0.
  __device__ __forceinline__ void load(const uint16_t *__restrict__ g, int64_t ld, int64_t mn_lim,
                                       int64_t K, int base, int k0, int vec) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = threadIdx.x + i * NT;
      int64_t row, col, row_lim, col_lim;
      if (KC) {
        row = base + q / 8;           // m or n
        col = k0 + 8 * (q % 8);       // k, contiguous
        row_lim = mn_lim;
        col_lim = K;
      } else {
        row = k0 + q / NCH;           // k
        col = base + 8 * (q % NCH);   // m or n, contiguous
        row_lim = K;
        col_lim = mn_lim;
      }
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row < row_lim) {
        const uint16_t *src = g + row * ld + col;
        if (vec && col + 8 <= col_lim) {
          v = *reinterpret_cast<const u32x4 *>(src);
        } else if (col < col_lim) {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) h[e] = (col + e < col_lim) ? src[e] : 0u;
          v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
        }
      }
      reg[i] = v;
    }
  }

  __device__ __forceinline__ void store(char *lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = threadIdx.x + i * NT;
      const int off = KC ? kc_off(q / 8, q % 8) : mn_off<NCH>(q / NCH, q % NCH);
      *reinterpret_cast<u32x4 *>(lds + off) = reg[i];
    }
  }

  // Operand fragment of 16 rows (tile-local r0 ..) for k-step s (k = 32s .. 32s+31).
  __device__ __forceinline__ u32x4 frag(const char *lds, int r0, int s, int lane) const {
    if (KC) {
      const int row = r0 + (lane & 15);
      const int chunk = 4 * s + (lane >> 4);
      return *reinterpret_cast<const u32x4 *>(lds + kc_off(row, chunk));
    } else {
      const int L = lane & 15, grp = lane >> 4;
      const int col = r0 + 4 * (L & 3);
      const int chunk = col >> 3, byte = (col & 7) * 2;
      const int krow = 32 * s + 8 * grp + (L >> 2);
      u32x2 lo = lds_read_tr16(lds + mn_off<NCH>(krow, chunk) + byte);
      u32x2 hi = lds_read_tr16(lds + mn_off<NCH>(krow + 4, chunk) + byte);
      return u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  }
};

template <class H, int BM, int BN, int WM, int WN, bool A_KC, bool B_KC>
__global__ void __launch_bounds__(WM * WN * 64)
mfma_gemm(LaunchArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int A_BYTES = BM * BK * 2, B_BYTES = BN * BK * 2, STAGE = A_BYTES + B_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  int tm, tn;
  tile_of(blockIdx.x, p.gm, p.gn, p.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const uint16_t *__restrict__ A = static_cast<const uint16_t *>(p.A);
  const uint16_t *__restrict__ B = static_cast<const uint16_t *>(p.B);

  OperandTile<BM, A_KC, NT> ta;
  OperandTile<BN, B_KC, NT> tb;
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = int((p.K + BK - 1) / BK);
  ta.load(A, p.lda, p.M, p.K, m0, 0, p.vec_a);
  tb.load(B, p.ldb, p.N, p.K, n0, 0, p.vec_b);
  ta.store(smem);
  tb.store(smem + A_BYTES);
  __syncthreads();

  for (int t = 0; t < KT; ++t) {
    const char *cur = smem + (t & 1) * STAGE;
    const bool more = t + 1 < KT;
    if (more) {
      ta.load(A, p.lda, p.M, p.K, m0, (t + 1) * BK, p.vec_a);
      tb.load(B, p.ldb, p.N, p.K, n0, (t + 1) * BK, p.vec_b);
    }
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      u32x4 af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) af[i] = ta.frag(cur, wm * WTM + i * 16, s, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) bf[j] = tb.frag(cur + A_BYTES, wn * WTN + j * 16, s, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16(H{}, af[i], bf[j], acc[i][j]);
    }
    if (more) {
      char *nxt = smem + ((t + 1) & 1) * STAGE;
      ta.store(nxt);
      tb.store(nxt + A_BYTES);
    }
    __syncthreads();
  }

  // Epilogue: lane holds rows 4*(lane/16) .. +3 of column lane%16 of each block.
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * WTN + j * 16 + (lane & 15);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * WTM + i * 16 + 4 * (lane >> 4) + r;
        if (row < p.M && col < p.N) store_out(p.C, row * p.ldc + col, acc[i][j][r], p.out_code);
      }
    }
}

template <class H, int BM, int BN, int WM, int WN>
hipError_t launch_tiles(const LaunchArgs &p, hipStream_t s) {
  const dim3 grid(unsigned(p.gm) * unsigned(p.gn)), block(WM * WN * 64);
  if (!p.a_col && !p.b_col)
    hipLaunchKernelGGL((mfma_gemm<H, BM, BN, WM, WN, true, false>), grid, block, 0, s, p);
  else if (!p.a_col && p.b_col)
    hipLaunchKernelGGL((mfma_gemm<H, BM, BN, WM, WN, true, true>), grid, block, 0, s, p);
  else if (p.a_col && !p.b_col)
    hipLaunchKernelGGL((mfma_gemm<H, BM, BN, WM, WN, false, false>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((mfma_gemm<H, BM, BN, WM, WN, false, true>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <class H>
hipError_t launch_typed(int launcher, const LaunchArgs &p, hipStream_t s) {
  switch (launcher) {
    case L_MFMA_64x64: return launch_tiles<H, 64, 64, 2, 2>(p, s);
    case L_MFMA_128x128: return launch_tiles<H, 128, 128, 2, 2>(p, s);
    case L_MFMA_256x128: return launch_tiles<H, 256, 128, 2, 2>(p, s);
    case L_MFMA_256x256: return launch_tiles<H, 256, 256, 2, 4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_mfma(int launcher, const LaunchArgs &p, hipStream_t s) {
  if (p.in_code == E_BF16) return launch_typed<HalfBF16>(launcher, p, s);
  if (p.in_code == E_F16) return launch_typed<HalfF16>(launcher, p, s);
  return hipErrorInvalidValue;
}

}  // namespace mhg

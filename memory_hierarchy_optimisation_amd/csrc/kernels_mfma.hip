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
// padding is the identity of the sum) without branching; operands that cannot take
// 16-byte loads use an instantiation that reads element by element.  LDS chunk positions are XOR-swizzled by row (same page, bank
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

// Buffer resource over `bytes` bytes from `base` (raw addressing, stride 0).  Loads
// whose offset lies at or beyond the range return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Offset that a load takes for a chunk outside the matrix: beyond every resource range.
constexpr uint32_t kOutside = 0x80000000u;

// One operand's share of a K slab: R rows of C-tile extent (BM for A, BN for B),
// K-contiguous (KC) or not, staged by NT threads.  Chunk q of the slab is 8
// consecutive elements along the storage's contiguous dimension.
//
// VEC: 16-byte buffer loads.  The host selects it only when the base is 16-byte
// aligned and the leading dimension and the contiguous extent are multiples of 8
// elements, so every chunk lies wholly inside or wholly outside the matrix.  Each
// slab gets a buffer resource whose base is the slab's origin in storage; a chunk's
// byte offset from that origin does not change from slab to slab, and a chunk
// outside the matrix takes the out-of-range offset, which loads zeros.  No branch or
// select touches the loaded value, so the compiler can leave the load in flight
// across the matrix instructions and wait only before the LDS store.
// !VEC: element loads with per-element masks (unaligned or ragged storage).
template <int R, bool KC, int NT, bool VEC>
struct OperandTile {
  static constexpr int CHUNKS = R * BK / 8;
  static constexpr int PER = CHUNKS / NT;
  static constexpr int NCH = R / 8;
  static_assert(CHUNKS % NT == 0, "tile chunks must divide evenly over the threads");
  static_assert(KC || (NCH & (NCH - 1)) == 0, "chunks per row must be a power of two");

  u32x4 reg[PER];
  const uint16_t *base;   // operand storage
  int64_t ld;
  int64_t mn_lim, K;
  int mn0;                // m0 or n0 of this workgroup
  uint32_t off[VEC ? PER : 1];   // byte offset of chunk i from the slab origin
  bool mn_ok[VEC ? PER : 1];     // chunk i's m (or n) coordinate lies inside the matrix

  __device__ __forceinline__ OperandTile(const uint16_t *g, int64_t ld_, int64_t mn_lim_, int64_t K_, int mn0_)
      : base(g), ld(ld_), mn_lim(mn_lim_), K(K_), mn0(mn0_) {
    if (VEC) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int q = threadIdx.x + i * NT;
        // KC: storage row = m (or n), column = k.  Else: storage row = k, column = m (n).
        const int r = KC ? q / 8 : q / NCH;
        const int c = KC ? 8 * (q % 8) : 8 * (q % NCH);
        off[i] = uint32_t((int64_t(r) * ld + c) * 2);
        mn_ok[i] = KC ? (mn0 + r < mn_lim) : (mn0 + c < mn_lim);
      }
    }
  }

  // k coordinate within the slab of chunk i
  __device__ __forceinline__ int kin(int i) const {
    const int q = threadIdx.x + i * NT;
    return KC ? 8 * (q % 8) : q / NCH;
  }

  // Issue the global loads of the slab starting at k0 into registers.  `full`: the
  // whole slab lies inside the matrix (uniform across the workgroup).
  __device__ __forceinline__ void load(int k0, bool full) {
    if (VEC) {
      // slab origin: (row m0/n0, column k0) for KC storage, (row k0, column m0/n0) otherwise
      const uint16_t *origin = KC ? base + int64_t(mn0) * ld + k0 : base + int64_t(k0) * ld + mn0;
      const __amdgpu_buffer_rsrc_t rsrc = make_rsrc(origin, 0x7fffffffu);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const bool in = full || (mn_ok[i] && k0 + kin(i) < K);
        reg[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, in ? off[i] : kOutside, 0, 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int q = threadIdx.x + i * NT;
        const int64_t row = KC ? mn0 + q / 8 : k0 + q / NCH;
        const int64_t col = KC ? k0 + 8 * (q % 8) : mn0 + 8 * (q % NCH);
        const int64_t row_lim = KC ? mn_lim : K, col_lim = KC ? K : mn_lim;
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const bool in = row < row_lim && col + e < col_lim;
          const uint16_t *src = in ? base + row * ld + col + e : base;
          const uint32_t x = *src;
          h[e] = in ? x : 0u;
        }
        reg[i] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      }
    }
  }

  __device__ __forceinline__ void store(char *lds) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int q = threadIdx.x + i * NT;
      const int off_lds = KC ? kc_off(q / 8, q % 8) : mn_off<NCH>(q / NCH, q % NCH);
      *reinterpret_cast<u32x4 *>(lds + off_lds) = reg[i];
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

template <class H, int BM, int BN, int WM, int WN, bool A_KC, bool B_KC, bool VEC>
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

  OperandTile<BM, A_KC, NT, VEC> ta(A, p.lda, p.M, p.K, m0);
  OperandTile<BN, B_KC, NT, VEC> tb(B, p.ldb, p.N, p.K, n0);
  // Slabs lie wholly inside the matrix when the tile does and k0 + BK <= K.
  const bool tile_in = (m0 + BM <= p.M) && (n0 + BN <= p.N);
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int KT = int((p.K + BK - 1) / BK);
  ta.load(0, tile_in && BK <= p.K);
  tb.load(0, tile_in && BK <= p.K);
  ta.store(smem);
  tb.store(smem + A_BYTES);
  __syncthreads();

  for (int t = 0; t < KT; ++t) {
    const char *cur = smem + (t & 1) * STAGE;
    const bool more = t + 1 < KT;
    if (more) {
      const int k1 = (t + 1) * BK;
      const bool full = tile_in && k1 + BK <= p.K;
      ta.load(k1, full);
      tb.load(k1, full);
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
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16(H{}, bf[j], af[i], acc[i][j]);
    }
    if (more) {
      char *nxt = smem + ((t + 1) & 1) * STAGE;
      ta.store(nxt);
      tb.store(nxt + A_BYTES);
    }
    __syncthreads();
  }

  // The instructions take B's fragment first and A's second, so each accumulator holds
  // the transposed 16 x 16 block: lane l has C[row 16 i + l % 16][cols 16 j + 4 (l / 16) .. +3]
  // of the wave's block, four consecutive columns written as one 8- or 16-byte piece.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t row = m0 + wm * WTM + i * 16 + (lane & 15);
    if (row >= p.M) continue;
    // With an epilogue, the row block's bias and prior values are requested before its
    // first store (a load may not move above a store that might alias it).
    if (p.epi) {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t col = n0 + wn * WTN + j * 16 + 4 * (lane >> 4);
        if (col < p.N) acc[i][j] = epilogue4(p, acc[i][j], row, col, p.N - col);
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * WTN + j * 16 + 4 * (lane >> 4);
      const int64_t n_in = p.N - col;
      if (n_in <= 0) continue;
      store_out4(p.C, row * p.ldc + col, acc[i][j], p.out_code, p.c_vec && n_in >= 4, int(n_in));
    }
  }
}

template <class H, int BM, int BN, int WM, int WN>
hipError_t launch_tiles(const LaunchArgs &p, hipStream_t s) {
  const dim3 grid(unsigned(p.gm) * unsigned(p.gn)), block(WM * WN * 64);
  // 16-byte staging needs both operands aligned with contiguous extents that are
  // multiples of 8 elements (so chunks never straddle an edge).
  const int64_t a_ext = p.a_col ? p.M : p.K, b_ext = p.b_col ? p.K : p.N;
  const bool vec = p.vec_a && p.vec_b && a_ext % 8 == 0 && b_ext % 8 == 0;
#define MHG_LAUNCH(AK, BKC, V) \
  hipLaunchKernelGGL((mfma_gemm<H, BM, BN, WM, WN, AK, BKC, V>), grid, block, 0, s, p)
  if (vec) {
    if (!p.a_col && !p.b_col) MHG_LAUNCH(true, false, true);
    else if (!p.a_col && p.b_col) MHG_LAUNCH(true, true, true);
    else if (p.a_col && !p.b_col) MHG_LAUNCH(false, false, true);
    else MHG_LAUNCH(false, true, true);
  } else {
    if (!p.a_col && !p.b_col) MHG_LAUNCH(true, false, false);
    else if (!p.a_col && p.b_col) MHG_LAUNCH(true, true, false);
    else if (p.a_col && !p.b_col) MHG_LAUNCH(false, false, false);
    else MHG_LAUNCH(false, true, false);
  }
#undef MHG_LAUNCH
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

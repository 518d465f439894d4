// kernels_mfma32.hip -- fp32 tiled GEMM on the gfx950 matrix cores
// (v_mfma_f32_32x32x2_f32, fp32 products accumulated in fp32).
//
// The fp32 counterpart of the register-tiled kernel of "CUDA tile", 2.2 (a workgroup
// tile of C, K walked in slabs through shared memory, a register tile per worker),
// with the register level done by matrix instructions as "寄存器Tiling", 3.1 describes
// for AMD's wave64 parts:
//   * a workgroup of four waves owns a 128 x 128 tile of C and walks K in 16-deep
//     slabs, double-buffered in LDS through registers: the global loads of slab t+1
//     are issued before the matrix instructions of slab t and written to the other
//     buffer after them, one barrier a slab;
//   * each wave owns a 64 x 64 register tile, 2 x 2 blocks of 32 x 32;
//   * both operands sit in LDS k-major, [k][m] and [k][n], so the operand of one
//     instruction (lane l: element l % 32 of k-row l / 32) is 32 consecutive floats of
//     two k-rows; each k-row is padded by 32 floats, which puts those two rows on
//     opposite halves of the banks;
//   * the product is computed transposed (B's block as the instruction's first
//     operand), so that a lane's accumulators are four consecutive columns of one row
//     of C and go out as 16-byte stores.
// Global loads are 16-byte chunks of four elements along the contiguous dimension of
// each operand's storage; a K-contiguous operand (row-major A, column-major B) is
// written to LDS element by element (transposed), an M/N-contiguous one as whole
// chunks.  Chunks outside the matrix read zeros (the additive identity, "CUDA tile",
// 4) through an offset beyond the buffer resource; operands whose storage does not
// allow 16-byte chunks use an instantiation that loads element by element.
#include "device.h"

namespace mhg {
namespace f32mfma {

constexpr int BM = 128, BN = 128, BK = 16, NT = 256;
constexpr int PAD = 32;              // floats added to each LDS k-row
constexpr int SA = BM + PAD, SB = BN + PAD;
constexpr uint32_t kOut = 0x80000000u;

__device__ __forceinline__ f32x16 mfma(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}

// One operand's BK x R slab (R = BM or BN along m or n).  KC: storage rows are m (or
// n) with k contiguous; else storage rows are k with m (or n) contiguous.  Chunk q of
// the slab is four consecutive elements of one storage row.
template <int R, bool KC, bool VEC>
struct Slab {
  static constexpr int CHUNKS = R * BK / 4;
  static constexpr int PER = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0, "slab chunks must divide over the threads");
  f32x4 v[PER];
  const float *base;
  int64_t ld, mn_lim, K;
  int mn0;

  __device__ __forceinline__ Slab(const float *g, int64_t ld_, int64_t mn_lim_, int64_t K_, int mn0_)
      : base(g), ld(ld_), mn_lim(mn_lim_), K(K_), mn0(mn0_) {}

  // (m or n within the tile, k within the slab) of chunk i's first element
  __device__ __forceinline__ void coords(int i, int &r, int &kk) const {
    const int q = threadIdx.x + NT * i;
    if (KC) {
      r = q % R;
      kk = 4 * (q / R);
    } else {
      kk = q / (R / 4);
      r = 4 * (q % (R / 4));
    }
  }

  __device__ __forceinline__ void load(int64_t k0) {
    if (VEC) {
      // The host allows this only when every chunk lies wholly inside or wholly
      // outside the matrix and the slab's byte span is below 2^31.
      const float *origin = KC ? base + int64_t(mn0) * ld + k0 : base + k0 * ld + mn0;
      const __amdgpu_buffer_rsrc_t rs = rsrc_of(origin);
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int r, kk;
        coords(i, r, kk);
        const bool in = mn0 + r < mn_lim && k0 + kk < K;
        const uint32_t off = uint32_t(KC ? (int64_t(r) * ld + kk) * 4 : (int64_t(kk) * ld + r) * 4);
        v[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, in ? off : kOut, 0, 0));
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        int r, kk;
        coords(i, r, kk);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t mn = mn0 + r + (KC ? 0 : e), k = k0 + kk + (KC ? e : 0);
          v[i][e] = mn < mn_lim && k < K ? base[KC ? mn * ld + k : k * ld + mn] : 0.0f;
        }
      }
    }
  }

  // Into an LDS buffer laid out [k][R + PAD].
  __device__ __forceinline__ void store(float *lds, int stride) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      int r, kk;
      coords(i, r, kk);
      if (KC) {
#pragma unroll
        for (int e = 0; e < 4; ++e) lds[(kk + e) * stride + r] = v[i][e];
      } else {
        *reinterpret_cast<f32x4 *>(&lds[kk * stride + r]) = v[i];
      }
    }
  }
};

template <bool A_COL, bool B_COL, bool VEC_A, bool VEC_B>
__global__ void __launch_bounds__(NT) mfma32_gemm(LaunchArgs p) {
  __shared__ __attribute__((aligned(16))) float As[2][BK * SA];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK * SB];
  int tm, tn;
  tile_of(blockIdx.x, p.gm, p.gn, p.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int wm = wave >> 1, wn = wave & 1;
  // A is K-contiguous when row-major, B when column-major.
  Slab<BM, !A_COL, VEC_A> sa(static_cast<const float *>(p.A), p.lda, p.M, p.K, m0);
  Slab<BN, B_COL, VEC_B> sb(static_cast<const float *>(p.B), p.ldb, p.N, p.K, n0);
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int64_t nk = (p.K + BK - 1) / BK;
  sa.load(0);
  sb.load(0);
  sa.store(As[0], SA);
  sb.store(Bs[0], SB);
  __syncthreads();
  const int kl = lane >> 5, ml = lane & 31;
  for (int64_t t = 0; t < nk; ++t) {
    const int cur = int(t & 1);
    const bool more = t + 1 < nk;
    if (more) {
      sa.load((t + 1) * BK);
      sb.load((t + 1) * BK);
    }
    const float *a = As[cur] + wm * 64 + ml;
    const float *b = Bs[cur] + wn * 64 + ml;
#pragma unroll
    for (int kp = 0; kp < BK / 2; ++kp) {
      const int k = 2 * kp + kl;
      float af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = a[k * SA + 32 * i];
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = b[k * SB + 32 * j];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma(bf[j], af[i], acc[i][j]);
    }
    if (more) {
      sa.store(As[cur ^ 1], SA);
      sb.store(Bs[cur ^ 1], SB);
    }
    __syncthreads();
  }

  // acc[i][j] holds the transposed 32 x 32 block: element r of lane l is
  // C[row 64 wm + 32 i + l % 32][col 64 wn + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4].
  const bool c_vec = p.c_vec != 0;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t row = m0 + wm * 64 + 32 * i + ml;
    if (row >= p.M) continue;
    f32x4 out[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n0 + wn * 64 + 32 * j + 8 * q + 4 * kl;
        out[j][q] = f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        // With an epilogue, the row block's bias and prior values are read before its
        // first store (a load may not move above a store that might alias it).
        if (p.epi && col < p.N) out[j][q] = epilogue4(p, out[j][q], row, col, p.N - col);
      }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = n0 + wn * 64 + 32 * j + 8 * q + 4 * kl;
        const int64_t n_in = p.N - col;
        if (n_in <= 0) continue;
        store_out4(p.C, row * p.ldc + col, out[j][q], p.out_code, c_vec && n_in >= 4, int(n_in));
      }
  }
}

#define MHG_F32_INST(AC, BC)                                      \
  template __global__ void mfma32_gemm<AC, BC, true, true>(LaunchArgs);   \
  template __global__ void mfma32_gemm<AC, BC, true, false>(LaunchArgs);  \
  template __global__ void mfma32_gemm<AC, BC, false, true>(LaunchArgs);  \
  template __global__ void mfma32_gemm<AC, BC, false, false>(LaunchArgs);
MHG_F32_INST(false, false)
MHG_F32_INST(false, true)
MHG_F32_INST(true, false)
MHG_F32_INST(true, true)
#undef MHG_F32_INST

// 16-byte chunks are allowed when the base is 16-byte aligned, the leading dimension
// and the contiguous extent are multiples of 4 elements (so every chunk is wholly
// inside or outside), and a slab's byte span stays below 2^31.
bool vec_ok(const void *base, int64_t ld, int64_t contiguous_extent, int64_t rows_in_slab) {
  return reinterpret_cast<uintptr_t>(base) % 16 == 0 && ld % 4 == 0 && contiguous_extent % 4 == 0 &&
         rows_in_slab * ld * 4 < (int64_t(1) << 31);
}

template <bool AC, bool BC>
hipError_t launch_layout(const LaunchArgs &p, hipStream_t s) {
  const bool va = vec_ok(p.A, p.lda, AC ? p.M : p.K, AC ? BK : BM);
  const bool vb = vec_ok(p.B, p.ldb, BC ? p.K : p.N, BC ? BN : BK);
  const dim3 grid(static_cast<unsigned>(p.gm) * static_cast<unsigned>(p.gn)), block(NT);
  if (va && vb) hipLaunchKernelGGL((mfma32_gemm<AC, BC, true, true>), grid, block, 0, s, p);
  else if (va) hipLaunchKernelGGL((mfma32_gemm<AC, BC, true, false>), grid, block, 0, s, p);
  else if (vb) hipLaunchKernelGGL((mfma32_gemm<AC, BC, false, true>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((mfma32_gemm<AC, BC, false, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace f32mfma

hipError_t launch_mfma32(const LaunchArgs &p, hipStream_t s) {
  if (p.in_code != E_F32) return hipErrorInvalidValue;
  if (!p.a_col && !p.b_col) return f32mfma::launch_layout<false, false>(p, s);
  if (!p.a_col && p.b_col) return f32mfma::launch_layout<false, true>(p, s);
  if (p.a_col && !p.b_col) return f32mfma::launch_layout<true, false>(p, s);
  return f32mfma::launch_layout<true, true>(p, s);
}

}  // namespace mhg

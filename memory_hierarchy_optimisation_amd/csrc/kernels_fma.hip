// kernels_fma.hip -- fp32 tiled GEMM on the vector ALUs, and the zero fill for K = 0.
//
// The shape is the register-tiled kernel of "CUDA tile", 2.2, written for 64-lane
// waves: a workgroup of (BM/TM) x (BN/TN) lanes owns a BM x BN tile of C and walks K
// in slabs of BK; every lane accumulates a TM x TN block of C in registers as an
// outer product of a TM-vector of A and a TN-vector of B per k ("寄存器Tiling", 1.1:
// the register level of the three tiling levels).  Slabs are double-buffered in LDS
// (one barrier per slab).  Both tiles are stored k-major so that a lane's TM (TN)
// operand values are contiguous in LDS and come back as 16-byte reads; each k-row
// is padded by four floats ("CUDA tile", 4, padding against bank conflicts).
// Out-of-range loads are zero ("CUDA tile", 4: 0 is the identity of the sum) and
// stores are masked.
//
// Global loads: with 16-byte aligned operands whose leading dimensions are multiples
// of four floats (VEC), each lane loads 16-byte chunks of four consecutive elements
// along the operand's contiguous dimension, consecutive lanes consecutive chunks (the
// 128-bit coalesced loads of "Tiling 策略与内存层次优化", step 4); a chunk that
// crosses an edge of the matrix is loaded element by element.  Otherwise every lane
// loads single elements, consecutive lanes consecutive addresses.
#include "device.h"

namespace mhg {
namespace {

template <int BM, int BN, int BK, int TM, int TN, bool A_COL, bool B_COL, bool VEC>
__global__ void __launch_bounds__((BM / TM) * (BN / TN))
fma_gemm(LaunchArgs p) {
  constexpr int TX = BN / TN, TY = BM / TM, NT = TX * TY;
  constexpr int AP = BM + 4, BP = BN + 4;
  constexpr int A_PER = BM * BK / NT, B_PER = BK * BN / NT;
  static_assert((BM * BK) % NT == 0 && (BK * BN) % NT == 0, "slab must divide over the lanes");
  static_assert(!VEC || (A_PER % 4 == 0 && B_PER % 4 == 0), "16-byte chunks must divide over the lanes");
  __shared__ __attribute__((aligned(16))) float As[2][BK][AP];
  __shared__ __attribute__((aligned(16))) float Bs[2][BK][BP];

  int tm, tn;
  tile_of(blockIdx.x, p.gm, p.gn, p.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int tx = threadIdx.x % TX, ty = threadIdx.x / TX;
  const float *__restrict__ A = static_cast<const float *>(p.A);
  const float *__restrict__ B = static_cast<const float *>(p.B);

  // Element e of the A slab -> (r, c) = (row of the C tile, k within the slab),
  // numbered so that consecutive lanes read consecutive addresses of the storage.
  auto a_rc = [](int e, int &r, int &c) {
    if (A_COL) { c = e / BM; r = e % BM; } else { r = e / BK; c = e % BK; }
  };
  auto b_rc = [](int e, int &r, int &c) {  // r: column of the C tile, c: k
    if (B_COL) { r = e / BK; c = e % BK; } else { c = e / BN; r = e % BN; }
  };

  float ra[A_PER], rb[B_PER];
  // VEC: chunk e of four consecutive elements of the contiguous dimension -> the
  // tile position (r, c) of its first element.
  auto a_chunk = [](int e, int &r, int &c) {
    if (A_COL) { c = e / (BM / 4); r = 4 * (e % (BM / 4)); } else { r = e / (BK / 4); c = 4 * (e % (BK / 4)); }
  };
  auto b_chunk = [](int e, int &r, int &c) {
    if (B_COL) { r = e / (BK / 4); c = 4 * (e % (BK / 4)); } else { c = e / (BN / 4); r = 4 * (e % (BN / 4)); }
  };
  // Four elements starting at src, the first `n` of them inside the matrix.
  auto load4 = [](const float *src, int n, float *dst) {
    if (n >= 4) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(src);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = v[e];
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = e < n ? src[e] : 0.f;
    }
  };
  auto load_vec = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PER / 4; ++i) {
      int r, c;
      a_chunk(int(threadIdx.x) + i * NT, r, c);
      const int64_t gm = m0 + r, gk = k0 + c;
      // the chunk runs along k (row-major A) or along m (column-major A)
      const int64_t n = A_COL ? (gk < p.K ? p.M - gm : 0) : (gm < p.M ? p.K - gk : 0);
      load4(A + (A_COL ? gk * p.lda + gm : gm * p.lda + gk), int(n < 4 ? n : 4), &ra[4 * i]);
    }
#pragma unroll
    for (int i = 0; i < B_PER / 4; ++i) {
      int r, c;
      b_chunk(int(threadIdx.x) + i * NT, r, c);
      const int64_t gn = n0 + r, gk = k0 + c;
      const int64_t n = B_COL ? (gn < p.N ? p.K - gk : 0) : (gk < p.K ? p.N - gn : 0);
      load4(B + (B_COL ? gn * p.ldb + gk : gk * p.ldb + gn), int(n < 4 ? n : 4), &rb[4 * i]);
    }
  };
  auto store_vec = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER / 4; ++i) {
      int r, c;
      a_chunk(int(threadIdx.x) + i * NT, r, c);
      if (A_COL) {
        *reinterpret_cast<f32x4 *>(&As[buf][c][r]) = f32x4{ra[4 * i], ra[4 * i + 1], ra[4 * i + 2], ra[4 * i + 3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) As[buf][c + e][r] = ra[4 * i + e];
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER / 4; ++i) {
      int r, c;
      b_chunk(int(threadIdx.x) + i * NT, r, c);
      if (!B_COL) {
        *reinterpret_cast<f32x4 *>(&Bs[buf][c][r]) = f32x4{rb[4 * i], rb[4 * i + 1], rb[4 * i + 2], rb[4 * i + 3]};
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) Bs[buf][c + e][r] = rb[4 * i + e];
      }
    }
  };
  auto load_el = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      int r, c;
      a_rc(int(threadIdx.x) + i * NT, r, c);
      const int64_t gm = m0 + r, gk = k0 + c;
      ra[i] = (gm < p.M && gk < p.K) ? A[A_COL ? gk * p.lda + gm : gm * p.lda + gk] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      int r, c;
      b_rc(int(threadIdx.x) + i * NT, r, c);
      const int64_t gn = n0 + r, gk = k0 + c;
      rb[i] = (gn < p.N && gk < p.K) ? B[B_COL ? gn * p.ldb + gk : gk * p.ldb + gn] : 0.f;
    }
  };
  auto store_el = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      int r, c;
      a_rc(int(threadIdx.x) + i * NT, r, c);
      As[buf][c][r] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      int r, c;
      b_rc(int(threadIdx.x) + i * NT, r, c);
      Bs[buf][c][r] = rb[i];
    }
  };

  auto load = [&](int k0) {
    if constexpr (VEC) load_vec(k0); else load_el(k0);
  };
  auto store = [&](int buf) {
    if constexpr (VEC) store_vec(buf); else store_el(buf);
  };

  float acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = 0.f;

  const int KT = int((p.K + BK - 1) / BK);
  load(0);
  store(0);
  __syncthreads();
  for (int t = 0; t < KT; ++t) {
    const int cur = t & 1;
    const bool more = t + 1 < KT;
    if (more) load((t + 1) * BK);
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float a[TM], b[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) a[i] = As[cur][k][ty * TM + i];
#pragma unroll
      for (int j = 0; j < TN; ++j) b[j] = Bs[cur][k][tx * TN + j];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = __builtin_fmaf(a[i], b[j], acc[i][j]);
    }
    if (more) store(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t row = m0 + ty * TM + i;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t col = n0 + tx * TN + j;
      if (row < p.M && col < p.N)
        store_out(p.C, row * p.ldc + col, p.epi ? epilogue1(p, acc[i][j], row, col) : acc[i][j], p.out_code);
    }
  }
}

template <int BM, int BN, int BK, int TM, int TN, bool VEC>
void launch_fma_layout(const LaunchArgs &p, hipStream_t s) {
  const dim3 grid(unsigned(p.gm) * unsigned(p.gn)), block((BM / TM) * (BN / TN));
  if (!p.a_col && !p.b_col)
    hipLaunchKernelGGL((fma_gemm<BM, BN, BK, TM, TN, false, false, VEC>), grid, block, 0, s, p);
  else if (!p.a_col && p.b_col)
    hipLaunchKernelGGL((fma_gemm<BM, BN, BK, TM, TN, false, true, VEC>), grid, block, 0, s, p);
  else if (p.a_col && !p.b_col)
    hipLaunchKernelGGL((fma_gemm<BM, BN, BK, TM, TN, true, false, VEC>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((fma_gemm<BM, BN, BK, TM, TN, true, true, VEC>), grid, block, 0, s, p);
}

// 16-byte chunks need 16-byte aligned operands with leading dimensions that are
// multiples of four floats (vec_a, vec_b: checked by gemm_run for fp32 inputs).
template <int BM, int BN, int BK, int TM, int TN>
hipError_t launch_fma_tiles(const LaunchArgs &p, hipStream_t s) {
  if (p.vec_a && p.vec_b) launch_fma_layout<BM, BN, BK, TM, TN, true>(p, s);
  else launch_fma_layout<BM, BN, BK, TM, TN, false>(p, s);
  return hipGetLastError();
}

// C = 0 for K = 0 (the empty sum), any output type.
// K = 0: every element is the empty sum, 0, passed through the epilogue when there
// is one (then C = act(beta * C + bias)).
__global__ void fill_zero(LaunchArgs p) {
  const int64_t total = p.M * p.N;
  for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += int64_t(gridDim.x) * blockDim.x) {
    const int64_t i = e / p.N, j = e % p.N;
    store_out(p.C, i * p.ldc + j, p.epi ? epilogue1(p, 0.f, i, j) : 0.f, p.out_code);
  }
}

}  // namespace

hipError_t launch_fma(int launcher, const LaunchArgs &p, hipStream_t s) {
  switch (launcher) {
    case L_FMA_32: return launch_fma_tiles<32, 32, 32, 2, 2>(p, s);
    case L_FMA_64: return launch_fma_tiles<64, 64, 16, 4, 4>(p, s);
    case L_FMA_128: return launch_fma_tiles<128, 128, 16, 8, 8>(p, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fill(const LaunchArgs &p, hipStream_t s) {
  const int64_t total = p.M * p.N;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_zero, dim3(unsigned(std::max<int64_t>(blocks, 1))), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace mhg

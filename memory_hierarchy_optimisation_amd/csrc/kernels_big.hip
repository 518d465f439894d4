// kernels_big.hip -- fp16 / bf16 GEMM for large problems with row-major A: 256 x 256
// workgroup tiles, four waves of 128 x 128 register tiles.
//
// The three tiling levels of "Tiling 策略与内存层次优化" (multi-level tiling) sized for
// gfx950:
//   * workgroup tile 256 x 256: tile intensity 2*256*256 / (512*2) = 128 FLOP/B (same
//     page, how tiling raises intensity), the largest whose two 64-deep slabs
//     (2 x 64 KiB) fit the 160 KB LDS (constraint 1);
//   * four waves, one per SIMD, each owning a 128 x 128 block of C: 256 fp32
//     accumulators per lane (in AGPRs), the largest register tile the 512-entry
//     register file allows ("寄存器Tiling", 1.3: registers bound the tile), and the
//     one that reads the fewest LDS bytes per matrix instruction (each 16 x 32 operand
//     fragment feeds 8 instructions);
//   * v_mfma_f32_32x32x16_{bf16,f16}: a wave's 128 x 128 block is 4 x 4 accumulators
//     of 32 x 32 (16 fp32 each).  Sixteen large accumulators keep the compiler's
//     register allocation stable across the K loop (64 accumulators of 16 x 16 made
//     it shuffle accumulator registers every iteration).  The instruction is fed B's
//     fragment as its first operand and A's as its second, so it accumulates the
//     transposed block: a lane then holds four consecutive columns of one row of C and
//     the epilogue writes 8- or 16-byte pieces instead of single elements.
// Both operands sit in LDS K-contiguous, so every fragment is one 16-byte LDS read per
// lane.  Row-major B (N-contiguous in memory) is transposed in registers while it is
// staged: each lane loads an 8 x 8 block (8 k-rows of 8 n-values) and repacks it into
// 8 n-rows of 8 k-values before the LDS store.
//
// Pipeline per 64-deep slab t (LDS double buffer, register-staged global loads):
//   read fragments of k-step 1        | matrix instructions of k-step 0
//   store slab t+1 (loaded during t-1) to the other LDS buffer; load slab t+2
//   first half of k-step 1's matrix instructions
//   wait for this wave's LDS operations; barrier
//   read fragments of slab t+1, k-step 0 | second half of k-step 1
// so the LDS reads after the barrier overlap matrix instructions.  The barrier is an
// s_barrier after an explicit LDS wait: the C++ block barrier would also wait for the
// global loads of slab t+2, which are meant to stay in flight across it.
//
// Edges: loads outside the matrix read zeros through buffer-resource range checks
// ("CUDA tile", 4: zero is the identity of the sum); stores are masked.  The kernel
// requires 16-byte aligned operands with leading dimensions and contiguous extents
// that are multiples of 8 elements (checked by the host).
#include <type_traits>

#include "device.h"

namespace mhg {
namespace big {

constexpr int BM = 256, BN = 256, BK = 64, NT = 256;
constexpr int WTM = 128, WTN = 128;
constexpr int FM = 8, FN = 8;   // operand fragments per 32-deep k-step: 4 row blocks x 2 k-halves
constexpr int TILE_BYTES = 256 * BK * 2;      // one operand's slab: 32 KiB
constexpr int STAGE = 2 * TILE_BYTES;          // A and B
constexpr uint32_t kOut = 0x80000000u;         // beyond every buffer range: loads zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}

// Byte offset of 16-byte chunk c (0..7) of row r in a K-contiguous 256 x 64 tile.
// Eight consecutive rows read at one chunk column land on eight distinct bank groups.
__device__ __forceinline__ int koff(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

__device__ __forceinline__ void lds_wait_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Instruction-group masks of the scheduling barriers.
constexpr int kMfma = 0x008, kVmemRead = 0x020, kDsRead = 0x100, kDsWrite = 0x200, kValu = 0x002;

// Interleave the preceding region: n rounds of (1 matrix instruction, k LDS reads).
template <int n, int k>
__device__ __forceinline__ void interleave_mfma_dsread() {
#pragma unroll
  for (int i = 0; i < n; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, k, 0);
  }
}

// Staging of the A slab (row-major: K-contiguous): 2048 chunks, 8 per lane.
// Chunk q = lane_id + 256 i: row q / 8, k-chunk q % 8.
// Load i reads row threadIdx.x / 8 + 32 i: one per-lane byte offset plus a uniform
// stride of 32 rows, passed as the load's scalar offset.
struct StageA {
  u32x4 r[8];
  uint32_t off;        // byte offset of row threadIdx.x / 8, chunk threadIdx.x % 8
  uint32_t stride;     // 32 rows, in bytes
  int rows_left;       // rows of the matrix at and below this lane's first row
  __device__ __forceinline__ void init(int64_t lda, int m0, int64_t M) {
    off = uint32_t((int64_t(threadIdx.x / 8) * lda + 8 * (threadIdx.x % 8)) * 2);
    stride = uint32_t(32 * lda * 2);
    rows_left = int(min<int64_t>(M - m0 - int64_t(threadIdx.x / 8), 1 << 30));
  }
  __device__ __forceinline__ void load(const uint16_t *A, int64_t lda, int m0, int k0, int64_t K) {
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(A + int64_t(m0) * lda + k0);
    const bool k_in = k0 + 8 * int(threadIdx.x % 8) < K;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool in = k_in && 32 * i < rows_left;
      r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, in ? off : kOut, int(i * stride), 0);
    }
  }
  __device__ __forceinline__ void store(char *tile) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int q = threadIdx.x + NT * i;
      *reinterpret_cast<u32x4 *>(tile + koff(q / 8, q % 8)) = r[i];
    }
  }
};

// Staging of a column-major B slab (K-contiguous): same shape as A with n for m.
using StageBk = StageA;

// Staging of a row-major B slab (N-contiguous): lane t owns the 8 x 8 block of k-rows
// 8*(t % 8) .. +7 and n-columns 8*(t / 8) .. +7.  Load i reads k-row 8*(t%8) + i; eight
// neighbouring lanes read eight k-rows, and the eight lane-groups of a wave read 128
// contiguous bytes of each.
struct StageBn {
  u32x4 r[8];
  uint32_t off;        // byte offset of k-row 8*(t%8), n-chunk t/8
  uint32_t stride;     // one k-row, in bytes
  bool col_ok;
  __device__ __forceinline__ void init(int64_t ldb, int n0, int64_t N) {
    const int kg = threadIdx.x % 8, nc = threadIdx.x / 8;
    off = uint32_t((int64_t(8 * kg) * ldb + 8 * nc) * 2);
    stride = uint32_t(ldb * 2);
    col_ok = n0 + 8 * nc < N;
  }
  __device__ __forceinline__ void load(const uint16_t *B, int64_t ldb, int n0, int k0, int64_t K) {
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(B + int64_t(k0) * ldb + n0);
    const int kleft = int(min<int64_t>(K - k0 - 8 * int(threadIdx.x % 8), 1 << 30));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool in = col_ok && i < kleft;
      r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, in ? off : kOut, int(i * stride), 0);
    }
  }
  // Transpose the 8 x 8 block of 16-bit values and store n-row by n-row.
  __device__ __forceinline__ void store(char *tile) const {
    const int kg = threadIdx.x % 8, nc = threadIdx.x / 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {        // n = 8*nc + j
      // byte selector: low halves of both words for even j, high halves for odd j
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      const int w = j >> 1;
      u32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e)   // k = 8kg + 2e (low half) and 8kg + 2e + 1 (high half)
        v[e] = __builtin_amdgcn_perm(r[2 * e + 1][w], r[2 * e][w], sel);
      *reinterpret_cast<u32x4 *>(tile + koff(8 * nc + j, kg)) = v;
    }
  }
};

template <class H, bool B_KC>
__global__ void __launch_bounds__(NT)
big_gemm(LaunchArgs p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  using StageB = typename std::conditional<B_KC, StageBk, StageBn>::type;

  int tm, tn;
  tile_of(blockIdx.x, p.gm, p.gn, p.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint16_t *A = static_cast<const uint16_t *>(p.A);
  const uint16_t *B = static_cast<const uint16_t *>(p.B);
  const int64_t K = p.K;

  StageA sa;
  StageB sb;
  sa.init(p.lda, m0, p.M);
  sb.init(p.ldb, n0, p.N);

  // Fragment f of k-step s (k = 32 s .. 32 s + 31): row block f / 2 (32 rows), k-half
  // f % 2; lane reads row (lane % 32) of the block, k-chunk 4 s + 2 (f % 2) + lane / 32.
  const int arow = wm * WTM + (lane & 31), brow = wn * WTN + (lane & 31);
  auto fragA = [&](const char *tile, int f, int s) {
    const int r = arow + 32 * (f >> 1);
    return *reinterpret_cast<const u32x4 *>(tile + koff(r, 4 * s + 2 * (f & 1) + (lane >> 5)));
  };
  auto fragB = [&](const char *tile, int f, int s) {
    const int r = brow + 32 * (f >> 1);
    return *reinterpret_cast<const u32x4 *>(tile + koff(r, 4 * s + 2 * (f & 1) + (lane >> 5)));
  };
  // acc[i][j] += A block i x B block j over k-half h of a 32-deep k-step, for the
  // blocks i in [i0, i1).  Consecutive matrix instructions update different
  // accumulators; the two k-halves of one accumulator are a whole half-step apart.
  auto half = [&](f32x16 (&acc)[4][4], const u32x4 (&fa)[FM], const u32x4 (&fb)[FN], int h, int i0, int i1) {
#pragma unroll
    for (int i = i0; i < i1; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(H{}, fb[2 * j + h], fa[2 * i + h], acc[i][j]);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int KT = int((K + BK - 1) / BK);
  sa.load(A, p.lda, m0, 0, K);
  sb.load(B, p.ldb, n0, 0, K);
  sa.store(smem);
  sb.store(smem + TILE_BYTES);
  sa.load(A, p.lda, m0, BK, K);       // past K these read zeros: the loop body is
  sb.load(B, p.ldb, n0, BK, K);       // branch-free so its phases can be interleaved
  lds_wait_barrier();

  u32x4 a0[FM], b0[FN], a1[FM], b1[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) a0[i] = fragA(smem, i, 0);
#pragma unroll
  for (int j = 0; j < FN; ++j) b0[j] = fragB(smem + TILE_BYTES, j, 0);

  for (int t = 0; t < KT; ++t) {
    const char *cur = smem + (t & 1) * STAGE;
    char *nxt = smem + ((t + 1) & 1) * STAGE;
    // Phase 1: k-step 0 (32 matrix instructions), interleaved one-for-one with the
    // 16 LDS reads of k-step 1's fragments.
#pragma unroll
    for (int j = 0; j < FN; ++j) b1[j] = fragB(cur + TILE_BYTES, j, 1);
    half(acc, a0, b0, 0, 0, 4);
#pragma unroll
    for (int i = 0; i < FM; ++i) a1[i] = fragA(cur, i, 1);
    half(acc, a0, b0, 1, 0, 4);
    interleave_mfma_dsread<16, 1>();
    __builtin_amdgcn_sched_barrier(0);
    // Phase 2: first half of k-step 1 (16 matrix instructions) with slab t+1's LDS
    // stores and slab t+2's global loads between them.
    // (On the last slabs these store and load zeros into a buffer nobody reads.)
    sa.store(nxt);
    sb.store(nxt + TILE_BYTES);
    sa.load(A, p.lda, m0, (t + 2) * BK, K);
    sb.load(B, p.ldb, n0, (t + 2) * BK, K);
    half(acc, a1, b1, 0, 0, 2);
    half(acc, a1, b1, 1, 0, 2);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kDsWrite, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kValu, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kVmemRead, 1, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    lds_wait_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // Phase 3: second half of k-step 1 with the LDS reads of slab t+1's k-step 0.
#pragma unroll
    for (int i = 0; i < FM; ++i) a0[i] = fragA(nxt, i, 0);
#pragma unroll
    for (int j = 0; j < FN; ++j) b0[j] = fragB(nxt + TILE_BYTES, j, 0);
    half(acc, a1, b1, 0, 2, 4);
    half(acc, a1, b1, 1, 2, 4);
    interleave_mfma_dsread<16, 1>();
    __builtin_amdgcn_sched_barrier(0);
  }

  // acc[i][j] holds the transposed 32 x 32 block: element r of lane l is
  // C[row m0 + 128 wm + 32 i + l % 32][col n0 + 128 wn + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4].
  const int64_t row0 = m0 + wm * WTM + (lane & 31);
  const int64_t colL = n0 + wn * WTN + 4 * (lane >> 5);
  const bool c_vec = p.c_vec != 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = row0 + 32 * i;
    if (row >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t col = colL + 32 * j + 8 * q;
        const int64_t n_in = p.N - col;
        if (n_in <= 0) continue;
        const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        store_out4(p.C, row * p.ldc + col, v, p.out_code, c_vec && n_in >= 4, int(n_in));
      }
  }
}

template __global__ void big_gemm<HalfBF16, false>(LaunchArgs);
template __global__ void big_gemm<HalfBF16, true>(LaunchArgs);
template __global__ void big_gemm<HalfF16, false>(LaunchArgs);
template __global__ void big_gemm<HalfF16, true>(LaunchArgs);

}  // namespace big

// Row-major A only; B row- or column-major.
hipError_t launch_big(const LaunchArgs &p, hipStream_t s) {
  const dim3 grid(unsigned(p.gm) * unsigned(p.gn)), block(big::NT);
  if (p.a_col) return hipErrorInvalidValue;
  if (p.in_code == E_BF16) {
    if (p.b_col) hipLaunchKernelGGL((big::big_gemm<HalfBF16, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((big::big_gemm<HalfBF16, false>), grid, block, 0, s, p);
  } else if (p.in_code == E_F16) {
    if (p.b_col) hipLaunchKernelGGL((big::big_gemm<HalfF16, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((big::big_gemm<HalfF16, false>), grid, block, 0, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mhg

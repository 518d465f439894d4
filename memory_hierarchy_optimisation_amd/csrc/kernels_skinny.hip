// kernels_skinny.hip -- fp16 / bf16 product with at most 16 rows of A (row-major A and
// B): C[M <= 16][N] = A[M][K] x B[K][N].
//
// Such a product reads B once and does 2*M flops per element of B, so it is bound by
// the HBM stream of B, not by the matrix units (roofline of "Tiling 策略与内存层次优化":
// intensity about M flop per byte, far left of the ridge).  What matters is keeping
// enough bytes in flight on every compute unit, and the pages' lever for a grid that
// is too small to do that ("GPU Kernel 的 Tile、Grid、Wave 与 Launch Overhead",
// per-shape section: too few workers to hide latency) is more workers.  Along N alone
// there are N / 128 column blocks (64 at N = 8192), a quarter of the compute units,
// so K is split as well:
//   * a workgroup owns 128 columns of C and every split-th 128-deep block of K (all
//     workgroups then stream through the same window of B's rows); its four waves
//     take one 32-deep round of each block;
//   * the waves' partial sums are added in LDS in a fixed order;
//   * with split_k > 1 each workgroup writes its 16 x 128 partial to the plan's
//     workspace, and the last workgroup of a column block to arrive (a per-block
//     arrival counter) adds the split_k partials in chunk order and writes C.  The
//     result is the same bits on every run, whatever the arrival order.  No
//     device-wide fence is used (see the end of run).
// Splitting K across workgroups is not on the pages (they split K only inside a
// block); it is the standard answer to a grid with too few workgroups.
//
// Per round a lane loads 16 bytes from each of 8 consecutive k-rows of B (lane
// (g, q) = (lane / 16, lane % 16): k-rows 8 g .. 8 g + 7 of the round, columns
// 8 q .. 8 q + 7; 16 lanes read 256 contiguous bytes of a row), transposes the
// 8 x 8 block in registers into 8 columns of 8 k-values, and feeds 8
// v_mfma_f32_16x16x32 instructions: A's 16 rows are the instruction's 16 rows, the
// 16 lanes of a group supply 16 columns (column 8 q + c in instruction c) with the
// group's 8 k-values, and A's fragment (row lane % 16, k 8 g .. 8 g + 7) is one
// 16-byte load.  Two register sets keep the next round's loads in flight while one
// is multiplied.
//
// Edges: rows of A at or beyond M, k-rows at or beyond K and column chunks at or
// beyond N are loaded as zeros (buffer offsets beyond the resource
// range); stores are masked.  The kernel requires 16-byte aligned A and B with K, N,
// lda and ldb multiples of 8 (checked by the host, which otherwise runs a
// register-staged kernel instead).
#include "device.h"

namespace mhg {
namespace skinny {

constexpr int BN = 128;        // columns of C per workgroup
constexpr int NT = 256;        // four waves
constexpr int ROUND = 32;      // k per round and wave
constexpr int CHUNK_ALIGN = 4 * ROUND;
constexpr uint32_t kOut = 0x80000000u;   // beyond every buffer range: loads zeros
constexpr int MAX_SPLIT = 16;
// Cache-policy operand of the buffer instructions: B is streamed once (non-temporal);
// the workspace partials use the device-scope coherence bit (sc1), the policy the
// compiler gives agent-scope atomic loads and stores.
constexpr int kNonTemporal = 2, kDeviceScope = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}


template <class H>
struct Skinny {
  const LaunchArgs &p;
  int lane, g, q;
  // B: lane's byte offset (k-row 8 g, column chunk q) from a round's origin; k-rows of
  // the matrix at and below the lane's first row of round k = 0 (very negative when
  // the lane's columns lie past N).
  uint32_t b_off, b_row;
  int b_klim;
  // A: lane's byte offset (row q, k 8 g) from a round's origin; k of the matrix at and
  // beyond the lane's first k of round k = 0 (very negative when row q lies past M).
  uint32_t a_off;
  int a_klim;
  f32x4 acc[8];
  u32x4 rb[2][8];
  u32x4 ra[2];

  __device__ __forceinline__ Skinny(const LaunchArgs &p_) : p(p_) {}

  template <int SET>
  __device__ __forceinline__ void load(const uint16_t *A, const uint16_t *B, int64_t kr, int kround) {
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(B + kr * p.ldb);
    const int lim = b_klim - kround;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      rb[SET][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, i < lim ? b_off : kOut, int(i * b_row), kNonTemporal);
    const __amdgpu_buffer_rsrc_t ar = rsrc_of(A + kr);
    ra[SET] = __builtin_amdgcn_raw_buffer_load_b128(ar, kround < a_klim ? a_off : kOut, 0, 0);
  }

  // Column c of the lane's 8 x 8 block as 8 k-values (k-row pairs packed per word).
  template <int SET>
  __device__ __forceinline__ u32x4 column(int c) const {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    const int w = c >> 1;
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __builtin_amdgcn_perm(rb[SET][2 * e + 1][w], rb[SET][2 * e][w], sel);
    return v;
  }

  template <int SET>
  __device__ __forceinline__ void multiply() {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = mfma16(H{}, ra[SET], column<SET>(c), acc[c]);
  }

  __device__ void run(float (*red)[16][BN], int *last) {
    const int gn = p.gn, split = p.split_k;
    const int tn = int(blockIdx.x % unsigned(gn)), z = int(blockIdx.x / unsigned(gn));
    // Uniform per wave: keeps the buffer resources of A and B in scalar registers.
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    lane = threadIdx.x & 63;
    g = lane >> 4;
    q = lane & 15;
    const int64_t n0 = int64_t(tn) * BN;
    // The workgroup of chunk z takes the 128-deep blocks z, z + split, z + 2 split, ...
    // of K (its waves one 32-deep round of each block), so all workgroups stream
    // through the same moving window of B's rows rather than split separate regions.
    const int rounds = int((p.K + int64_t(CHUNK_ALIGN) * split - 1) / (int64_t(CHUNK_ALIGN) * split));
    const uint16_t *A = static_cast<const uint16_t *>(p.A);
    const uint16_t *B = static_cast<const uint16_t *>(p.B) + n0;
    // k of round j of this wave: ROUND * (wave + 4 (z + split j)).
    b_off = uint32_t((int64_t(8 * g) * p.ldb + 8 * q) * 2);
    b_row = uint32_t(p.ldb * 2);
    b_klim = n0 + 8 * q < p.N ? int(p.K - 8 * g) : -(1 << 30);
    a_off = uint32_t((int64_t(q) * p.lda + 8 * g) * 2);
    a_klim = q < p.M ? int(p.K - 8 * g) : -(1 << 30);
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = f32x4{};

    auto kr_of = [&](int j) { return int64_t(ROUND) * (wave + 4 * (z + int64_t(split) * j)); };
    load<0>(A, B, kr_of(0), int(kr_of(0)));
    load<1>(A, B, kr_of(1), int(kr_of(1)));
    // Rounds past K load zeros, so the loop needs no branches inside.
    int j = 0;
    for (; j + 1 < rounds; j += 2) {
      multiply<0>();
      load<0>(A, B, kr_of(j + 2), int(kr_of(j + 2)));
      multiply<1>();
      load<1>(A, B, kr_of(j + 3), int(kr_of(j + 3)));
    }
    if (j < rounds) multiply<0>();
    // The loads still in flight read zeros past K; let them land before the
    // registers are reused by the epilogue.
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));

    // acc[c] lane l: rows 4 g .. 4 g + 3 of column 8 q + c.  Waves' partials meet in
    // LDS and are added in wave order.  A row of red holds columns 8 u .. 8 u + 3 at
    // float 4 u and 8 u + 4 .. 8 u + 7 at float 64 + 4 u, so that the 16 lanes an LDS
    // pass serves touch 16 different 16-byte chunks of the 256 bytes of banks (at float
    // 8 u, lanes u and u + 8 shared banks: half the LDS cycles were conflict cycles).
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float *dst = &red[wave][4 * g + r][0];
      *reinterpret_cast<f32x4 *>(dst + 4 * q) = f32x4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
      *reinterpret_cast<f32x4 *>(dst + 64 + 4 * q) = f32x4{acc[4][r], acc[5][r], acc[6][r], acc[7][r]};
    }
    __syncthreads();
    const int row = threadIdx.x >> 4, u = threadIdx.x & 15, col = 8 * u;
    f32x4 s0 = *reinterpret_cast<const f32x4 *>(&red[0][row][4 * u]);
    f32x4 s1 = *reinterpret_cast<const f32x4 *>(&red[0][row][64 + 4 * u]);
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      s0 += *reinterpret_cast<const f32x4 *>(&red[w][row][4 * u]);
      s1 += *reinterpret_cast<const f32x4 *>(&red[w][row][64 + 4 * u]);
    }
    const int64_t cg = n0 + col;
    const bool c_vec = p.c_vec != 0;
    auto store = [&](f32x4 a, f32x4 b) {
      if (row >= p.M) return;
      const int64_t n_in = p.N - cg;
      if (n_in <= 0) return;
      if (p.epi) {
        a = epilogue4(p, a, row, cg, n_in);
        b = epilogue4(p, b, row, cg + 4, n_in - 4);
      }
      store_out4(p.C, row * p.ldc + cg, a, p.out_code, c_vec && n_in >= 4, int(n_in));
      if (n_in > 4) store_out4(p.C, row * p.ldc + cg + 4, b, p.out_code, c_vec && n_in >= 8, int(n_in - 4));
    };
    if (split == 1) {
      store(s0, s1);
      return;
    }
    // Split K: partial to the workspace, then the last arrival of the column block
    // adds all partials in chunk order.  Workspace: gn arrival counters (padded to
    // 256 bytes), then partials [split][gn][16][BN] fp32.
    //
    // Visibility across the XCDs' separate L2 caches without a device-wide fence (an
    // agent-scope release writes back the whole L2 and cost more than the product
    // itself once every workgroup issued one).  The LLVM AMDGPU backend's memory model
    // for gfx942/gfx950 encodes a relaxed agent-scope atomic store or load as the plain
    // access with the sc1 bit, an agent-scope release as an L2 write-back (buffer_wbl2
    // sc1) followed by a wait for all outstanding memory accesses (vmcnt 0), and an
    // agent-scope acquire as that wait followed by an L2 invalidate (buffer_inv sc1);
    // the write-back and the invalidate exist for ordinary accesses only.  So: the
    // partials are written as agent-scope atomic stores (sc1 buffer stores, written
    // through to the coherent level); each lane waits for them to be acknowledged
    // (vmcnt 0, the release's ordering part; __syncthreads alone does not wait for
    // them); the workgroup barrier then precedes the arrival RMW; and the last arrival
    // reads the partials back as agent-scope atomic loads (sc1), issued only after its
    // RMW returned.  No ordinary access touches the workspace.
    unsigned *count = static_cast<unsigned *>(p.workspace);
    const float *part = reinterpret_cast<const float *>(static_cast<char *>(p.workspace) +
                                                        ((int64_t(gn) * 4 + 255) / 256) * 256);
    // One resource over the column block's partials: chunk zz at scalar offset
    // zz * slice bytes (the plan keeps all partials below 2^31 bytes).
    const __amdgpu_buffer_rsrc_t pr = rsrc_of(part + int64_t(tn) * (16 * BN));
    const uint32_t slice = uint32_t(int64_t(gn) * (16 * BN) * 4);
    const uint32_t voff = uint32_t((row * BN + col) * 4);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s0), pr, voff, int(z * slice), kDeviceScope);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s1), pr, voff + 16, int(z * slice), kDeviceScope);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned before = __hip_atomic_fetch_add(count + tn, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *last = before == unsigned(split - 1);
    }
    __syncthreads();
    if (!*last) return;
    // All chunks' partials requested at once (chunks past split read zeros), then
    // added in chunk order.
    u32x4 v[MAX_SPLIT][2];
#pragma unroll
    for (int zz = 0; zz < MAX_SPLIT; ++zz) {
      const uint32_t o = zz < split ? voff : kOut;
      v[zz][0] = __builtin_amdgcn_raw_buffer_load_b128(pr, o, int(zz * slice), kDeviceScope);
      v[zz][1] = __builtin_amdgcn_raw_buffer_load_b128(pr, o == kOut ? kOut : o + 16, int(zz * slice), kDeviceScope);
    }
    f32x4 t0 = __builtin_bit_cast(f32x4, v[0][0]), t1 = __builtin_bit_cast(f32x4, v[0][1]);
#pragma unroll
    for (int zz = 1; zz < MAX_SPLIT; ++zz) {
      t0 += __builtin_bit_cast(f32x4, v[zz][0]);
      t1 += __builtin_bit_cast(f32x4, v[zz][1]);
    }
    store(t0, t1);
    // Re-arm the counter for the next call on this workspace.
    if (threadIdx.x == 0) __hip_atomic_store(count + tn, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
};

template <class H>
__global__ void __launch_bounds__(NT, 2) skinny_gemm(LaunchArgs p) {
  __shared__ float red[4][16][BN];
  __shared__ int last;
  // The arguments the stream needs, and those the compiler fetches early anyway, in
  // scalar registers before anything else: requested together, waited for once.
  asm volatile("" ::"s"(p.gn), "s"(p.split_k), "s"(p.A), "s"(p.B), "s"(p.M), "s"(p.N), "s"(p.K), "s"(p.lda),
               "s"(p.ldb), "s"(p.epi), "s"(p.alpha), "s"(p.beta));
  Skinny<H> s(p);
  s.run(red, &last);
}

template __global__ void skinny_gemm<HalfBF16>(LaunchArgs);
template __global__ void skinny_gemm<HalfF16>(LaunchArgs);

__global__ void zero_words(unsigned *w, int64_t n) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) w[i] = 0u;
}

}  // namespace skinny

// Row-major A and B, M <= 16, operands checked by the host (see the file comment).
hipError_t launch_skinny(const LaunchArgs &p, hipStream_t s) {
  if (p.a_col || p.b_col || p.M > 16 || p.split_k < 1) return hipErrorInvalidValue;
  if (p.split_k > 1 && !p.workspace) return hipErrorInvalidValue;
  const dim3 grid(unsigned(p.gn) * unsigned(p.split_k)), block(skinny::NT);
  if (p.in_code == E_BF16) hipLaunchKernelGGL(skinny::skinny_gemm<HalfBF16>, grid, block, 0, s, p);
  else if (p.in_code == E_F16) hipLaunchKernelGGL(skinny::skinny_gemm<HalfF16>, grid, block, 0, s, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// Zero n 32-bit words (the arrival counters of a fresh workspace) on a stream, with a
// kernel rather than a memset so that the call is safe to record into a graph.
hipError_t launch_zero_words(void *w, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = unsigned((n + 255) / 256);
  hipLaunchKernelGGL(skinny::zero_words, dim3(blocks), dim3(256), 0, s, static_cast<unsigned *>(w), n);
  return hipGetLastError();
}

}  // namespace mhg

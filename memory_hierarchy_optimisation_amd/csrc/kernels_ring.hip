// kernels_ring.hip -- fp16 / bf16 GEMM for large aligned problems: a deep LDS ring fed
// by direct global-to-LDS loads.
//
// Same three tiling levels as kernels_mfma.hip (workgroup tile, K slabs in LDS,
// per-wave MFMA register tiles), with the staging step moved off the registers:
//   * every lane issues 16-byte buffer loads that write straight into LDS (the
//     gfx950 counterpart of the asynchronous global-to-shared copy described in
//     "Tiling 策略与内存层次优化", cp.async section: no register round trip);
//   * LDS holds a ring of STAGES slabs of BK = 32 (N-stage pipelining, same page,
//     double buffering section: LDS = tile x elem x stages), so STAGES - 1 slabs are
//     in flight while one is consumed;
//   * each wave double-buffers its operand fragments in registers: right after the
//     barrier that publishes slab t+1 it issues the LDS reads of slab t+1, then runs
//     the matrix instructions of slab t, which hide those reads' latency.
// A loaded lane's 16 bytes land at the wave's LDS destination + 16 * lane, so the
// XOR swizzle of the LDS layout is applied on the global side: lane l loads the
// chunk that belongs at LDS slot l.  Chunks outside the matrix take an out-of-range
// buffer offset and arrive as zeros ("CUDA tile", 4: zero is the identity of the sum).
//
// One barrier per slab.  It is issued as an s_barrier in an asm statement with a
// memory clobber, after an explicit wait that leaves the younger slabs' loads in
// flight: the C++ block barrier would also wait for those.  Before the barrier each
// wave waits for its own loads of the next slab and for its own LDS reads, so after
// it (a) the next slab is visible to every wave and (b) no wave still reads the
// buffer that the next loads overwrite.
#include "device.h"

namespace mhg {
namespace ring {

constexpr int RBK = 32;                 // slab depth
constexpr uint32_t kOut = 0x80000000u;  // offset beyond every buffer range: loads zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}

// s_waitcnt with only vmcnt = n (n < 64) and lgkmcnt = 0; expcnt left free.
template <int n>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(n >= 0 && n < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (0 << 8));
}

__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// K-contiguous tile: rows of 32 elements (64 bytes, 4 chunks).  Chunk c of row r is
// stored at slot c ^ ((r >> 1) & 3): eight consecutive rows read at one chunk column
// cover eight distinct 16-byte bank groups.
__device__ __forceinline__ int kc_slot(int r, int c) { return r * 4 + (c ^ ((r >> 1) & 3)); }

// M/N-contiguous tile: 32 k-rows of NCH chunks.  Chunk c of k-row r is stored at
// slot c ^ (2 * (r & 3)), spreading the four k-rows of a transpose read.
template <int NCH>
__device__ __forceinline__ int mn_slot(int r, int c) { return r * NCH + (c ^ (((r & 3) << 1) & (NCH - 1))); }

// One operand's slab staging and fragment reads.
//   R: tile extent (BM or BN); KC: K-contiguous storage; NT: threads.
template <int R, bool KC, int NT>
struct RingOperand {
  static constexpr int SLOTS = R * RBK / 8;          // 16-byte chunks per slab
  static constexpr int LOADS = SLOTS / NT;           // loads per thread per slab
  static constexpr int NCH = R / 8;                   // chunks per k-row (MN tiles)
  static constexpr int BYTES = SLOTS * 16;
  static_assert(SLOTS % NT == 0, "slab must divide over the threads");
  static_assert(KC || (NCH & (NCH - 1)) == 0, "chunks per k-row must be a power of two");

  const uint16_t *base;
  int64_t ld, K;
  int mn0;
  uint32_t off[LOADS];   // byte offset from the slab origin of the chunk this lane loads
  int kin[LOADS];        // its k within the slab
  bool mn_ok[LOADS];     // its m (or n) lies inside the matrix

  __device__ __forceinline__ RingOperand(const uint16_t *g, int64_t ld_, int64_t mn_lim, int64_t K_, int mn0_)
      : base(g), ld(ld_), K(K_), mn0(mn0_) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      // LDS slot written by this lane for load j: wave-major blocks of 64 slots
      const int slot = (j * (NT / 64) + wave) * 64 + lane;
      int r, c;   // storage row / chunk column of the chunk that belongs at `slot`
      if (KC) {
        r = slot / 4;
        c = (slot % 4) ^ ((r >> 1) & 3);
        off[j] = uint32_t((int64_t(r) * ld + 8 * c) * 2);
        kin[j] = 8 * c;
        mn_ok[j] = mn0 + r < mn_lim;
      } else {
        r = slot / NCH;
        c = (slot % NCH) ^ (((r & 3) << 1) & (NCH - 1));
        off[j] = uint32_t((int64_t(r) * ld + 8 * c) * 2);
        kin[j] = r;
        mn_ok[j] = mn0 + 8 * c < mn_lim;
      }
    }
  }

  // Loads of the slab starting at k0 into the LDS stage `dst` (wave-uniform).
  __device__ __forceinline__ void issue(int k0, char *dst) const {
    const uint16_t *origin = KC ? base + int64_t(mn0) * ld + k0 : base + int64_t(k0) * ld + mn0;
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(origin);
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const bool in = mn_ok[j] && (k0 + kin[j] < K);
      char *ldst = dst + (j * (NT / 64) + wave) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (MHG_LDS void *)ldst, 16, in ? off[j] : kOut, 0, 0, 0);
    }
  }

  // Fragment of 16 rows starting at tile-local r0 (k = 0 .. 31 of the slab).
  __device__ __forceinline__ u32x4 frag(const char *src, int r0, int lane) const {
    if (KC) {
      const int r = r0 + (lane & 15);
      return *reinterpret_cast<const u32x4 *>(src + kc_slot(r, lane >> 4) * 16);
    } else {
      const int L = lane & 15, grp = lane >> 4;
      const int col = r0 + 4 * (L & 3);
      const int c = col >> 3, byte = (col & 7) * 2;
      const int kr = 8 * grp + (L >> 2);
      u32x2 lo = lds_read_tr16(src + mn_slot<NCH>(kr, c) * 16 + byte);
      u32x2 hi = lds_read_tr16(src + mn_slot<NCH>(kr + 4, c) * 16 + byte);
      return u32x4{lo.x, lo.y, hi.x, hi.y};
    }
  }
};

template <class H, int BM, int BN, int WM, int WN, int STAGES, bool A_KC, bool B_KC>
__global__ void __launch_bounds__(WM * WN * 64)
ring_gemm(LaunchArgs p) {
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  using OA = RingOperand<BM, A_KC, NT>;
  using OB = RingOperand<BN, B_KC, NT>;
  constexpr int STAGE = OA::BYTES + OB::BYTES;
  constexpr int LOADS = OA::LOADS + OB::LOADS;   // per thread per slab
  static_assert(STAGES >= 2, "ring needs two stages");
  static_assert(LOADS * (STAGES - 1) < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE];

  int tm, tn;
  tile_of(blockIdx.x, p.gm, p.gn, p.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;

  const OA oa(static_cast<const uint16_t *>(p.A), p.lda, p.M, p.K, m0);
  const OB ob(static_cast<const uint16_t *>(p.B), p.ldb, p.N, p.K, n0);
  const int KT = int((p.K + RBK - 1) / RBK);

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Prologue: slabs 0 .. STAGES-1 in flight (past K they load zeros, which keeps the
  // count of loads in flight the same in every iteration).
#pragma unroll
  for (int s = 0; s < STAGES; ++s) {
    oa.issue(s * RBK, smem + s * STAGE);
    ob.issue(s * RBK, smem + s * STAGE + OA::BYTES);
  }
  u32x4 fa[FM], fb[FN];
  wait_vm_lgkm0<LOADS * (STAGES - 1)>();     // slab 0 landed
  block_barrier();
#pragma unroll
  for (int i = 0; i < FM; ++i) fa[i] = oa.frag(smem, wm * WTM + i * 16, lane);
#pragma unroll
  for (int j = 0; j < FN; ++j) fb[j] = ob.frag(smem + OA::BYTES, wn * WTN + j * 16, lane);

  for (int t = 0; t < KT; ++t) {
    // Slab t+1 landed (slabs t+2 .. t+STAGES-1 may still be in flight); this wave's
    // reads of slab t are in registers.
    wait_vm_lgkm0<LOADS * (STAGES - 2)>();
    block_barrier();
    // Buffer t % STAGES is free: refill it with slab t + STAGES.
    char *refill = smem + (t % STAGES) * STAGE;
    oa.issue((t + STAGES) * RBK, refill);
    ob.issue((t + STAGES) * RBK, refill + OA::BYTES);
    u32x4 na[FM], nb[FN];
    if (t + 1 < KT) {
      const char *nxt = smem + ((t + 1) % STAGES) * STAGE;
#pragma unroll
      for (int i = 0; i < FM; ++i) na[i] = oa.frag(nxt, wm * WTM + i * 16, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) nb[j] = ob.frag(nxt + OA::BYTES, wn * WTN + j * 16, lane);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma16(H{}, fb[j], fa[i], acc[i][j]);
    if (t + 1 < KT) {
#pragma unroll
      for (int i = 0; i < FM; ++i) fa[i] = na[i];
#pragma unroll
      for (int j = 0; j < FN; ++j) fb[j] = nb[j];
    }
  }
  // Drain the zero-filling loads past K before the workgroup's LDS can be reused.
  wait_vm_lgkm0<0>();

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

// Every kernel is instantiated explicitly.  Without this, the ROCm 7.2 host compiler
// declared but did not define the launch stubs of all but the first instantiation
// that shared its operand-staging types, and the library failed to load.
#define MHG_RING_INST(H, BM, BN, WM, WN)                                               \
  template __global__ void ring_gemm<H, BM, BN, WM, WN, 4, true, false>(LaunchArgs);  \
  template __global__ void ring_gemm<H, BM, BN, WM, WN, 4, true, true>(LaunchArgs);   \
  template __global__ void ring_gemm<H, BM, BN, WM, WN, 4, false, false>(LaunchArgs); \
  template __global__ void ring_gemm<H, BM, BN, WM, WN, 4, false, true>(LaunchArgs);
MHG_RING_INST(HalfBF16, 256, 256, 2, 2)
MHG_RING_INST(HalfBF16, 256, 256, 2, 4)
MHG_RING_INST(HalfBF16, 128, 128, 2, 2)
MHG_RING_INST(HalfF16, 256, 256, 2, 2)
MHG_RING_INST(HalfF16, 256, 256, 2, 4)
MHG_RING_INST(HalfF16, 128, 128, 2, 2)
#undef MHG_RING_INST

template <class H, int BM, int BN, int WM, int WN, int STAGES>
hipError_t launch_ring_t(const LaunchArgs &p, hipStream_t s) {
  const dim3 grid(unsigned(p.gm) * unsigned(p.gn)), block(WM * WN * 64);
  if (!p.a_col && !p.b_col)
    hipLaunchKernelGGL((ring_gemm<H, BM, BN, WM, WN, STAGES, true, false>), grid, block, 0, s, p);
  else if (!p.a_col && p.b_col)
    hipLaunchKernelGGL((ring_gemm<H, BM, BN, WM, WN, STAGES, true, true>), grid, block, 0, s, p);
  else if (p.a_col && !p.b_col)
    hipLaunchKernelGGL((ring_gemm<H, BM, BN, WM, WN, STAGES, false, false>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((ring_gemm<H, BM, BN, WM, WN, STAGES, false, true>), grid, block, 0, s, p);
  return hipGetLastError();
}

template <class H>
hipError_t launch_ring_typed(int launcher, const LaunchArgs &p, hipStream_t s) {
  switch (launcher) {
    case L_RING_256x256_W4: return launch_ring_t<H, 256, 256, 2, 2, 4>(p, s);
    case L_RING_256x256_W8: return launch_ring_t<H, 256, 256, 2, 4, 4>(p, s);
    case L_RING_128x128_W4: return launch_ring_t<H, 128, 128, 2, 2, 4>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ring

hipError_t launch_ring(int launcher, const LaunchArgs &p, hipStream_t s) {
  if (p.in_code == E_BF16) return ring::launch_ring_typed<HalfBF16>(launcher, p, s);
  if (p.in_code == E_F16) return ring::launch_ring_typed<HalfF16>(launcher, p, s);
  return hipErrorInvalidValue;
}

// The ring kernels read with 16-byte buffer loads whose offsets from a slab origin
// must stay below 2^31 bytes; the C++ side checks this and the alignment before
// choosing them.
bool ring_supported(const LaunchArgs &p, int bm, int bn) {
  const int64_t a_ext = p.a_col ? p.M : p.K, b_ext = p.b_col ? p.K : p.N;
  if (!(p.vec_a && p.vec_b && a_ext % 8 == 0 && b_ext % 8 == 0)) return false;
  const int64_t a_span = (p.a_col ? ring::RBK : bm) * p.lda * 2, b_span = (p.b_col ? bn : ring::RBK) * p.ldb * 2;
  return a_span < (int64_t(1) << 31) && b_span < (int64_t(1) << 31);
}

}  // namespace mhg

// kernels_w8.hip -- fp16 / bf16 GEMM for large aligned problems: 256 x 256 workgroup
// tiles, eight waves (two per SIMD) of 128 x 64 register tiles, both operands loaded
// straight into a five-slot LDS ring of 32-deep K slabs.
//
// The three tiling levels of "Tiling 策略与内存层次优化" (multi-level tiling) sized for
// gfx950:
//   * workgroup tile 256 x 256: tile intensity 2*256*256 / (512*2) = 128 FLOP/B (same
//     page, how tiling raises intensity), one tile per compute unit at 4096^2;
//   * K slabs of 32 in a ring of five 32 KiB LDS slots (160 KB, constraint 1 of the
//     same page with stages = 5): three slabs in flight while one is consumed (N-stage
//     pipelining, double-buffering section), loaded with 16-byte LDS-destination
//     buffer loads, the gfx950 counterpart of cp.async (cp.async section);
//   * eight waves, two per SIMD, each owning 128 x 64 of C as 4 x 2 accumulators of
//     32 x 32 (v_mfma_f32_32x32x16_{bf16,f16}; 128 fp32 registers a lane).  With one
//     wave per SIMD the wave stalls on its own global and LDS instructions and the
//     matrix pipe idles meanwhile; with two, the other wave's matrix instructions
//     issue in those gaps, so a register tile of half the size ("寄存器Tiling", 1.3:
//     the register budget trades tile size for resident waves) pays for itself.
// Operands are stored in LDS in their global orientation:
//   * a K-contiguous operand (row-major A, column-major B) as 256 rows of 64 bytes;
//     each fragment is one 16-byte LDS read per lane;
//   * an M/N-contiguous operand (column-major A, row-major B) as 32 k-rows of 512
//     bytes; each fragment is two LDS transpose reads (ds_read_b64_tr_b16), so the
//     operand is never transposed in registers.
// Both layouts XOR-swizzle 16-byte chunks (bank conflicts and swizzle section:
// row XOR column) so that the fragment reads are conflict-free; a loaded lane's 16
// bytes land at the wave's LDS destination + 16 * lane, so the swizzle is applied on
// the global side (each lane loads the chunk that belongs at its LDS slot).
//
// Edges: chunks outside the matrix are loaded through an offset beyond the buffer
// range and arrive as zeros ("CUDA tile", 4: zero is the identity of the sum); stores
// are masked.  The host requires 16-byte aligned operands whose contiguous extents and
// leading dimensions are multiples of 8 elements.
#include <type_traits>

#include "device.h"

namespace mhg {
namespace w8 {

constexpr int BM = 256, BN = 256, BK = 32, NT = 512, SLOTS = 5;
constexpr int OP_BYTES = 256 * BK * 2;          // one operand's slab: 16 KiB
constexpr int SLOT_BYTES = 2 * OP_BYTES;        // A at +0, B at +16 KiB
constexpr int WTM = 128, WTN = 64;              // register tile of a wave
constexpr int LOADS = OP_BYTES / (NT * 16);     // 16-byte loads per lane per operand and slab (2)
constexpr int PER_SLAB = 2 * LOADS;             // loads per lane and slab, both operands
constexpr uint32_t kOut = 0x80000000u;          // beyond every buffer range: loads zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}

__device__ __forceinline__ u32x4 lds_ld(uint32_t a) {
  return *reinterpret_cast<const MHG_LDS u32x4 *>(size_t(a));
}
__device__ __forceinline__ u32x2 lds_ld_tr(uint32_t a) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MHG_LDS bf16x4 *)(size_t)a));
}

// LDS layouts of one operand's slab (byte offsets within its 16 KiB):
//   K-contiguous: row r (0..255) of four 16-byte k-chunks; chunk c at r*64 + 16*(c ^ ((r >> 2) & 3)).
//     Sixteen consecutive rows read at one chunk (a fragment read, 16 lanes an LDS
//     cycle) land on 16 distinct 16-byte bank groups.
//   M/N-contiguous: k-row k (0..31) of 32 chunks of 8 m/n-values; chunk c at
//     k*512 + 16*(c ^ (4*(k & 3))).  A transpose read touches four consecutive k-rows,
//     64 bytes each; the XOR moves them to four distinct quarters of the banks.
__device__ __forceinline__ uint32_t kc_off(int r, int c) { return uint32_t(r * 64 + 16 * (c ^ ((r >> 2) & 3))); }
__device__ __forceinline__ uint32_t mn_off(int k, int c) { return uint32_t(k * 512 + 16 * (c ^ (4 * (k & 3)))); }

// One operand: its slab loads and its fragment reads.
template <bool KC>
struct Operand {
  uint32_t off[LOADS];   // byte offset of the lane's chunk from the slab origin, per load
  int kin[LOADS];        // k of the chunk within the slab; 2^30 when its rows (m or n)
                         // lie outside the matrix, so that it is never loaded
  int64_t ld;
  // Load j of wave w fills LDS bytes (8 j + w) * 1024 .. +1023 of the slab; lane l
  // writes chunk slot (8 j + w) * 64 + l and loads the chunk that belongs there.
  __device__ __forceinline__ void init(int64_t ld_, int mn0, int64_t MN, int wave, int lane) {
    ld = ld_;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int slot = (8 * j + wave) * 64 + lane;
      if (KC) {
        const int r = slot >> 2, c = (slot & 3) ^ ((r >> 2) & 3);
        off[j] = uint32_t((int64_t(r) * ld + 8 * c) * 2);
        kin[j] = mn0 + r < MN ? 8 * c : 1 << 30;
      } else {
        const int k = slot >> 5, c = (slot & 31) ^ (4 * (k & 3));
        off[j] = uint32_t((int64_t(k) * ld + 8 * c) * 2);
        kin[j] = mn0 + 8 * c < MN ? k : 1 << 30;
      }
    }
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint16_t *g, int mn0, int k0) const {
    return rsrc_of(KC ? g + int64_t(mn0) * ld + k0 : g + int64_t(k0) * ld + mn0);
  }
  // Load j of the slab at k0 into the operand's LDS area `dst` (wave-uniform; so is
  // `wave`: the LDS destination of these loads is a scalar register).
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, int k_left, uint32_t dst, uint32_t wave,
                                        int j) const {
    const bool in = kin[j] < k_left;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (MHG_LDS void *)(size_t)(dst + (8 * j + wave) * 1024), 16,
                                             in ? off[j] : kOut, 0, 0, 0);
  }
};

// Fragment addressing.  A 32 x 16 fragment (32 rows of m or n, 16 k) for
// v_mfma_f32_32x32x16: lane l holds row l % 32, k = 8 (l / 32) .. +7 of the 16-deep
// step.
//   K-contiguous: one 16-byte read at kc_off(b + l % 32, 2 s + l / 32).  The swizzle
//     term depends on the lane only (b is a multiple of 32), so the step s is an XOR of
//     32 on the lane's offset and the block b a constant 64 b.
//   M/N-contiguous: two transpose reads (e = 0, 1) for k = 8 (l / 32) + 4 e .. +3.  In
//     each 16-lane group g = l / 16, lane 4 q + u addresses the 8 bytes of k-row
//     16 s + 8 (g / 2) + 4 e + q, columns b + 16 (g % 2) + 4 u .. +3, and lane t then
//     receives column b + 16 (g % 2) + t of those four k-rows.
__device__ __forceinline__ uint32_t kc_lane(int lane) { return kc_off(lane & 31, lane >> 5); }
// Offset of the transpose read of block index jb (= b / 32) for k-half e = 0, step 0.
__device__ __forceinline__ uint32_t mn_lane(int lane, int jb) {
  const int g = lane >> 4, t = lane & 15, q = t >> 2, u = t & 3;
  const int k = 8 * (g >> 1) + q;
  const int c = 4 * jb + 2 * (g & 1) + (u >> 1);
  return mn_off(k, c) + 8 * (u & 1);
}

// s_waitcnt with vmcnt = n and expcnt / lgkmcnt left free.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }
#define MHG_ORDER() __builtin_amdgcn_sched_barrier(0)

// LDS reads of the fragments, issued as plain instructions.  The compiler would treat
// a transpose read as possibly aliasing the LDS-destination loads in flight and wait
// for all of them; the ring's waits and barriers already order those accesses, so
// these reads are not shown to it as memory accesses, and their completion is awaited
// explicitly (lgkmcnt) before the instruction that consumes them.
template <int OFF>
__device__ __forceinline__ void ds_b128(u32x4 &d, uint32_t a) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(a), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_tr(u32x2 &d, uint32_t a) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(d) : "v"(a), "i"(OFF));
}
template <int n>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(n >= 0 && n < 16, "lgkmcnt field");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (n << 8));
}

template <class H, bool A_KC, bool B_KC>
struct W8Gemm {
  const LaunchArgs &p;
  const uint16_t *A, *B;
  int m0, n0;
  int kdim;                   // K (below 2^31 by the plan's validation)
  uint32_t lds0, wave;
  Operand<A_KC> oa;
  Operand<B_KC> ob;
  // Lane offsets of the fragment reads within an operand slab (step 0), the wave's
  // block offset included: K-contiguous operands use [0] (step 1 is [0] ^ 32, the
  // wave's block i adds 2048 i); M/N-contiguous ones one per block (step 1 adds 8192,
  // the high k-half 2048).
  uint32_t fa_off[4], fb_off[2];
  f32x16 acc[4][2];
  // Fragment sets (step s of a slab uses set s), as low and high halves (k 0..3 and
  // 4..7 of the lane's eight): a 16-byte read fills both, a transpose read one.
  u32x2 fa[2][4][2], fb[2][2][2];

  // Reads of one step, in the order the next step needs them: B block 0, A block 0,
  // B block 1, A blocks 1..3; a fragment is one read (K-contiguous) or two.
  static constexpr int NA = A_KC ? 1 : 2, NB = B_KC ? 1 : 2;
  static constexpr int T = 2 * NB + 4 * NA;          // reads per step
  // Fragment (0..3: A block, 4..5: B block) and half of read k.
  static constexpr int read_frag(int k) {
    return k < NB ? 4 : k < NB + NA ? 0 : k < 2 * NB + NA ? 5 : 1 + (k - 2 * NB - NA) / NA;
  }
  static constexpr int read_half(int k) {
    return k < NB ? k : k < NB + NA ? k - NB : k < 2 * NB + NA ? k - NB - NA : (k - 2 * NB - NA) % NA;
  }
  // Reads the matrix instruction m of a step needs, counted from the first.
  static constexpr int needed(int m) {
    return m == 0 ? NB + NA : m == 1 ? 2 * NB + NA : m < 4 ? 2 * NB + 2 * NA : m < 6 ? 2 * NB + 3 * NA : T;
  }
  // Reads issued after matrix instruction n of a step: [first(n), first(n + 1)).
  static constexpr int first(int n) { return n * T / 8; }
  // LDS operations that may still be outstanding when matrix instruction m starts:
  // the previous step's reads after the ones it needs, and this step's reads so far.
  static constexpr int allowed(int m) {
    return (T - needed(m) + first(m)) < 15 ? T - needed(m) + first(m) : 15;
  }

  __device__ __forceinline__ W8Gemm(const LaunchArgs &p_) : p(p_) {}

  // Read k of step S into set SET from the slab whose A area starts at `slot`.
  template <int SET, int S, int K>
  __device__ __forceinline__ void read(uint32_t slot) {
    constexpr int f = read_frag(K), h = read_half(K);
    if constexpr (f < 4) {
      if constexpr (A_KC) {
        ds_b128<2048 * f>(*reinterpret_cast<u32x4 *>(&fa[SET][f][0]), slot + (fa_off[0] ^ uint32_t(32 * S)));
      } else {
        ds_tr<8192 * S + 2048 * h>(fa[SET][f][h], slot + fa_off[f]);
      }
    } else {
      constexpr int j = f - 4;
      if constexpr (B_KC) {
        ds_b128<OP_BYTES + 2048 * j>(*reinterpret_cast<u32x4 *>(&fb[SET][j][0]), slot + (fb_off[0] ^ uint32_t(32 * S)));
      } else {
        ds_tr<OP_BYTES + 8192 * S + 2048 * h>(fb[SET][j][h], slot + fb_off[j]);
      }
    }
  }
  // Reads first(n) .. first(n + 1) - 1.
  template <int SET, int S, int N>
  __device__ __forceinline__ void reads_after(uint32_t slot) {
    if constexpr (first(N) < first(N + 1)) { read<SET, S, first(N)>(slot); MHG_ORDER(); }
    if constexpr (first(N) + 1 < first(N + 1)) { read<SET, S, first(N) + 1>(slot); MHG_ORDER(); }
  }
  // Matrix instruction m of a step on set SET (accumulator (m / 2, m % 2)), after the
  // wait for the fragments it needs.
  template <int SET, int M>
  __device__ __forceinline__ void mma() {
    if constexpr (M == 0 || M == 1 || M == 2 || M == 4 || M == 6) { wait_lgkm<allowed(M)>(); MHG_ORDER(); }
    constexpr int i = M >> 1, j = M & 1;
    const u32x4 a = {fa[SET][i][0].x, fa[SET][i][0].y, fa[SET][i][1].x, fa[SET][i][1].y};
    const u32x4 b = {fb[SET][j][0].x, fb[SET][j][0].y, fb[SET][j][1].x, fb[SET][j][1].y};
    acc[i][j] = mfma32(H{}, b, a, acc[i][j]);
  }

  __device__ __forceinline__ uint32_t slot_addr(int t) const { return lds0 + uint32_t(t % SLOTS) * SLOT_BYTES; }
  __device__ __forceinline__ void issue_a(int t, int j) const {
    const int k0 = t * BK;
    oa.issue(oa.rsrc(A, m0, k0), kdim - k0, slot_addr(t), wave, j);
  }
  __device__ __forceinline__ void issue_b(int t, int j) const {
    const int k0 = t * BK;
    ob.issue(ob.rsrc(B, n0, k0), kdim - k0, slot_addr(t) + OP_BYTES, wave, j);
  }

  // Step S of slab t: matrix instructions on set S; after instruction n the next
  // step's reads first(n) .. (into the other set, from slot `rd`), and loads at n = 1
  // and n = 5 (`S == 0`: B of slab t+3, else A of slab t+4).
  template <int S, int N>
  __device__ __forceinline__ void step_from(int t, uint32_t rd) {
    if constexpr (N < 8) {
      mma<S, N>(); MHG_ORDER();
      reads_after<S ^ 1, S ^ 1, N>(rd);
      if constexpr (N == 1 || N == 5) {
        if constexpr (S == 0) issue_b(t + 3, N >> 2);
        else issue_a(t + 4, N >> 2);
        MHG_ORDER();
      }
      step_from<S, N + 1>(t, rd);
    }
  }

  template <int K>
  __device__ __forceinline__ void prologue_reads(uint32_t slot) {
    if constexpr (K < T) { read<0, 0, K>(slot); MHG_ORDER(); prologue_reads<K + 1>(slot); }
  }

  // One 32-deep slab t in two 16-deep steps of 8 matrix instructions.
  //   step 0: multiply set 0 (step 0 of slab t); read step 1 of slab t into set 1;
  //           load B of slab t+3 (its slot held slab t-2, free since the last barrier).
  //   wait for this wave's loads of slab t+1, barrier: slab t+1 is in LDS and every
  //           wave has finished reading slab t-1.
  //   step 1: multiply set 1; read step 0 of slab t+1 into set 0; load A of slab t+4
  //           into the slot of slab t-1.
  // Loads in flight per wave after the wait: slab t+2 and slab t+3 (four each).
  __device__ __forceinline__ void slab(int t) {
    step_from<0, 0>(t, slot_addr(t));
    wait_vm<2 * PER_SLAB>();
    barrier();
    MHG_ORDER();
    step_from<1, 0>(t, slot_addr(t + 1));
  }

  __device__ __forceinline__ void run(uint32_t lds_base) {
    int tm, tn;
    tile_of(blockIdx.x, p.gm, p.gn, p.group_m, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
    lds0 = lds_base;
    const int lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    A = static_cast<const uint16_t *>(p.A);
    B = static_cast<const uint16_t *>(p.B);
    oa.init(p.lda, m0, p.M, wave, lane);
    ob.init(p.ldb, n0, p.N, wave, lane);
    if (A_KC) {
      fa_off[0] = kc_lane(lane) + 2048 * 4 * wm;     // row blocks 4 wm .. 4 wm + 3
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) fa_off[i] = mn_lane(lane, 4 * wm + i);
    }
    if (B_KC) {
      fb_off[0] = kc_lane(lane) + 2048 * 2 * wn;     // column blocks 2 wn, 2 wn + 1
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) fb_off[j] = mn_lane(lane, 2 * wn + j);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
    kdim = int(p.K);
    const int KT = (kdim + BK - 1) / BK;

    // Prologue: slabs 0..2 and A of slab 3 requested (B of slab 3 goes out in slab 0's
    // first step, as in every later slab), in the order the loop's waits assume.
    for (int t = 0; t < 3; ++t) {
      issue_a(t, 0); issue_a(t, 1); issue_b(t, 0); issue_b(t, 1);
    }
    issue_a(3, 0); issue_a(3, 1);
    wait_vm<2 * PER_SLAB + LOADS>();   // slab 0 landed (younger: slabs 1, 2, A of 3)
    wait_lgkm<0>();                    // nothing else counts against lgkmcnt below
    barrier();
    MHG_ORDER();
    prologue_reads<0>(slot_addr(0));

    for (int t = 0; t < KT; ++t) slab(t);
    // Loads past K (zeros) are still writing LDS: drain them before the workgroup ends.
    // The last step's fragment reads are never consumed; the compiler does not know
    // they are in flight, so they must land before their registers are reused.
    wait_vm<0>();
    wait_lgkm<0>();
    MHG_ORDER();

    // acc[i][j] holds the transposed 32 x 32 block: element r of lane l is
    // C[row m0 + 128 wm + 32 i + l % 32][col n0 + 64 wn + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4].
    const int64_t row0 = m0 + wm * WTM + (lane & 31);
    const int64_t colL = n0 + wn * WTN + 4 * (lane >> 5);
    const bool c_vec = p.c_vec != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = row0 + 32 * i;
      if (row >= p.M) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j)
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
};

template <class H, bool A_KC, bool B_KC>
__global__ void __launch_bounds__(NT)
w8_gemm(LaunchArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[SLOTS * SLOT_BYTES];
  W8Gemm<H, A_KC, B_KC> g(p);
  g.run(uint32_t(size_t((MHG_LDS char *)smem)));
}

#define MHG_W8_INST(H)                                            \
  template __global__ void w8_gemm<H, true, false>(LaunchArgs);  \
  template __global__ void w8_gemm<H, true, true>(LaunchArgs);   \
  template __global__ void w8_gemm<H, false, false>(LaunchArgs); \
  template __global__ void w8_gemm<H, false, true>(LaunchArgs);
MHG_W8_INST(HalfBF16)
MHG_W8_INST(HalfF16)
#undef MHG_W8_INST

template <class H>
hipError_t launch_typed(const LaunchArgs &p, hipStream_t s) {
  const dim3 grid(unsigned(p.gm) * unsigned(p.gn)), block(NT);
  if (!p.a_col && !p.b_col) hipLaunchKernelGGL((w8_gemm<H, true, false>), grid, block, 0, s, p);
  else if (!p.a_col && p.b_col) hipLaunchKernelGGL((w8_gemm<H, true, true>), grid, block, 0, s, p);
  else if (p.a_col && !p.b_col) hipLaunchKernelGGL((w8_gemm<H, false, false>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((w8_gemm<H, false, true>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace w8

hipError_t launch_w8(const LaunchArgs &p, hipStream_t s) {
  if (p.in_code == E_BF16) return w8::launch_typed<HalfBF16>(p, s);
  if (p.in_code == E_F16) return w8::launch_typed<HalfF16>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mhg

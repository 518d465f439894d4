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
// Staging keeps two slabs in flight in the 160 KB of LDS:
//   * A slabs are loaded straight into LDS (buffer loads with an LDS destination, the
//     gfx950 counterpart of the asynchronous global-to-shared copy of "Tiling 策略与
//     内存层次优化", cp.async section) into a ring of three 32 KiB slots;
//   * B slabs go through two register sets (each loaded two slabs ahead), are
//     transposed there if B is row-major, and are stored into two 32 KiB LDS slots.
// Each 64-deep slab runs 64 matrix instructions in four groups of 16; between them the
// wave issues the B stores and loads, the A loads, and the LDS reads of the next
// fragments, interleaved instruction by instruction (scheduling-group barriers).  One
// block barrier per slab, issued as s_barrier after an explicit wait that leaves the
// younger loads in flight (the C++ block barrier would wait for all of them).
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
constexpr int TILE_BYTES = 256 * BK * 2;      // one operand's slab: 32 KiB
constexpr uint32_t kOut = 0x80000000u;         // beyond every buffer range: loads zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}

// Byte offset of 16-byte chunk c (0..7) of row r in a K-contiguous 256 x 64 tile (128
// bytes a row), chunks XOR-swizzled per row.  The LDS serves a 16-byte-per-lane access
// 16 lanes at a time from 64 four-byte banks, i.e. 16 distinct 16-byte slots (address
// / 16 mod 16) per cycle; row r starts at slot 8 (r % 2).  The swizzle depends on bits
// 1..4 of r only, so it repeats every 32 rows (a row-block step is a plain offset of
// 4096 bytes), and it spreads over 16 distinct slots both
//   * 16 consecutive rows read at one chunk column (the fragment reads), and
//   * the transposed stores of row-major B (16 lanes: 4 k-chunks x 4 n-rows 8 apart,
//     see GeoBn), which is what its bit-4 term is for.
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 7) ^ ((r >> 2) & 4); }
__device__ __forceinline__ int koff(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }

// LDS accesses through 32-bit LDS addresses, so that every per-lane address is one
// register plus a constant the instruction's 16-bit offset field absorbs.
__device__ __forceinline__ u32x4 lds_ld(uint32_t a) {
  return *reinterpret_cast<const MHG_LDS u32x4 *>(size_t(a));
}
__device__ __forceinline__ void lds_st(uint32_t a, u32x4 v) {
  *reinterpret_cast<MHG_LDS u32x4 *>(size_t(a)) = v;
}
// A copy of x the compiler cannot see through.  Taken once per slab, it keeps the
// per-slab address arithmetic (one XOR or add each) inside the loop instead of
// letting it be hoisted into dozens of loop-invariant registers.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Row-major B (N-contiguous in memory): lane t owns the 8 x 8 block of k-rows
// 8 kg .. +7 and n-columns 8 nc .. +7 of the slab, with (lane l = t % 64 of wave
// w = t / 64) m = l % 4, kg = (l / 4) % 8, nc = 8 w + 4 (l / 32) + m.  Load i reads
// k-row 8 kg + i: every four consecutive lanes read 64 contiguous bytes of one row, so
// a quad of lanes touches one cache line.  The block is transposed in registers and
// stored as 8 n-rows of 8 k-values (n-row 8 nc + jj, k-chunk kg).
struct GeoBn {
  uint32_t off;        // byte offset of k-row 8 kg, n-chunk nc
  uint32_t stride;     // one k-row, in bytes
  int klim;            // k-rows of the matrix at and below 8 kg; very negative if the
                       // lane's columns lie past N
  uint32_t st_base;    // see store_one
  uint32_t sel[2];     // byte selectors of store_one for even and odd j
  __device__ __forceinline__ void init(int64_t ldb, int n0, int64_t N, int64_t K) {
    const int w = threadIdx.x / 64, l = threadIdx.x % 64;
    const int m = l % 4, kg = (l / 4) % 8, nc = 8 * w + 4 * (l / 32) + m, par = m & 1;
    off = uint32_t((int64_t(8 * kg) * ldb + 8 * nc) * 2);
    stride = uint32_t(ldb * 2);
    klim = n0 + 8 * nc < N ? int(min<int64_t>(K - 8 * kg, 1 << 30)) : -(1 << 30);
    st_base = uint32_t(1024 * nc) | uint32_t(128 * par) | uint32_t((kg ^ (4 * ((m ^ (m >> 1)) & 1))) << 4);
    // low halves of both words for an even n-row, high halves for an odd one
    sel[0] = par ? 0x07060302u : 0x05040100u;
    sel[1] = par ? 0x05040100u : 0x07060302u;
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint16_t *B, int64_t ldb, int n0, int k0) const {
    return rsrc_of(B + int64_t(k0) * ldb + n0);
  }
  __device__ __forceinline__ u32x4 load_one(__amdgpu_buffer_rsrc_t rs, int k0, int i) const {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, i < klim - k0 ? off : kOut, int(i * stride), 0);
  }
  // Store j writes n-row jj = j ^ (m % 2) of the lane's block: the 16 lanes of an LDS
  // cycle (k-chunks kg..kg+3, four n-chunks) so cover rows of both parities and, with
  // the swizzle, 16 distinct slots.  Its offset koff(8 nc + jj, kg) is
  // st_base ^ (128 j + 16 (j / 2)), st_base = 1024 nc | 128 (m % 2) |
  // 16 (kg ^ 4 ((m ^ m / 2) % 2)); `base` is st_base.  jj and j share the register word
  // j / 2; the half is picked per lane by the selector.
  __device__ __forceinline__ void store_one(const u32x4 (&r)[8], uint32_t base, uint32_t tile, int j) const {
    const uint32_t s = sel[j & 1];
    const int w = j >> 1;
    u32x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e)   // k = 8 kg + 2e (low half) and 8 kg + 2e + 1 (high half)
      v[e] = __builtin_amdgcn_perm(r[2 * e + 1][w], r[2 * e][w], s);
    lds_st((base ^ uint32_t(128 * j + 16 * (j >> 1))) + tile, v);
  }
};

// Column-major B (K-contiguous): 2048 16-byte chunks, 8 per lane; chunk
// t + 256 i is n-row t / 8 + 32 i, k-chunk t % 8, stored unchanged.
struct GeoBk {
  uint32_t off;        // byte offset of n-row t / 8, k-chunk t % 8
  uint32_t stride;     // 32 n-rows, in bytes
  int rows_left;       // n-rows of the matrix at and below the lane's first
  int klim;            // slabs with k0 < klim have the lane's chunk inside K
  uint32_t st_base;    // koff(t / 8, t % 8)
  __device__ __forceinline__ void init(int64_t ldb, int n0, int64_t N, int64_t K) {
    const int row = threadIdx.x / 8, c = threadIdx.x % 8;
    off = uint32_t((int64_t(row) * ldb + 8 * c) * 2);
    stride = uint32_t(32 * ldb * 2);
    rows_left = int(min<int64_t>(N - n0 - row, 1 << 30));
    klim = int(min<int64_t>(K - 8 * c, 1 << 30));
    st_base = uint32_t(koff(row, c));
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint16_t *B, int64_t ldb, int n0, int k0) const {
    return rsrc_of(B + int64_t(n0) * ldb + k0);
  }
  __device__ __forceinline__ u32x4 load_one(__amdgpu_buffer_rsrc_t rs, int k0, int i) const {
    const int lim = k0 < klim ? rows_left : 0;
    return __builtin_amdgcn_raw_buffer_load_b128(rs, 32 * i < lim ? off : kOut, int(i * stride), 0);
  }
  __device__ __forceinline__ void store_one(const u32x4 (&r)[8], uint32_t base, uint32_t tile, int i) const {
    lds_st(base + tile + 4096 * i, r[i]);
  }
};

// A's slab (K-contiguous) loaded straight into LDS.  A load instruction of a wave
// fills 64 consecutive 16-byte slots: load j of wave w covers rows 32 j + 8 w .. +7,
// lane l the row 32 j + 8 w + l / 8 and LDS slot l % 8 of it, which holds the row's
// k-chunk (l % 8) ^ swz(row) -- the XOR swizzle of koff applied on the global side.
struct DmaA {
  uint32_t off;        // byte offset of this lane's chunk for j = 0, from the slab origin
  uint32_t stride;     // 32 rows, in bytes
  int rows_left;       // rows of the matrix at and below this lane's first row
  int klim;            // slabs with k0 < klim have this lane's chunk inside K
  __device__ __forceinline__ void init(int64_t lda, int m0, int64_t M, int64_t K) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int row = 8 * wave + lane / 8, c = (lane % 8) ^ swz(row);
    off = uint32_t((int64_t(row) * lda + 8 * c) * 2);
    stride = uint32_t(32 * lda * 2);
    rows_left = int(min<int64_t>(M - m0 - row, 1 << 30));
    klim = int(min<int64_t>(K - 8 * c, 1 << 30));
  }
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const uint16_t *A, int64_t lda, int m0, int k0) const {
    return rsrc_of(A + int64_t(m0) * lda + k0);
  }
  // Rows of the slab at k0 this lane may load: 0 when its chunk lies past K.
  __device__ __forceinline__ int lim(int k0) const { return k0 < klim ? rows_left : 0; }
  // Load j of the slab (resource rs, row limit l) into the LDS tile at `dst`.  `dst`
  // and `wave` are wave-uniform: the LDS destination of these loads is a scalar register.
  __device__ __forceinline__ void issue_one(__amdgpu_buffer_rsrc_t rs, int l, uint32_t dst, uint32_t wave,
                                            int j) const {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (MHG_LDS void *)(size_t)(dst + (4 * j + wave) * 1024), 16,
                                             32 * j < l ? off : kOut, int(j * stride), 0, 0);
  }
  __device__ __forceinline__ void issue(const uint16_t *A, int64_t lda, int m0, int k0, uint32_t dst,
                                        uint32_t wave) const {
    const __amdgpu_buffer_rsrc_t rs = rsrc(A, lda, m0, k0);
    const int l = lim(k0);
#pragma unroll
    for (int j = 0; j < 8; ++j) issue_one(rs, l, dst, wave, j);
  }
};

// s_waitcnt with vmcnt = n and lgkmcnt = 0 (expcnt free), then the block barrier.
template <int n>
__device__ __forceinline__ void wait_vm_lgkm_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));
  asm volatile("s_barrier" ::: "memory");
}
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8)); }
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14)); }
// Nothing moves across it: the instruction order of a phase is the source order.
#define MHG_ORDER() __builtin_amdgcn_sched_barrier(0)

// LDS map: B slabs in slots 0 and 1 (slab s in slot s % 2), the A ring in slots 2..4
// (slab s in slot 2 + s % 3); a slot is one 256 x 64 K-contiguous tile (32 KiB).  B's
// slots come first so that their offsets fit the LDS instructions' offset field.
template <class H, bool B_KC>
struct BigGemm {
  using GeoB = typename std::conditional<B_KC, GeoBk, GeoBn>::type;
  const LaunchArgs &p;
  const uint16_t *A, *B;
  int m0, n0, KT;
  uint32_t lds0;                 // LDS address of slot 0
  uint32_t wave;                 // wave index, wave-uniform
  uint32_t fa_base, fb_base;     // koff of the lane's fragment rows for k-half 0
  DmaA da;
  GeoB gb;
  u32x4 rb[4][8];                // B register sets: slab s is staged in set s % 4
  f32x16 acc[4][4];
  // Fragments of one k-half (16 deep): 4 row blocks of A, 4 column blocks of B.  Phase
  // p of a slab multiplies the half in set p % 2 while the next half is read into the
  // other set, so 64 registers hold all fragments.
  u32x4 fa[2][4], fb[2][4];

  __device__ __forceinline__ BigGemm(const LaunchArgs &p_) : p(p_) {}

  __device__ __forceinline__ uint32_t a_slot(int slab) const { return lds0 + (2 + slab % 3) * TILE_BYTES; }

  // Fragment of row block i, k-half q (q = 0..3 over the slab): the lane reads row
  // (lane % 32) of the block and k-chunk 2 q + lane / 32, i.e. koff(row, chunk) =
  // base ^ (32 q) + 4096 i with base = koff(row, lane / 32).
  template <int SET>
  __device__ __forceinline__ void read_half(uint32_t ab, uint32_t bb, uint32_t ta, uint32_t tb, int q) {
    const uint32_t xa = (ab ^ uint32_t(q << 5)) + ta, xb = (bb ^ uint32_t(q << 5)) + tb;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[SET][i] = lds_ld(xa + 4096 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[SET][j] = lds_ld(xb + 4096 * j);
  }
  template <int SET>
  __device__ __forceinline__ void load_b(int k0) {
    const __amdgpu_buffer_rsrc_t rs = gb.rsrc(B, p.ldb, n0, k0);
#pragma unroll
    for (int i = 0; i < 8; ++i) rb[SET][i] = gb.load_one(rs, k0, i);
  }
  template <int SET>
  __device__ __forceinline__ void store_b(uint32_t base, uint32_t tile) {
#pragma unroll
    for (int j = 0; j < 8; ++j) gb.store_one(rb[SET], base, tile, j);
  }

  // Matrix instruction n (0..15) of a k-half: accumulator (n / 4, n % 4).
  template <int SET>
  __device__ __forceinline__ void mma(int n) {
    const int i = n >> 2, j = n & 3;
    acc[i][j] = mfma32(H{}, fb[SET][j], fa[SET][i], acc[i][j]);
  }
  // LDS read n (0..7) of a k-half: A row block n for n < 4, else B column block n - 4;
  // xa, xb are the half's lane offsets (half_off).
  template <int SET>
  __device__ __forceinline__ void read_one(uint32_t xa, uint32_t xb, int n) {
    if (n < 4) fa[SET][n] = lds_ld(xa + 4096 * n);
    else fb[SET][n - 4] = lds_ld(xb + 4096 * (n - 4));
  }
  __device__ __forceinline__ static uint32_t half_off(uint32_t base, int q, uint32_t tile) {
    return (base ^ uint32_t(q << 5)) + tile;
  }

  // One 64-deep slab t: four phases of 16 matrix instructions, each multiplying the
  // k-half in fragment set p % 2 while the next half is read into the other set, with
  // one global or LDS operation after every other matrix instruction.  The order inside
  // a phase is fixed (MHG_ORDER between steps) so that the matrix pipe never waits
  // behind a burst of memory instructions.  Every phase starts by waiting for the LDS
  // operations of the previous one (issued a whole phase earlier): the LDS counter
  // saturates at 15, and without that wait a fragment consumed late in a phase would
  // also wait for the reads and writes issued early in it.
  //
  // Global traffic is spread evenly, four loads per wave and phase: A slab t+2 in
  // phases 0 and 1 (into the ring slot of slab t-1, free since the previous barrier;
  // it must have landed by the barrier of slab t+1), B slab t+4 in phases 2 and 3 into
  // register set t % 4, which slab t left in the previous slab.  B slab t+1 is
  // transposed out of its set into its LDS slot over phases 0..2.
  //
  // S = t % 4.  On entry: fragment set 0 holds k-half 0 of slab t; A slab t is in LDS
  // and A slab t+1 in flight; B slab t is in LDS and slabs t+1..t+3 are in (or on their
  // way into) register sets (S+1..S+3) % 4.
  template <int S>
  __device__ __forceinline__ void slab(int t) {
    constexpr int BS = (S + 1) & 3;                 // register set of B slab t+1
    const uint32_t ab = opaque(fa_base), bb = opaque(fb_base), sbase = opaque(gb.st_base);
    const uint32_t ca = a_slot(t), cb = lds0 + (S & 1) * TILE_BYTES, nb = lds0 + ((S + 1) & 1) * TILE_BYTES;
    const int ka = (t + 2) * BK, kb = (t + 4) * BK;
    const __amdgpu_buffer_rsrc_t ra = da.rsrc(A, p.lda, m0, ka);
    const __amdgpu_buffer_rsrc_t rbs = gb.rsrc(B, p.ldb, n0, kb);
    const int la = da.lim(ka);
    const uint32_t adst = a_slot(t + 2);
    // Phase 0: A loads 0..3, B stores 0..2.
    wait_lgkm0();
    MHG_ORDER();
    {
      const uint32_t xa = half_off(ab, 1, ca), xb = half_off(bb, 1, cb);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        mma<0>(2 * k); MHG_ORDER();
        read_one<1>(xa, xb, k); MHG_ORDER();
        mma<0>(2 * k + 1); MHG_ORDER();
        if (k % 2 == 0) { da.issue_one(ra, la, adst, wave, k / 2); MHG_ORDER(); }
        else if (k < 7) { gb.store_one(rb[BS], sbase, nb, k / 2); MHG_ORDER(); }
      }
    }
    // Phase 1: A loads 4..7, B stores 3..5.
    wait_lgkm0();
    MHG_ORDER();
    {
      const uint32_t xa = half_off(ab, 2, ca), xb = half_off(bb, 2, cb);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        mma<1>(2 * k); MHG_ORDER();
        read_one<0>(xa, xb, k); MHG_ORDER();
        mma<1>(2 * k + 1); MHG_ORDER();
        if (k % 2 == 0) { da.issue_one(ra, la, adst, wave, 4 + k / 2); MHG_ORDER(); }
        else if (k < 7) { gb.store_one(rb[BS], sbase, nb, 3 + k / 2); MHG_ORDER(); }
      }
    }
    // Phase 2: B loads 0..3 of slab t+4, B stores 6 and 7.
    wait_lgkm0();
    MHG_ORDER();
    {
      const uint32_t xa = half_off(ab, 3, ca), xb = half_off(bb, 3, cb);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        mma<0>(2 * k); MHG_ORDER();
        read_one<1>(xa, xb, k); MHG_ORDER();
        mma<0>(2 * k + 1); MHG_ORDER();
        if (k % 2 == 0) { rb[S][k / 2] = gb.load_one(rbs, kb, k / 2); MHG_ORDER(); }
        else if (k < 5) { gb.store_one(rb[BS], sbase, nb, 6 + k / 2); MHG_ORDER(); }
      }
    }
    // A slab t+1 landed: the loads issued after its last one are slab t-1's 8 B loads,
    // this slab's 8 A loads and its first 4 B loads.  Every wave stored B slab t+1 and
    // finished reading slab t.
    wait_vm_lgkm_barrier<20>();
    MHG_ORDER();
    // Phase 3: k-half 0 of slab t+1 read; B loads 4..7 of slab t+4.
    {
      const uint32_t xa = half_off(ab, 0, a_slot(t + 1)), xb = half_off(bb, 0, nb);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        mma<1>(2 * k); MHG_ORDER();
        read_one<0>(xa, xb, k); MHG_ORDER();
        mma<1>(2 * k + 1); MHG_ORDER();
        if (k % 2 == 0) { rb[S][4 + k / 2] = gb.load_one(rbs, kb, 4 + k / 2); MHG_ORDER(); }
      }
    }
  }

  __device__ __forceinline__ void run(uint32_t lds_base) {
    int tm, tn;
    tile_of(blockIdx.x, p.gm, p.gn, p.group_m, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
    lds0 = lds_base;
    const int lane = threadIdx.x & 63;
    wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    fa_base = uint32_t(koff(wm * WTM + (lane & 31), lane >> 5));
    fb_base = uint32_t(koff(wn * WTN + (lane & 31), lane >> 5));
    A = static_cast<const uint16_t *>(p.A);
    B = static_cast<const uint16_t *>(p.B);
    const int64_t K = p.K;
    KT = int((K + BK - 1) / BK);
    da.init(p.lda, m0, p.M, K);
    gb.init(p.ldb, n0, p.N, K);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

    // Prologue: B slab 0 through set 0 into slot 0, A slabs 0 and 1 requested, B slabs
    // 1..3 into sets 1..3, in the order the loop's waits assume (A slab 1 before the
    // last eight B loads).  Past K every load reads zeros, so the loop body has no
    // branches and issues the same loads in every slab.
    load_b<0>(0);
    da.issue(A, p.lda, m0, 0, a_slot(0), wave);
    load_b<1>(BK);
    load_b<2>(2 * BK);
    wait_vm0();
    store_b<0>(gb.st_base, lds0);
    da.issue(A, p.lda, m0, BK, a_slot(1), wave);
    load_b<3>(3 * BK);
    wait_vm_lgkm_barrier<16>();    // A slab 0 came before the wait above
    read_half<0>(fa_base, fb_base, a_slot(0), lds0, 0);

    // Four slabs per trip (register-set and LDS-slot indices are compile-time); the
    // last KT % 4 slabs are peeled.  A conditional slab inside the loop would merge two
    // copies of the 256 accumulators at the loop's end, which the register allocator
    // resolves with spills.
    int t = 0;
    for (; t + 3 < KT; t += 4) {
      slab<0>(t);
      slab<1>(t + 1);
      slab<2>(t + 2);
      slab<3>(t + 3);
    }
    if (t < KT) {
      slab<0>(t);
      if (t + 1 < KT) {
        slab<1>(t + 1);
        if (t + 2 < KT) slab<2>(t + 2);
      }
    }
    // Loads still in flight write LDS: drain them before the workgroup ends.
    wait_vm0();

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
          f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          if (p.epi) v = epilogue4(p, v, row, col, n_in);
          store_out4(p.C, row * p.ldc + col, v, p.out_code, c_vec && n_in >= 4, int(n_in));
        }
    }
  }
};

template <class H, bool B_KC>
__global__ void __launch_bounds__(NT)
big_gemm(LaunchArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[5 * TILE_BYTES];
  BigGemm<H, B_KC> g(p);
  g.run(uint32_t(size_t((MHG_LDS char *)smem)));
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

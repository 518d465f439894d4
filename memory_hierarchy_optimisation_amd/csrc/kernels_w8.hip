// kernels_w8.hip -- fp16 / bf16 GEMM for large aligned problems: eight waves (two per
// SIMD) in a ping-pong schedule, both operands loaded straight into a five-slot LDS
// ring of K slabs.  Three tile shapes:
//   * 256 x 256, 32-deep slabs: the two wave groups split the tile's rows, each wave
//     owns 128 x 64 of C (8 x 4 accumulators of 16 x 16);
//   * 128 x 128, 64-deep slabs: the two wave groups take alternate slabs (group 0 the
//     even ones, group 1 the odd ones), each wave owns 64 x 64 of C (4 x 4
//     accumulators), and the two partial sums of a block are added through LDS at the
//     end;
//   * 64 x 64, 128-deep slabs: as 128 x 128, with 32 x 32 of C per wave.
// Every slab is 32 KiB (16 KiB of A at +0, 16 KiB of B at +16 KiB), so all shapes use
// the same ring: five slots, 160 KB, four slabs requested ahead.  One exception: the
// 256 x 256 tile with both operands K-contiguous (row-major A, column-major B) keeps A
// in a ring of slab pairs (whole 128-byte rows; a single 32-deep slab would request
// half lines) beside a ring of B slabs.
//
// The three tiling levels of "Tiling 策略与内存层次优化" (multi-level tiling) sized for
// gfx950:
//   * workgroup tile: 256 x 256 has tile intensity 2*256*256 / (512*2) = 128 FLOP/B
//     (same page, how tiling raises intensity) and covers 4096^2 with one tile per
//     compute unit; 128 x 128 (64 FLOP/B) covers 2048^2 the same way and 64 x 64
//     (32 FLOP/B) covers 1024^2, where the product is short and load latency, not
//     reuse, decides: four 128-deep slabs in flight are half of K;
//   * K slabs in a ring of five 32 KiB LDS slots (constraint 1 of the same page with
//     stages = 5), requested four slabs ahead with 16-byte LDS-destination buffer
//     loads, the gfx950 counterpart of cp.async (cp.async section);
//   * eight waves, two per SIMD, each with a register tile of 16 x 16 accumulator blocks
//     of v_mfma_f32_16x16x32_{bf16,f16} ("寄存器Tiling", 1.3: the register budget trades
//     tile size for resident waves; 128, 64 or 16 fp32 accumulators a lane).  The
//     16 x 16 instruction does the same work per cycle as the 32 x 32 one but moves half
//     the accumulator bytes per multiply-add; on random data the chip, at its power
//     limit, holds a higher clock with it (a stream of either instruction alone: 2.03 vs
//     1.76 GHz; these kernels at 4096^3: 1.74-1.77 vs 1.51-1.63 GHz).
// Ping-pong: the waves form two groups, one wave of each per SIMD.  Block barriers
// cut time into phases; in each phase one group runs the matrix instructions of a
// slab back to back while the other group reads its fragments of the next slab from
// LDS (at 256 x 256 each group also loads one operand of every slab in its memory
// phase; at 128 x 128 and 64 x 64 a group requests both operands of its own slabs
// between its matrix instructions).  A phase holds 32 matrix instructions per wave (16
// at 64 x 64).  A
// wave that interleaves its own loads with its matrix instructions stalls at them, and
// a SIMD whose two waves do the same thing at the same time stalls with them; here the
// matrix pipe of every SIMD is fed by one wave while the other waits on memory.
// Operands are stored in LDS in their global orientation:
//   * a K-contiguous operand (row-major A, column-major B) as rows of BK values; each
//     fragment is one 16-byte LDS read per lane;
//   * an M/N-contiguous operand (column-major A, row-major B) as k-rows of the tile's
//     width; each fragment is two LDS transpose reads (ds_read_b64_tr_b16), so the
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
//
// Output: the accumulators go through LDS once the ring is free, so that every store
// writes whole row segments of C (write-through stores: C is written once).  A fused
// epilogue (alpha, beta times the prior C, bias, ReLU) runs there in fp32 before the
// one rounding.  The 256 x 256 tile has a second instantiation for a 16-bit prior C:
// the four slab requests past K load the prior C tile into the ring instead of zeros,
// so its reads overlap the last slabs' arithmetic.
#include <type_traits>

#include "device.h"

namespace mhg {
namespace w8 {

constexpr int NT = 512, SLOTS = 5;
constexpr int OP_BYTES = 16384;                 // one operand's slab (both shapes)
constexpr int SLOT_BYTES = 2 * OP_BYTES;        // A at +0, B at +16 KiB
constexpr int GROUP = 4;                        // waves of a group (one per SIMD)
constexpr int LOADS = OP_BYTES / (GROUP * 64 * 16);   // 16-byte loads per lane of a slab's operand (4)
constexpr int AHEAD = 4;                        // slab t+4 is requested while slab t is read
constexpr uint32_t kOut = 0x80000000u;          // beyond every buffer range: loads zeros

// The tile shapes.  A wave's block of C is 32 FM x 32 FN (2 FM x 2 FN accumulators of
// 16 x 16); KSPLIT = 2: the groups take alternate slabs (halves of K) instead of halves
// of the rows.
// PAIRA: with A row-major and B column-major, the 256 x 256 tile brings A in pairs of
// slabs, whole 128-byte rows (see the pair ring below).
struct Tile256 { static constexpr int BM = 256, BN = 256, BK = 32, FM = 4, FN = 2, KSPLIT = 1; static constexpr bool PAIRA = true; };
struct Tile128 { static constexpr int BM = 128, BN = 128, BK = 64, FM = 2, FN = 2, KSPLIT = 2; static constexpr bool PAIRA = false; };
struct Tile64 { static constexpr int BM = 64, BN = 64, BK = 128, FM = 1, FN = 1, KSPLIT = 2; static constexpr bool PAIRA = false; };

// Cache-policy bits of a buffer store: sc1, the device-scope (write-through) form.
constexpr int kStoreDeviceScope = 16;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const void *base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, 0x7fffffff, 0x00020000);
}

// LDS layouts of one operand's slab (byte offsets within its 16 KiB), for a tile side
// of R rows (m or n) and slabs BK deep:
//   K-contiguous: row r (0..R-1) of BK/8 16-byte k-chunks; chunk c at
//     r * 2BK + 16 (c ^ kswz(r)).  A fragment read has lane l read chunk l / 16 of row
//     l % 16 (plus the block's and step's offsets).  The LDS serves a 16-byte read in four
//     passes of 16 lanes: the four-lane quads of one half-wave (lane bit 5) whose quad
//     index has the same parity (bits 2 ^ 3 ^ 4), e.g. lanes 0-3, 12-15, 20-23 and 24-27
//     (measured on the MI355X with the LDS conflict counter: one lane pair per dispatch
//     at the same banks, the rest broadcasting).  In a pass, row bits 0 and 1 and two of
//     bits 2, 3 and 4 vary; kswz puts its 16 reads on distinct 16-byte bank groups.  With
//     4 chunks a row (4 rows per 256 bytes of banks) kswz(r) = 2 ((r >> 3) & 1): then
//     chunk bit 0 follows bit 2 ^ 3 ^ 4 ^ parity and chunk bit 1 bit 3, which separate
//     the four (bit 2, bit 3) choices (the plain (r >> 2) & 3 left only bit 3 and
//     conflicted two-way); (r >> 1) & 7 for 8 chunks and r & 15 for 16 separate them
//     already.
//   M/N-contiguous: k-row k (0..BK-1) of R/8 chunks of 8 m/n-values; chunk c at
//     k * 2R + 16 (c ^ mswz(k)).  The 32 lanes of a transpose read served together read
//     32 bytes of the same columns in each of four consecutive k-rows k0 + q and of four
//     more, k0 + 8 + q (their fragments' k differ by 8).  mswz(k) = 4 (k & 3) moves 512-
//     or 256-byte k-rows to four distinct quarters of the banks (4 ((k >> 1) & 1) the
//     128-byte k-rows of the 64-wide tile, whose rows k and k+1 already sit half the
//     banks apart), and the term 2 ((k >> 3) & 1) puts the second four k-rows in the
//     other half of each quarter.
template <int BK>
__device__ __forceinline__ constexpr int kswz(int r) {
  return BK == 32 ? 2 * ((r >> 3) & 1) : BK == 64 ? (r >> 1) & 7 : r & 15;
}
template <int R>
__device__ __forceinline__ constexpr int mswz(int k) {
  return (R >= 128 ? 4 * (k & 3) : 4 * ((k >> 1) & 1)) ^ (2 * ((k >> 3) & 1));
}
template <int BK>
__device__ __forceinline__ uint32_t kc_off(int r, int c) { return uint32_t(r * 2 * BK + 16 * (c ^ kswz<BK>(r))); }
template <int R>
__device__ __forceinline__ uint32_t mn_off(int k, int c) { return uint32_t(k * 2 * R + 16 * (c ^ mswz<R>(k))); }

// A 64-bit value as the first lane holds it.  The builtin reads 32 bits and returns a
// signed int: each half goes back to unsigned before it is widened, or a low half with
// bit 31 set would sign-extend over the high half.
__device__ __forceinline__ uint64_t first_lane_u64(uint64_t v) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v))));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(v >> 32))));
  return (uint64_t(hi) << 32) | uint64_t(lo);
}

// The slab loads of one wave for one operand.  The four waves of a group fill an
// operand's 16 KiB slab: load j of group wave w fills LDS bytes b * 1024 .. +1023 of
// it, b = 4 j + w (loads of one index side by side) or, with OWN, b = 4 w + j (a
// wave's four loads side by side: at 256 x 256 with a K-contiguous operand that is
// exactly the 64 rows whose fragments the wave reads); lane l writes chunk slot
// b * 64 + l and loads the chunk that belongs there.
struct Loader {
  uint32_t off[LOADS];   // byte offset of the lane's chunk from the slab origin, per load
  int kin[LOADS];        // k of the chunk within the slab; 2^30 when its rows (m or n)
                         // lie outside the matrix, so that it is never loaded
  const uint16_t *origin0;   // slab origin at k = 0 (wave-uniform)
  int64_t kstep;             // elements between the origins of consecutive k (1 or ld)
  uint32_t lds_off;          // the operand's area in a slot (0: A, OP_BYTES: B)
  // KC: the operand is K-contiguous (rows of m or n with k inside), else M/N-contiguous;
  // R: the tile's extent in m or n.
  template <bool OWN>
  static __device__ __forceinline__ int block_of(int wave, int j) { return OWN ? GROUP * wave + j : GROUP * j + wave; }
  template <bool KC, int R, int BK, bool OWN = false>
  __device__ __forceinline__ void init(const uint16_t *g, int64_t ld, int mn0, int64_t MN, int wave, int lane,
                                       uint32_t area) {
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int slot = block_of<OWN>(wave, j) * 64 + lane;
      if (KC) {
        constexpr int CPR = BK / 8;                       // chunks a row
        const int r = slot / CPR, c = (slot % CPR) ^ kswz<BK>(r);
        off[j] = uint32_t((int64_t(r) * ld + 8 * c) * 2);
        kin[j] = mn0 + r < MN ? 8 * c : 1 << 30;
      } else {
        constexpr int CPK = R / 8;                        // chunks a k-row
        const int k = slot / CPK, c = (slot % CPK) ^ mswz<R>(k);
        off[j] = uint32_t((int64_t(k) * ld + 8 * c) * 2);
        kin[j] = mn0 + 8 * c < MN ? k : 1 << 30;
      }
    }
    // Both are the same on every lane; reading them through the first lane tells the
    // compiler so, which keeps the buffer resource built from them in scalar registers
    // (a resource it takes for per-lane wraps every load in a loop over lanes).
    origin0 = reinterpret_cast<const uint16_t *>(
        first_lane_u64(reinterpret_cast<uint64_t>(KC ? g + int64_t(mn0) * ld : g + mn0)));
    kstep = int64_t(first_lane_u64(uint64_t(KC ? int64_t(1) : ld)));
    lds_off = area;
  }
  // Load j of the slab at k0 into `slot` (wave-uniform; so is `wave`, the wave's index
  // in its group: the LDS destination of these loads is a scalar register).  OWN as
  // in init.
  template <bool OWN = false>
  __device__ __forceinline__ void issue(int k0, int k_left, uint32_t slot, uint32_t wave, int j) const {
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(origin0 + k0 * kstep);
    const bool in = kin[j] < k_left;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (MHG_LDS void *)(size_t)(slot + lds_off + uint32_t(block_of<OWN>(int(wave), j)) * 1024), 16,
        in ? off[j] : kOut, 0, 0, 0);
  }
};

// A row-major A in pairs of slabs (PAIRA): the tile's 256 rows of 2 BK = 64 values, 128
// bytes, in two 16 KiB halves of 128 rows; load j of wave w in half h brings rows
// 128 h + 32 j + 8 w .. + 7, lane l the chunk (l % 8) ^ kswz(row) of row 128 h + 32 j +
// 8 w + l / 8.  The swizzle of a row depends on its bits 1..3 only, so a lane's chunk is
// the same for every load and both halves, and a load's offset is the lane's base plus
// a wave-uniform multiple of the leading dimension.
struct PairLoader {
  uint32_t base;             // lane's byte offset at row 8 w + l / 8, its chunk
  int rows_left;             // M - (tile row of that lane's first row)
  int kc;                    // k of the lane's chunk within the pair (8 c)
  const uint16_t *origin0;   // A at the tile's first row, k = 0 (wave-uniform)
  int64_t ld2;               // 2 * lda (bytes per row, wave-uniform)
  __device__ __forceinline__ void init(const uint16_t *g, int64_t ld, int m0, int64_t M, int wave, int lane) {
    const int r0 = 8 * wave + (lane >> 3), c = (lane & 7) ^ kswz<64>(r0);
    base = uint32_t((int64_t(r0) * ld + 8 * c) * 2);
    rows_left = int(M - m0 < (int64_t(1) << 30) ? M - m0 : (int64_t(1) << 30)) - r0;
    kc = 8 * c;
    origin0 = reinterpret_cast<const uint16_t *>(first_lane_u64(reinterpret_cast<uint64_t>(g + int64_t(m0) * ld)));
    ld2 = int64_t(first_lane_u64(uint64_t(2 * ld)));
  }
  __device__ __forceinline__ void issue(int k0, int k_left, uint32_t dst, uint32_t wave, int j, int h) const {
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(origin0 + k0);
    const int row = 128 * h + 32 * j;
    const bool in = row < rows_left && kc < k_left;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (MHG_LDS void *)(size_t)(dst + uint32_t(h) * 16384u + (GROUP * j + wave) * 1024), 16,
        in ? base + uint32_t(int64_t(row) * ld2) : kOut, 0, 0, 0);
  }
};

// Fragment addressing.  A 16 x 32 fragment (16 rows of m or n, 32 k) for
// v_mfma_f32_16x16x32: lane l holds row l % 16, k = 8 (l / 16) .. +7 of the 32-deep
// step s.
//   K-contiguous: one 16-byte read at kc_off(16 b + l % 16, 4 s + l / 16).  The swizzle
//     term depends on the row's bits 0..3 only, i.e. on the lane (16 b leaves them
//     alone), and (4 s + l / 16) ^ x = 4 s ^ (l / 16 ^ x) since 4 s has no bit in common
//     with l / 16, so step s is an XOR of 64 s on the lane's offset (below the row's 2BK
//     bytes: only slabs 64 or more deep have a second step) and block b a constant
//     16 b * 2BK.
//   M/N-contiguous: two transpose reads (e = 0, 1) for k = 8 (l / 16) + 4 e .. +3.  In
//     each 16-lane group g = l / 16, lane 4 q + u addresses the 8 bytes of k-row
//     32 s + 8 g + 4 e + q, columns 16 b + 4 u .. +3, and lane t then receives column
//     16 b + t of those four k-rows; step s adds 32 s * 2R and e adds 4 * 2R to the
//     lane's offset for step 0, e = 0 (mswz depends on k's bits 0, 1 and 3, which are
//     q's and g's).
template <int BK>
__device__ __forceinline__ uint32_t kc_lane(int lane) { return kc_off<BK>(lane & 15, lane >> 4); }
template <int R>
__device__ __forceinline__ uint32_t mn_lane(int lane, int b) {
  const int g = lane >> 4, t = lane & 15, q = t >> 2, u = t & 3;
  const int k = 8 * g + q;
  const int c = 2 * b + (u >> 1);
  return mn_off<R>(k, c) + 8 * (u & 1);
}

// LDS reads of the fragments, issued as plain instructions.  The compiler would treat
// a transpose read as possibly aliasing the LDS-destination loads in flight and wait
// for all of them; the ring's waits and barriers already order those accesses, so
// these reads are not shown to it as memory accesses, and their completion is awaited
// explicitly (lgkmcnt) before any instruction consumes them.
template <int OFF>
__device__ __forceinline__ void ds_b128(u32x4 &d, uint32_t a) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(d) : "v"(a), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void ds_tr(u32x2 &d, uint32_t a) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(d) : "v"(a), "i"(OFF));
}
// s_waitcnt with only lgkmcnt = n, or only vmcnt = n.
template <int n>
__device__ __forceinline__ void wait_lgkm() {
  static_assert(n >= 0 && n < 16, "lgkmcnt field");
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (n << 8));
}
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }
#define MHG_ORDER() __builtin_amdgcn_sched_barrier(0)

// PRIOR (256 x 256 only): the fused epilogue reads a 16-bit prior C, which arrives in
// LDS through the ring's last four slab loads.
template <class H, bool A_KC, bool B_KC, class TL, bool PRIOR>
struct W8Gemm {
  static constexpr int BM = TL::BM, BN = TL::BN, BK = TL::BK, FM = TL::FM, FN = TL::FN;
  static constexpr bool ALT = TL::KSPLIT == 2;           // groups take alternate slabs
  static constexpr int STEPS = BK / 32;                  // 32-deep steps of a slab
  static constexpr int WTM = 32 * FM, WTN = 32 * FN;      // a wave's block of C
  static constexpr int MB = 2 * FM, NBL = 2 * FN;         // its 16 x 16 blocks
  static_assert(BM * BK * 2 == OP_BYTES && BN * BK * 2 == OP_BYTES, "slab size");
  static_assert(!PRIOR || (!ALT && FM == 4 && FN == 2), "prior C through LDS: 256 x 256 tile only");
  // PA: A (row-major) in a ring of three 32 KiB pair slots, each the tile's 256 rows of
  // 2 BK values (128 bytes) of two consecutive slabs; B in a ring of four 16 KiB slots.
  // A 32-deep slab holds only 64 bytes of a K-contiguous row, so its loads are half-line
  // requests; in pairs they are whole lines.  Used when B is K-contiguous as well
  // (column-major), where it measured 1157 -> 1207 TFLOP/s at 4096^3 bf16 (about 2%
  // more with B four slabs ahead, its slot refilled right after group 1's reads); with
  // B row-major it was slower either way (1317 -> 1256 with B four ahead).
  static constexpr bool PA = TL::PAIRA && !ALT && A_KC && B_KC && !PRIOR;
  static constexpr int BKA = PA ? 2 * BK : BK;            // k values in an LDS row of A
  static constexpr uint32_t PA_B = 3 * 32768;              // byte offset of the B ring

  const LaunchArgs &p;
  int m0, n0;
  int kdim;                   // K (below 2^31 by the plan's validation)
  uint32_t lds0;
  uint32_t grp, gw;           // group (0: waves 0-3, 1: waves 4-7), wave within the group
  int wm, wn;                 // the wave's block of C: rows WTM wm, columns WTN wn
  // 256 x 256: ld is the group's operand (group 0 A, group 1 B); 128 x 128: ld is A and
  // ld2 B of the group's own slabs.
  Loader ld, ld2;
  PairLoader lp;              // PA: group 0's loader of A
  uint32_t fa_cur;            // fa_off[0] with the slab's half of an A pair applied (PA)
  // Lane offsets of the fragment reads within an operand slab (step 0), the wave's
  // block offset included: K-contiguous operands use [0] (step s is [0] ^ 64 s, block i
  // adds 32 BK i); M/N-contiguous ones one per block (step s adds 32 s k-rows).
  uint32_t fa_off[MB], fb_off[NBL];
  f32x4 acc[MB][NBL];
  // The fragments of one slab, [step][block][half] (k 0..3 and 4..7 of the lane's
  // eight): a 16-byte read fills both halves, a transpose read one.
  u32x2 fa[STEPS][MB][2], fb[STEPS][NBL][2];

  static constexpr int NA = A_KC ? 1 : 2, NB = B_KC ? 1 : 2;
  static constexpr int T = NBL * NB + MB * NA;           // LDS reads per step

  __device__ __forceinline__ W8Gemm(const LaunchArgs &p_) : p(p_) {}

  // Read k of a step: the B blocks, then the A blocks; a fragment is one read if
  // K-contiguous, two if M/N-contiguous.  Returns the fragment (0 .. MB-1: A block,
  // MB ..: B block).
  static constexpr int read_frag(int k) { return k < NBL * NB ? MB + k / NB : (k - NBL * NB) / NA; }
  static constexpr int read_half(int k) { return k < NBL * NB ? k % NB : (k - NBL * NB) % NA; }
  // Read k of the wave's step S from the slab whose A area is `slot`.
  template <int S, int K>
  __device__ __forceinline__ void read(uint32_t sa, uint32_t slot) {
    constexpr int f = read_frag(K), h = read_half(K);
    if constexpr (f < MB) {
      if constexpr (A_KC) {
        ds_b128<32 * BKA * f>(*reinterpret_cast<u32x4 *>(&fa[S][f][0]), sa + (fa_cur ^ uint32_t(64 * S)));
      } else {
        ds_tr<32 * S * 2 * BM + 4 * 2 * BM * h>(fa[S][f][h], sa + fa_off[f]);
      }
    } else {
      constexpr int j = f - MB;
      if constexpr (B_KC) {
        ds_b128<OP_BYTES + 32 * BK * j>(*reinterpret_cast<u32x4 *>(&fb[S][j][0]), slot + (fb_off[0] ^ uint32_t(64 * S)));
      } else {
        ds_tr<OP_BYTES + 32 * S * 2 * BN + 4 * 2 * BN * h>(fb[S][j][h], slot + fb_off[j]);
      }
    }
  }
  // Reads K .. T-1 of step S, back to back.
  template <int S, int K>
  __device__ __forceinline__ void reads_from(uint32_t sa, uint32_t slot) {
    if constexpr (K < T) {
      read<S, K>(sa, slot); MHG_ORDER();
      reads_from<S, K + 1>(sa, slot);
    }
  }
  // Every load of slab t this wave makes (prologue).
  __device__ __forceinline__ void issue_all(int t) const {
    const int k0 = t * BK;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      if (ALT) {
        ld.issue(k0, kdim - k0, slot_addr(t), gw, j);
        ld2.issue(k0, kdim - k0, slot_addr(t), gw, j);
      } else {
        load(t, slot_addr(t), j);
      }
    }
  }

  // Load j of the group's operand of slab t (256 x 256).  The four slabs past K would
  // load zeros; with the prior C in LDS (PRIOR), slab KT + q loads quarter q of
  // the tile's prior C instead: rows 64 q .. 64 q + 63, group g the 32 rows from
  // 64 q + 32 g, into the same half of the same slot and with the same number of loads,
  // so the ring's waits do not change.  A half is 32 rows of 512 bytes; the 16-byte
  // chunk c (columns 8 c .. 8 c + 7) of row r sits at 16 (c ^ pswz(r)).
  static __device__ __forceinline__ int pswz(int r) { return ((r >> 1) & 7) | ((r & 1) << 3); }
  __device__ __forceinline__ void load(int t, uint32_t dst, int j) const {
    const int k0 = t * BK;
    if (!PRIOR || k0 < kdim) {
      ld.issue(k0, kdim - k0, dst, gw, j);
      return;
    }
    const int q = t - (kdim + BK - 1) / BK;
    const int64_t row0 = int64_t(m0) + 64 * q + 32 * int(grp);
    const int lane = threadIdx.x & 63, b = GROUP * j + int(gw);
    const int r = 2 * b + (lane >> 5), c = (lane & 31) ^ pswz(r);
    const bool in = row0 + r < p.M && n0 + 8 * c < p.N;
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(static_cast<const uint16_t *>(p.C) + row0 * p.ldc + n0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (MHG_LDS void *)(size_t)(dst + ld.lds_off + b * 1024), 16,
                                             in ? uint32_t((int64_t(r) * p.ldc + 8 * c) * 2) : kOut, 0, 0, 0);
  }

  // Memory phase for slab t: read all of the wave's fragments of slab t, then (256 x 256)
  // request its loads of slab t+4 (into the slot of slab t-1, which every wave has
  // finished reading: the last reader ended its phase with every read complete).  The
  // requests come after the reads: issued among them they kept the reads apart (about
  // 20 cycles each); after them they overlap the wait for the last reads (4096^3: 1250
  // -> 1280 TFLOP/s).  PAST: slab t + 4 lies past K (the last four slabs of the
  // 256 x 256 loop).  When the groups take alternate slabs (128 x 128, 64 x 64) the
  // memory phase is the longer one of the pair (its reads and eight requests against
  // 16 or 8 matrix instructions), so the requests go into the compute phase instead,
  // between the matrix instructions (compute).
  template <int S>
  __device__ __forceinline__ void mem_steps(uint32_t sa, uint32_t slot) {
    if constexpr (S < STEPS) { reads_from<S, 0>(sa, slot); mem_steps<S + 1>(sa, slot); }
  }
  // PA memory phase for slab t: reads from A's pair slot (t / 2) % 3 (the slab's half of
  // each row) and B's slot t % 4, then group 0 requests half t % 2 of A's pair
  // (t + 4) / 2 (rows 128 (t % 2) ..) and group 1 B of slab t + 4 into slab t's B slot.
  // B's rows 64 w .. 64 w + 63 of a slab are read by wave w of each group only: by
  // group 0 one phase earlier (complete before the barrier between), by group 1 now.
  // So each wave of group 1 refills exactly those rows (OWN loads), once its own reads
  // are complete; a wave that refilled other rows would overwrite fragments that the
  // other waves of its group may still be reading in this phase.
  __device__ __forceinline__ void mem_pa(int t) {
    fa_cur = fa_off[0] ^ uint32_t(64 * (t & 1));
    mem_steps<0>(lds0 + uint32_t((t >> 1) % 3) * 32768u, lds0 + PA_B + uint32_t(t & 3) * 16384u - OP_BYTES);
    if (grp == 0) {
      const int pr = (t + 4) >> 1, k0 = pr * 2 * BK;
      const uint32_t dst = lds0 + uint32_t(pr % 3) * 32768u;
#pragma unroll
      for (int j = 0; j < LOADS; ++j) { lp.issue(k0, kdim - k0, dst, gw, j, t & 1); MHG_ORDER(); }
    } else {
      wait_lgkm<0>();       // the wave's own reads of its rows of slab t are complete
      MHG_ORDER();
      const int k0 = (t + 4) * BK;
      const uint32_t dst = lds0 + PA_B + uint32_t(t & 3) * 16384u - OP_BYTES;
#pragma unroll
      for (int j = 0; j < LOADS; ++j) { ld.issue<true>(k0, kdim - k0, dst, gw, j); MHG_ORDER(); }
    }
    wait_lgkm<0>();
    MHG_ORDER();
  }
  // One of the last four iterations of the 256 x 256 loop without the prior C: the
  // memory phase requests nothing, and each wave waits until at most W of its loads are
  // in flight (those of the slabs after slab t + 1).
  template <int W>
  __device__ __forceinline__ void last_iter(int t) {
    fa_cur = fa_off[0];
    mem_steps<0>(slot_addr(t), slot_addr(t));
    wait_lgkm<0>();
    MHG_ORDER();
    wait_vm<W>();
    barrier();
    MHG_ORDER();
    compute();
    wait_vm<W>();
    barrier();
    MHG_ORDER();
  }
  template <bool PAST = false>
  __device__ __forceinline__ void mem(int t) {
    fa_cur = fa_off[0];
    mem_steps<0>(slot_addr(t), slot_addr(t));
    if constexpr (!ALT) {             // ALT: requested by compute(t)
      const int k0 = (t + AHEAD) * BK;
      const uint32_t dst = slot_addr(t + AHEAD);
#pragma unroll
      for (int j = 0; j < LOADS; ++j) {
        if constexpr (PAST) load(t + AHEAD, dst, j);
        else ld.issue(k0, kdim - k0, dst, gw, j);
        MHG_ORDER();
      }
    }
    wait_lgkm<0>();
    MHG_ORDER();
  }
  // Compute phase: the wave's STEPS MB NBL matrix instructions of a slab, back to back.
  // Groups on alternate slabs (ALT) request both operands of their slab t + 4 here, one
  // request after every few matrix instructions: slab t + 4's slot held slab t - 1,
  // which the other group finished reading two phases ago, and the compute phase has
  // room for the requests that the memory phase has not (2048^3 NT 26.1 -> 25.6 us,
  // 1024^3 9.3-9.7 -> 8.8-8.9 us, 1000^3 10.1-10.3 -> 9.7 us on one box).
  template <bool ISSUE = true>
  __device__ __forceinline__ void compute(int t = 0) {
    constexpr int NMF = STEPS * MB * NBL, EVERY = NMF / (2 * LOADS);
    static_assert(!ALT || (EVERY >= 1 && NMF % (2 * LOADS) == 0), "requests spread over the matrix instructions");
    const int k0 = (t + AHEAD) * BK;
    const uint32_t dst = slot_addr(t + AHEAD);
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
      for (int m = 0; m < MB * NBL; ++m) {
        if constexpr (ALT && ISSUE) {
          const int n = s * MB * NBL + m;
          if (n % EVERY == EVERY - 1) {
            const int q = n / EVERY;
            if (q < LOADS) ld.issue(k0, kdim - k0, dst, gw, q);
            else ld2.issue(k0, kdim - k0, dst, gw, q - LOADS);
            MHG_ORDER();
          }
        }
        const int i = m / NBL, j = m % NBL;
        const u32x4 a = {fa[s][i][0].x, fa[s][i][0].y, fa[s][i][1].x, fa[s][i][1].y};
        const u32x4 b = {fb[s][j][0].x, fb[s][j][0].y, fb[s][j][1].x, fb[s][j][1].y};
        acc[i][j] = mfma16(H{}, b, a, acc[i][j]);
        MHG_ORDER();
      }
  }

  __device__ __forceinline__ uint32_t slot_addr(int t) const { return lds0 + uint32_t(t % SLOTS) * SLOT_BYTES; }

  __device__ __forceinline__ void run(uint32_t lds_base, int bid) {
    int tm, tn;
    tile_of(bid, p.gm, p.gn, p.group_m, tm, tn);
    m0 = tm * BM;
    n0 = tn * BN;
    lds0 = lds_base;
    const int lane = threadIdx.x & 63;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    grp = wave >> 2;
    gw = wave & 3;
    const uint16_t *A = static_cast<const uint16_t *>(p.A), *B = static_cast<const uint16_t *>(p.B);
    if (!ALT) {              // groups split the rows (128 x 64 blocks) and the operands
      wm = int(grp);
      wn = int(gw);
      if constexpr (PA) {    // group 0: rows 0..127 (ld) and 128..255 (ld2) of A's pairs
        if (grp == 0) {
          lp.init(A, p.lda, m0, p.M, int(gw), lane);
        } else {
          ld.init<B_KC, BN, BK, true>(B, p.ldb, n0, p.N, gw, lane, OP_BYTES);
        }
      } else if (grp == 0) {
        ld.init<A_KC, BM, BK>(A, p.lda, m0, p.M, gw, lane, 0);
      } else {
        ld.init<B_KC, BN, BK>(B, p.ldb, n0, p.N, gw, lane, OP_BYTES);
      }
    } else {                 // groups take alternate slabs; WTM x WTN blocks, 2 x 2 of them
      wm = int(gw >> 1);
      wn = int(gw & 1);
      ld.init<A_KC, BM, BK>(A, p.lda, m0, p.M, gw, lane, 0);
      ld2.init<B_KC, BN, BK>(B, p.ldb, n0, p.N, gw, lane, OP_BYTES);
    }
    if (A_KC) {
      fa_off[0] = kc_lane<BKA>(lane) + 2 * BKA * WTM * wm;
    } else {
#pragma unroll
      for (int i = 0; i < MB; ++i) fa_off[i] = mn_lane<BM>(lane, MB * wm + i);
    }
    if (B_KC) {
      fb_off[0] = kc_lane<BK>(lane) + 2 * BK * WTN * wn;
    } else {
#pragma unroll
      for (int j = 0; j < NBL; ++j) fb_off[j] = mn_lane<BN>(lane, NBL * wn + j);
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NBL; ++j) acc[i][j] = f32x4{};
    kdim = int(p.K);
    const int KT = (kdim + BK - 1) / BK;

    // Every wave runs the same loop, mem(t); barrier; compute(); barrier, but group 1
    // passes one extra barrier before it and group 0 one after it, so group 1 runs one
    // phase behind and the two groups of a SIMD alternate between reading and
    // multiplying.
    wait_lgkm<0>();                     // nothing else counts against lgkmcnt below
    if constexpr (PA) {
      // Prologue: group 0 requests A's pairs 0 and 1 (slabs 0..3), group 1 B of slabs
      // 0..3.  Group 0 needs pair t / 2 whole before slab t is read: its second half was
      // requested two memory phases earlier, so after multiplying at most 8 loads may
      // be in flight.  Group 1 needs B of slab t after its memory phase of slab t - 1:
      // requested four memory phases earlier, at most 12 in flight.
      if (grp == 0) {
#pragma unroll
        for (int pr = 0; pr < 2; ++pr)
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < LOADS; ++j)
              lp.issue(pr * 2 * BK, kdim - pr * 2 * BK, lds0 + uint32_t(pr) * 32768u, gw, j, h);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int j = 0; j < LOADS; ++j)
            ld.issue<true>(u * BK, kdim - u * BK, lds0 + PA_B + uint32_t(u) * 16384u - OP_BYTES, gw, j);
      }
      if (grp == 1) wait_vm<3 * LOADS>(); else wait_vm<2 * LOADS>();
      barrier();
      if (grp == 1) barrier();
      MHG_ORDER();
      for (int t = 0; t < KT; ++t) {
        mem_pa(t);
        wait_vm<3 * LOADS>();
        barrier();
        MHG_ORDER();
        compute();
        if (grp == 0) wait_vm<2 * LOADS>(); else wait_vm<3 * LOADS>();
        barrier();
        MHG_ORDER();
      }
    } else if (!ALT) {
      // Both groups read every slab: in phase 2t group 0 reads slab t while group 1
      // multiplies slab t-1, in phase 2t+1 group 0 multiplies slab t while group 1 reads
      // it.  Group 0 requests A of slab t+4 in phase 2t, group 1 B of slab t+4 in phase
      // 2t+1; slab t+1 must be in LDS when phase 2t+2 starts, so before every barrier
      // each wave waits until at most its three younger slabs' loads (12) are in flight.
      // Prologue: slabs 0 and 1, then (once slab 0 has landed and the groups are one
      // phase apart) slabs 2 and 3, first read four and six phases on.  Requests are
      // throttled at issue when every wave of every compute unit makes them at once, so
      // issuing all four first delayed the wait for slab 0 by the issue time of the
      // other two.
      issue_all(0);
      issue_all(1);
      wait_vm<LOADS>();                 // slab 0 landed
      barrier();
      if (grp == 1) barrier();
      MHG_ORDER();
      issue_all(2);
      issue_all(3);
      MHG_ORDER();
      // The last four iterations would request the slabs past K.  With the prior C they
      // load it; otherwise they request nothing, and each waits for exactly the slabs
      // still in flight that the next phase needs (a wave's loads complete in the order
      // issued).  Fewer than four slabs keep the uniform form, the prologue having
      // requested zeros past K.
      int t = 0;
      for (; t < KT - AHEAD; ++t) {
        mem(t);
        wait_vm<3 * LOADS>();
        barrier();
        MHG_ORDER();
        compute();
        wait_vm<3 * LOADS>();
        barrier();
        MHG_ORDER();
      }
      if (!PRIOR && KT >= AHEAD) {
        static_assert(AHEAD == 4, "tail of four iterations");
        last_iter<2 * LOADS>(t);
        last_iter<LOADS>(t + 1);
        last_iter<0>(t + 2);
        last_iter<0>(t + 3);
        t = KT;
      }
      for (; t < KT; ++t) {
        mem<true>(t);
        wait_vm<3 * LOADS>();
        barrier();
        MHG_ORDER();
        compute();
        wait_vm<3 * LOADS>();
        barrier();
        MHG_ORDER();
      }
    } else {
      // Group g reads, requests and multiplies the slabs t = g mod 2: slab t is read in
      // phase t and multiplied in phase t + 1, and slab t + 4 (the group's own) is
      // requested while slab t is multiplied.  Slab t + 2 must be in LDS when phase t + 2
      // starts, so after multiplying a wave waits until only its slab t + 4 (8 loads) is
      // in flight; slabs past K load zeros, so both groups run the same trip count.
      // (Issuing the group's second slab only after its first had landed, as the
      // 256 x 256 prologue does with slabs 2 and 3, was slower here: that slab is read
      // two phases on and then arrived late; 1024^3 8.4-8.7 -> 8.7 us.)
      issue_all(int(grp));
      issue_all(int(grp) + 2);
      wait_vm<2 * LOADS>();             // the group's first slab landed
      barrier();
      if (grp == 1) barrier();
      MHG_ORDER();
      // The slabs the group's last two iterations would request are never multiplied:
      // those iterations request nothing and wait for every load still in flight.
      const int U = (KT + 1) / 2;
      int u = 0;
      for (; u < U - 2; ++u) {
        mem(2 * u + int(grp));
        wait_vm<4 * LOADS>();
        barrier();
        MHG_ORDER();
        compute(2 * u + int(grp));
        wait_vm<2 * LOADS>();
        barrier();
        MHG_ORDER();
      }
      for (; u < U; ++u) {
        mem(2 * u + int(grp));
        wait_vm<4 * LOADS>();
        barrier();
        MHG_ORDER();
        compute<false>(2 * u + int(grp));
        wait_vm<0>();
        barrier();
        MHG_ORDER();
      }
    }
    if (grp == 0) barrier();
    // Loads past K (zeros, or the prior C) may still be writing LDS: drain them, then let
    // every wave finish with the ring before the epilogue reuses its memory.
    wait_vm<0>();
    barrier();
    MHG_ORDER();

    if constexpr (TL::KSPLIT == 2) {
      // The two waves that hold partial sums of one block of C (wave gw of each group)
      // finish half of its rows each: group 0 the 16-row blocks i < MB/2, group 1 the
      // others.  Each hands the half its partner finishes through LDS, lane-major so that
      // neither side has bank conflicts, and adds the half it receives (the sum of the
      // two partials is the same either way round).  All eight waves then run the
      // epilogue on half a block each, staging in 8 KiB past the hand-off areas.
      constexpr int H2 = MB / 2;
      const uint32_t handoff = lds0 + gw * (MB * NBL * 64 * 16);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBL; ++j)
          if ((i < H2) == (grp == 1))
            *reinterpret_cast<MHG_LDS f32x4 *>(size_t(handoff + ((i * NBL + j) * 64 + lane) * 16)) = acc[i][j];
      barrier();
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NBL; ++j)
          if ((i < H2) == (grp == 0))
            acc[i][j] += *reinterpret_cast<const MHG_LDS f32x4 *>(size_t(handoff + ((i * NBL + j) * 64 + lane) * 16));
      static_assert(4 * MB * NBL * 1024 <= 65536 && 65536 + 8 * 8192 <= SLOTS * SLOT_BYTES, "hand-off and staging");
      if (grp == 0) epilogue<0, H2>(lane, lds0 + 65536 + wave * 8192);
      else epilogue<H2, H2>(lane, lds0 + 65536 + wave * 8192);
    } else {
      epilogue<0, MB>(lane, lds0 + wave * 16384);
    }
  }

  // acc[i][j] holds the transposed 16 x 16 block (B's fragment is the instruction's
  // first operand): element e of lane l is C[row WTM wm + 16 i + l % 16][col WTN wn +
  // 16 j + 4 (l / 16) + e] of the tile.  A lane's four consecutive columns are a piece
  // of one row (16 bytes of fp32), and a store instruction would touch 16 rows; staged
  // through the wave's 16 KiB of LDS at `region` instead, every store writes whole
  // 64-column row segments of C.
  static __device__ __forceinline__ int piece_row(int i, int lane) { return 16 * i + (lane & 15); }
  static __device__ __forceinline__ int piece_col(int j, int lane) { return 16 * j + 4 * (lane >> 4); }
  // The epilogue on the wave's 16-row blocks I0 .. I0 + NI - 1 (all of them, or half
  // when the groups split K), staged at `region` (16 NI rows of 256 bytes at most).
  template <int I0, int NI>
  __device__ __forceinline__ void epilogue(int lane, uint32_t region) {
    const int64_t rowW = m0 + wm * WTM + 16 * I0, colW = n0 + wn * WTN;
    const int ob = p.out_code == E_F32 ? 4 : 2;
    if constexpr (PRIOR) {
      static_assert(I0 == 0 && NI == MB, "the prior-C epilogue takes the whole block");
      epilogue_prior(lane);
      return;
    }
    // Staging is laid out for 64-column row segments (32 or more rows); the 32 x 32
    // blocks of the 64 x 64 tile (2 KiB of C a wave) store directly.
    constexpr bool STAGE = FN == 2 && NI % 2 == 0;
    const bool c16 = ((uintptr_t(p.C) | uintptr_t(p.ldc * ob)) & 15) == 0;
    if (STAGE && c16) {
      // A fused epilogue that reads the prior C (beta != 0), or that writes fp32, runs in
      // the fp32 staging below, on whole row segments.  One that does not read C and
      // writes a 16-bit type is applied to the accumulators here, before the 16-bit
      // staging.  Either way the lane's bias chunks (and the pass's prior values of C)
      // are requested before its first store: the compiler may not move a load above
      // a store that might alias it.
      if (p.epi && p.beta == 0.0f && p.out_code != E_F32) {
        f32x4 b[NBL];
#pragma unroll
        for (int j = 0; j < NBL; ++j) {
          const int64_t col = colW + piece_col(j, lane);
          b[j] = col < p.N ? bias4(p, col, p.N - col) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int i = I0; i < I0 + NI; ++i)
#pragma unroll
          for (int j = 0; j < NBL; ++j) acc[i][j] = epilogue4pb(p, acc[i][j], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, b[j], 4);
      }
      if (p.out_code == E_F32 && !p.epi && rowW + 16 * NI <= p.M && colW + WTN <= p.N &&
          (int64_t(16 * NI) * p.ldc + WTN) * 4 < (int64_t(1) << 31)) {
        staged32_inside<I0, NI>(lane, region, rowW, colW);
        return;
      }
      if (p.out_code == E_F32 || (p.epi && p.beta != 0.0f)) {
        // Up to 64 rows (nb blocks) of 256 bytes a pass; chunk c of row r at
        // 16 (c ^ (r % 16)), which keeps the 16-byte writes (16 rows at 4 chunks) and the
        // read-back (4 rows at 16 chunks) free of bank conflicts
#pragma unroll
        for (int pass = 0; pass < (NI + 3) / 4; ++pass) {
          const int nb = NI - 4 * pass < 4 ? NI - 4 * pass : 4;
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
            for (int j = 0; j < NBL; ++j) {
              if (i4 >= nb) break;
              const int r = piece_row(i4, lane), c = piece_col(j, lane) >> 2;
              *reinterpret_cast<MHG_LDS f32x4 *>(size_t(region + r * 256 + 16 * (c ^ (r & 15)))) = acc[I0 + 4 * pass + i4][j];
            }
          if (!p.epi) {
#pragma unroll
            for (int k = 0; k < 16; ++k) {
              if (k >= 4 * nb) break;
              const int r = 4 * k + (lane >> 4), c = lane & 15;
              const u32x4 v = *reinterpret_cast<const MHG_LDS u32x4 *>(size_t(region + r * 256 + 16 * (c ^ (r & 15))));
              store_chunk(rowW + 64 * pass + r, colW + 4 * c, v, 4, rowW, colW);
            }
            continue;
          }
          // A lane stores the same four columns in every row of the pass.
          const int64_t colB = colW + 4 * (lane & 15);
          const f32x4 bias = colB < p.N ? bias4(p, colB, p.N - colB) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          f32x4 prior[16];
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            if (k >= 4 * nb) break;
            const int64_t row = rowW + 64 * pass + 4 * k + (lane >> 4);
            prior[k] = p.beta != 0.0f && row < p.M && colB < p.N ? prior4(p, row, colB, p.N - colB)
                                                                 : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          }
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            if (k >= 4 * nb) break;
            const int r = 4 * k + (lane >> 4), c = lane & 15;
            const int64_t row = rowW + 64 * pass + r, n_in = p.N - colB;
            if (row >= p.M || n_in <= 0) continue;
            const u32x4 v = *reinterpret_cast<const MHG_LDS u32x4 *>(size_t(region + r * 256 + 16 * (c ^ (r & 15))));
            const f32x4 f = epilogue4pb(p, __builtin_bit_cast(f32x4, v), prior[k], bias, n_in);
            store_out4(p.C, row * p.ldc + colB, f, p.out_code, n_in >= 4, int(n_in));
          }
        }
      } else {
        // A lane's converted piece (four columns, 8 bytes) of block 2 i2 and the one of
        // block 2 i2 + 1 (rows t and 16 + t of the pair, same columns) go out as one
        // 16-byte write.  8-byte writes are served 16 consecutive lanes at a time within
        // 128 bytes of banks, where 16 rows at one column offset can reach only 8 places;
        // 16-byte writes are served 16 lanes at a time over all 256 bytes.  The unit of
        // lane (t, g) for (i2, j) sits at slot 16 g + (t ^ (4 j + 2 (g / 2) + g % 2)) of that
        // pair and column block's 1 KiB.  The read-back takes a 16-byte row chunk as its
        // two 8-byte pieces (8-byte reads: 32 consecutive lanes a pass), each store
        // instruction covering four rows of each half of a pair, so that a pass reads
        // both halves of its units: no bank conflicts on either side.  (Column groups
        // g and g + 1 differ in the low bit of the slot as well, so that the two reads
        // are not a constant distance apart: the compiler fused such a pair into one
        // two-address read, and the conflict counter showed that form conflicting here,
        // 8 cycles an instruction; the two separate reads show none.)
        static_assert(!STAGE || (NI % 2 == 0 && NBL == 4), "pairs of 16-row blocks, 64 columns");
        if (!p.epi && p.out_code == kHalfOut && rowW + 16 * NI <= p.M && colW + WTN <= p.N &&
            (int64_t(16 * NI) * p.ldc + WTN) * 2 < (int64_t(1) << 31)) {
          staged16_inside<I0, NI>(lane, region, rowW, colW);
          return;
        }
        const int t = lane & 15, g = lane >> 4;
        const auto half = [&](f32x4 a) {
          uint16_t h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            h[e] = p.out_code == E_F16 ? __builtin_bit_cast(uint16_t, (_Float16)a[e])
                                       : __builtin_bit_cast(uint16_t, (__bf16)a[e]);
          return u32x2{uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16)};
        };
#pragma unroll
        for (int i2 = 0; i2 < NI / 2; ++i2)
#pragma unroll
          for (int j = 0; j < NBL; ++j) {
            const u32x2 lo = half(acc[I0 + 2 * i2][j]), hi = half(acc[I0 + 2 * i2 + 1][j]);
            const uint32_t slot = uint32_t((i2 * NBL + j) * 64 + 16 * g + (t ^ (4 * j + 2 * (g >> 1) + (g & 1))));
            *reinterpret_cast<MHG_LDS u32x4 *>(size_t(region + 16 * slot)) = u32x4{lo.x, lo.y, hi.x, hi.y};
          }
#pragma unroll
        for (int k = 0; k < 2 * NI; ++k) {
          const int i2 = k >> 2, rho = lane >> 3, sh = rho & 1, tt = 4 * (k & 3) + (rho >> 1), c = lane & 7;
          const int j = c >> 1, g0 = 2 * (c & 1);
          const uint32_t u = uint32_t((i2 * NBL + j) * 64 + 16 * g0), f = uint32_t(4 * j + 2 * (c & 1));
          const uint32_t at = region + 16 * (u + (tt ^ f)) + 8 * sh, at2 = region + 16 * (u + 16 + (tt ^ (f + 1))) + 8 * sh;
          const u32x2 a = *reinterpret_cast<const MHG_LDS u32x2 *>(size_t(at));
          const u32x2 b = *reinterpret_cast<const MHG_LDS u32x2 *>(size_t(at2));
          store_chunk(rowW + 32 * i2 + 16 * sh + tt, colW + 8 * c, u32x4{a.x, a.y, b.x, b.y}, 8, rowW, colW);
        }
      }
      return;
    }
    const bool c_vec = p.c_vec != 0;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int64_t row = rowW + piece_row(i, lane);
      if (row >= p.M) continue;
      // With an epilogue, the row block's bias and prior values are requested before its
      // first store (a load may not move above a store that might alias it).
      f32x4 ep[NBL];
      if (p.epi) {
#pragma unroll
        for (int j = 0; j < NBL; ++j) {
          const int64_t col = colW + piece_col(j, lane);
          ep[j] = col < p.N ? epilogue4(p, acc[I0 + i][j], row, col, p.N - col) : acc[I0 + i][j];
        }
      }
#pragma unroll
      for (int j = 0; j < NBL; ++j) {
        const int64_t col = colW + piece_col(j, lane);
        const int64_t n_in = p.N - col;
        if (n_in <= 0) continue;
        store_out4(p.C, row * p.ldc + col, p.epi ? ep[j] : acc[I0 + i][j], p.out_code, c_vec && n_in >= 4, int(n_in));
      }
    }
  }

  // The 16-bit staged epilogue above for a wave block wholly inside C, with no fused
  // epilogue: the same LDS layout and store pattern, with the arithmetic taken out of the
  // per-write and per-store work (the epilogue runs on all waves of all compute units at
  // once, two waves a SIMD, so every vector instruction counts: the general form took
  // ~6 us a workgroup at 4096^3, most of it instruction issue).  The conversion is the
  // output type's alone (16-bit output has the input's type); the four per-lane LDS
  // write offsets and the read-back offsets are computed once, the rest being immediate
  // offsets; the stores go through one buffer resource at the block's corner with a
  // fixed per-lane offset, the row step (uniform) in the scalar offset.
  static constexpr int kHalfOut = std::is_same<H, HalfBF16>::value ? E_BF16 : E_F16;
  static __device__ __forceinline__ u32x2 pack_half(f32x4 a) {
    uint16_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      h[e] = std::is_same<H, HalfBF16>::value ? __builtin_bit_cast(uint16_t, (__bf16)a[e])
                                              : __builtin_bit_cast(uint16_t, (_Float16)a[e]);
    return u32x2{uint32_t(h[0]) | (uint32_t(h[1]) << 16), uint32_t(h[2]) | (uint32_t(h[3]) << 16)};
  }
  template <int I0, int NI>
  __device__ __forceinline__ void staged16_inside(int lane, uint32_t region, int64_t rowW, int64_t colW) {
    const int t = lane & 15, g = lane >> 4;
    uint32_t woff[NBL];
#pragma unroll
    for (int j = 0; j < NBL; ++j) woff[j] = region + 16 * uint32_t(64 * j + 16 * g + (t ^ (4 * j + 2 * (g >> 1) + (g & 1))));
#pragma unroll
    for (int i2 = 0; i2 < NI / 2; ++i2)
#pragma unroll
      for (int j = 0; j < NBL; ++j) {
        const u32x2 lo = pack_half(acc[I0 + 2 * i2][j]), hi = pack_half(acc[I0 + 2 * i2 + 1][j]);
        *reinterpret_cast<MHG_LDS u32x4 *>(size_t(woff[j] + uint32_t(16 * 64 * NBL * i2))) = u32x4{lo.x, lo.y, hi.x, hi.y};
      }
    // Store k: rows 32 (k / 4) + 16 sh + 4 (k % 4) + r2 of the block, columns 8 c ..;
    // its two pieces at slot (k / 4) NBL 64 + 64 j + 16 (2 cb) + (tt ^ f) and 16 slots
    // on with f + 1, tt = 4 (k % 4) + r2, f = 4 j + 2 cb, where tt ^ f = 4 ((k % 4) ^ j)
    // + (r2 ^ 2 cb).
    const int rho = lane >> 3, sh = rho & 1, r2 = rho >> 1, c = lane & 7, j = c >> 1, cb = c & 1;
    const uint32_t rb = region + 16 * uint32_t(64 * j + 32 * cb + (r2 ^ (2 * cb))) + 8 * sh;
    const uint32_t rb2 = region + 16 * uint32_t(64 * j + 32 * cb + 16 + (r2 ^ (2 * cb + 1))) + 8 * sh;
    uint32_t qo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) qo[q] = 64 * uint32_t(q ^ j);
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(static_cast<const char *>(p.C) + (rowW * p.ldc + colW) * 2);
    const uint32_t voff = uint32_t(((16 * sh + r2) * p.ldc + 8 * c) * 2);
#pragma unroll
    for (int k = 0; k < 2 * NI; ++k) {
      const uint32_t kb = uint32_t(16 * 64 * NBL * (k >> 2));
      const u32x2 a = *reinterpret_cast<const MHG_LDS u32x2 *>(size_t(rb + qo[k & 3] + kb));
      const u32x2 b = *reinterpret_cast<const MHG_LDS u32x2 *>(size_t(rb2 + qo[k & 3] + kb));
      const int soff = int((32 * (k >> 2) + 4 * (k & 3)) * p.ldc * 2);
      __builtin_amdgcn_raw_buffer_store_b128(u32x4{a.x, a.y, b.x, b.y}, rs, voff, soff, kStoreDeviceScope);
    }
  }

  // The fp32 staged epilogue above, lean in the same way, for a wave block wholly inside
  // C with no fused epilogue.  With t = lane % 16 and g = lane / 16, the write of block
  // (i4, j) goes to row 16 i4 + t, chunk (4 j + g) ^ t = ((g ^ t) % 4) + 4 (j ^ (t / 4));
  // read-back k takes row 4 k + g, chunk u ^ (4 (k % 4) + g) = ((u ^ g) % 4) + 4 (((u ^ g)
  // / 4) ^ (k % 4)), u = lane % 16: four per-lane offsets each, the rest immediate.
  template <int I0, int NI>
  __device__ __forceinline__ void staged32_inside(int lane, uint32_t region, int64_t rowW, int64_t colW) {
    const int t = lane & 15, g = lane >> 4, u = lane & 15, ug = u ^ g;
    uint32_t woff[NBL], roff[4];
#pragma unroll
    for (int j = 0; j < NBL; ++j) woff[j] = region + uint32_t(t * 256 + 16 * ((g ^ t) & 3) + 64 * (j ^ (t >> 2)));
#pragma unroll
    for (int q = 0; q < 4; ++q) roff[q] = region + uint32_t(g * 256 + 16 * (ug & 3) + 64 * ((ug >> 2) ^ q));
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(static_cast<const char *>(p.C) + (rowW * p.ldc + colW) * 4);
    const uint32_t voff = uint32_t((g * p.ldc + 4 * u) * 4);
#pragma unroll
    for (int pass = 0; pass < (NI + 3) / 4; ++pass) {
      const int nb = NI - 4 * pass < 4 ? NI - 4 * pass : 4;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
        for (int j = 0; j < NBL; ++j) {
          if (i4 >= nb) break;
          *reinterpret_cast<MHG_LDS f32x4 *>(size_t(woff[j] + uint32_t(4096 * i4))) = acc[I0 + 4 * pass + i4][j];
        }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (k >= 4 * nb) break;
        const u32x4 v = *reinterpret_cast<const MHG_LDS u32x4 *>(size_t(roff[k & 3] + uint32_t(1024 * k)));
        const int soff = int((64 * pass + 4 * k) * p.ldc * 4);
        __builtin_amdgcn_raw_buffer_store_b128(v, rs, voff, soff, kStoreDeviceScope);
      }
    }
  }

  // The epilogue with the prior C (16-bit) already in LDS, quarter q of the tile in the
  // slot of slab KT + q.  Each lane combines its accumulators with the prior values at
  // the same places and writes the rounded results over them (one lane per place); the
  // wave then stores its 128 x 64 block from there in 128-byte row pieces.  Rows and
  // columns outside C were loaded as zeros and are not stored.
  __device__ __forceinline__ uint32_t prior_at(int R, int c) const {
    const int KT = (kdim + BK - 1) / BK, r = R & 31;
    return slot_addr(KT + R / 64) + uint32_t((R >> 5) & 1) * OP_BYTES + uint32_t(r * 512 + 16 * (c ^ pswz(r)));
  }
  __device__ __forceinline__ void epilogue_prior(int lane) {
    const int64_t rowW = m0 + wm * WTM, colW = n0 + wn * WTN;
    if (p.out_code == kHalfOut && rowW + WTM <= p.M && colW + WTN <= p.N &&
        (int64_t(WTM) * p.ldc + WTN) * 2 < (int64_t(1) << 31)) {
      if (p.act == 1) prior_inside<true>(lane, rowW, colW);
      else prior_inside<false>(lane, rowW, colW);
      return;
    }
    f32x4 b[NBL];
#pragma unroll
    for (int j = 0; j < NBL; ++j) {
      const int64_t col = colW + piece_col(j, lane);
      b[j] = col < p.N ? bias4(p, col, p.N - col) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NBL; ++j) {
        const int R = wm * WTM + piece_row(i, lane), Cc = wn * WTN + piece_col(j, lane);
        MHG_LDS u32x2 *at = reinterpret_cast<MHG_LDS u32x2 *>(size_t(prior_at(R, Cc >> 3) + 8 * ((Cc >> 2) & 1)));
        const u32x2 h = *at;
        f32x4 c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint16_t u = uint16_t(h[e >> 1] >> (16 * (e & 1)));
          c[e] = p.out_code == E_F16 ? float(__builtin_bit_cast(_Float16, u)) : float(__builtin_bit_cast(__bf16, u));
        }
        const f32x4 f = epilogue4pb(p, acc[i][j], c, b[j], 4);
        uint16_t o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          o[e] = p.out_code == E_F16 ? __builtin_bit_cast(uint16_t, (_Float16)f[e]) : __builtin_bit_cast(uint16_t, (__bf16)f[e]);
        *at = u32x2{uint32_t(o[0]) | (uint32_t(o[1]) << 16), uint32_t(o[2]) | (uint32_t(o[3]) << 16)};
        MHG_ORDER();     // one piece at a time: hoisting every read would spill
      }
#pragma unroll
    for (int k = 0; k < WTM / 8; ++k) {
      const int rr = 8 * k + (lane >> 3), cc = lane & 7;
      const u32x4 v = *reinterpret_cast<const MHG_LDS u32x4 *>(size_t(prior_at(wm * WTM + rr, wn * (WTN / 8) + cc)));
      store_chunk(rowW + rr, colW + 8 * cc, v, 8, rowW, colW);
    }
  }

  // The prior-C epilogue for a wave block wholly inside C, lean like the staged ones:
  // the prior C has the output's (and input's) 16-bit type, beta is not zero (this
  // kernel runs only then), the activation is a template parameter, and the per-element
  // arithmetic is epilogue4pb's, in the same order.  With t = lane % 16, g = lane / 16,
  // the piece (i, j) sits at prior_at(128 wm + 16 i + t, 8 wn + 2 j + g / 2) + 8 (g % 2):
  // slot KT + 2 wm + i / 4, half (i / 2) % 2, row 16 (i % 2) + t, chunk c ^ pswz(t); store
  // k reads row 8 k + r3 (r3 = lane / 8), chunk (8 wn + lane % 8) ^ (4 (k % 2) + r3 / 2 +
  // 8 (r3 % 2)) of slot KT + 2 wm + k / 8, half (k / 4) % 2.
  static __device__ __forceinline__ f32x4 unpack_half(u32x2 h) {
    f32x4 c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint16_t u = uint16_t(h[e >> 1] >> (16 * (e & 1)));
      c[e] = std::is_same<H, HalfBF16>::value ? float(__builtin_bit_cast(__bf16, u)) : float(__builtin_bit_cast(_Float16, u));
    }
    return c;
  }
  template <bool RELU>
  __device__ __forceinline__ void prior_inside(int lane, int64_t rowW, int64_t colW) {
    const int KT = (kdim + BK - 1) / BK;
    const int t = lane & 15, g = lane >> 4;
    f32x4 b[NBL];
#pragma unroll
    for (int j = 0; j < NBL; ++j) b[j] = bias4(p, colW + piece_col(j, lane), 4);
    const float alpha = p.alpha, beta = p.beta;
    const uint32_t sA = slot_addr(KT + 2 * wm), sB = slot_addr(KT + 2 * wm + 1);
    uint32_t lo[NBL];
#pragma unroll
    for (int j = 0; j < NBL; ++j) lo[j] = uint32_t(t * 512 + 16 * ((8 * wn + 2 * j + (g >> 1)) ^ pswz(t)) + 8 * (g & 1));
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NBL; ++j) {
        const uint32_t base = (i < 4 ? sA : sB) + uint32_t(((i >> 1) & 1) * OP_BYTES + (i & 1) * 16 * 512);
        MHG_LDS u32x2 *at = reinterpret_cast<MHG_LDS u32x2 *>(size_t(base + lo[j]));
        const f32x4 c = unpack_half(*at);
        f32x4 f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float x = alpha * acc[i][j][e];
          x += beta * c[e];
          x += b[j][e];
          if (RELU) x = x > 0.0f ? x : 0.0f;
          f[e] = x;
        }
        *at = pack_half(f);
        MHG_ORDER();     // one piece at a time: hoisting every read would spill
      }
    const int r3 = lane >> 3, cc = lane & 7;
    uint32_t so[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) so[q] = uint32_t(r3 * 512 + 16 * ((8 * wn + cc) ^ (4 * q + (r3 >> 1) + 8 * (r3 & 1))));
    const __amdgpu_buffer_rsrc_t rs = rsrc_of(static_cast<const char *>(p.C) + (rowW * p.ldc + colW) * 2);
    const uint32_t voff = uint32_t((r3 * p.ldc + 8 * cc) * 2);
#pragma unroll
    for (int k = 0; k < WTM / 8; ++k) {
      const uint32_t at = (k < 8 ? sA : sB) + uint32_t(((k >> 2) & 1) * OP_BYTES + 8 * (k & 3) * 512) + so[k & 1];
      const u32x4 v = *reinterpret_cast<const MHG_LDS u32x4 *>(size_t(at));
      __builtin_amdgcn_raw_buffer_store_b128(v, rs, voff, int(8 * k * p.ldc * 2), kStoreDeviceScope);
    }
  }

  // 16 bytes of converted output (W elements) for C[row][col .. col + W - 1], a piece
  // of the wave's block of C whose corner is (row0, col0): one store when all W lie
  // inside the matrix, else the elements that do.  C is written once and not read
  // again here, so the whole-chunk stores take the device-scope policy (sc1): they
  // write through to the level the XCDs share, and no line of C is left dirty in an
  // XCD's L2 for the write-back when the kernel ends.  Measured on the MI355X: 4096^3
  // 0.3-0.8% and 2048^3 NT 2-4% faster than streaming (nt) stores, which were in turn
  // 1.4% and 3.5% faster than ordinary ones.  The policy needs a buffer store, through
  // a resource based at the block's corner (its offsets stay below 2^31 bytes unless
  // C's rows are longer than 16 MiB; such a C takes streaming global stores).
  __device__ __forceinline__ void store_chunk(int64_t row, int64_t col, u32x4 v, int W, int64_t row0,
                                              int64_t col0) const {
    if (row >= p.M || col >= p.N) return;
    const int64_t idx = row * p.ldc + col;
    if (col + W <= p.N) {
      const int eb = W == 4 ? 4 : 2;
      if ((int64_t(WTM) * p.ldc + WTN) * eb < (int64_t(1) << 31)) {
        const char *corner = static_cast<const char *>(p.C) + (row0 * p.ldc + col0) * eb;
        const uint32_t off = uint32_t(((row - row0) * p.ldc + (col - col0)) * eb);
        __builtin_amdgcn_raw_buffer_store_b128(v, rsrc_of(corner), off, 0, kStoreDeviceScope);
      } else if (W == 4) {
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(static_cast<float *>(p.C) + idx));
      } else {
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(p.C) + idx));
      }
      return;
    }
    const int n_in = int(p.N - col);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (e >= W || e >= n_in) break;
      if (W == 4) static_cast<uint32_t *>(p.C)[idx + e] = v[e];
      else static_cast<uint16_t *>(p.C)[idx + e] = uint16_t(v[e >> 1] >> (16 * (e & 1)));
    }
  }
};

template <class H, bool A_KC, bool B_KC, class TL, bool SPLIT, bool PRIOR>
__global__ void __launch_bounds__(NT)
w8_gemm(LaunchArgs p) {
  __shared__ __attribute__((aligned(1024))) char smem[SLOTS * SLOT_BYTES];
  // Every argument the prologue needs, in scalar registers before anything else: the
  // compiler then requests them together and waits once, where it had fetched them in
  // three dependent rounds (tile mapping, then operand addresses) at ~0.2 us each on a
  // cold start (1024^3 8.4-8.6 -> 8.2-8.3 us).
  asm volatile("" ::"s"(p.gm), "s"(p.gn), "s"(p.group_m), "s"(p.A), "s"(p.B), "s"(p.M), "s"(p.N), "s"(p.K),
               "s"(p.lda), "s"(p.ldb));
  const int tiles = p.gm * p.gn;
  int bid = int(blockIdx.x);
  if constexpr (SPLIT) {
    // Split K: workgroup id = z * tiles + tile.  Chunk z of K is the product of A's
    // columns (B's rows) z * k_chunk .. + k_chunk - 1, computed as a GEMM of its own
    // into the fp32 partial z of the workspace (M x N, row-major, no epilogue); the
    // reduction kernel adds the partials in chunk order.
    const int z = bid / tiles;
    bid -= z * tiles;
    const int64_t kb = int64_t(z) * p.k_chunk;
    p.A = static_cast<const uint16_t *>(p.A) + (A_KC ? kb : kb * p.lda);
    p.B = static_cast<const uint16_t *>(p.B) + (B_KC ? kb : kb * p.ldb);
    p.K = p.K - kb < p.k_chunk ? p.K - kb : p.k_chunk;
    p.C = static_cast<float *>(p.workspace) + int64_t(z) * p.M * p.N;
    p.ldc = p.N;
    p.out_code = E_F32;
    p.c_vec = p.N % 4 == 0;
    p.epi = 0;
  }
  W8Gemm<H, A_KC, B_KC, TL, PRIOR> g(p);
  g.run(uint32_t(size_t((MHG_LDS char *)smem)), bid);
}

// C = epilogue(sum of the split_k fp32 partials in chunk order): one thread per four
// consecutive elements of a row of C.  The same partials give the same bits whatever
// order the chunks' workgroups ran in.
__global__ void __launch_bounds__(256) splitk_reduce(LaunchArgs p) {
  const int64_t cpr = (p.N + 3) / 4;   // four-element chunks a row
  const int64_t q = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (q >= p.M * cpr) return;
  const int64_t row = q / cpr, col = 4 * (q % cpr), n_in = p.N - col;
  const float *ws = static_cast<const float *>(p.workspace);
  const int64_t slice = p.M * p.N, idx = row * p.N + col;
  const bool vec = p.N % 4 == 0;
  f32x4 t = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int z = 0; z < p.split_k; ++z) {
    f32x4 v = {0.0f, 0.0f, 0.0f, 0.0f};
    if (vec) {
      v = *reinterpret_cast<const f32x4 *>(ws + z * slice + idx);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < n_in) v[e] = ws[z * slice + idx + e];
    }
    t = z == 0 ? v : t + v;
  }
  if (p.epi) t = epilogue4(p, t, row, col, n_in);
  store_out4(p.C, row * p.ldc + col, t, p.out_code, p.c_vec && n_in >= 4, int(n_in));
}

#define MHG_W8_INST(H, TL, SPLIT, PRIOR)                                            \
  template __global__ void w8_gemm<H, true, false, TL, SPLIT, PRIOR>(LaunchArgs);  \
  template __global__ void w8_gemm<H, true, true, TL, SPLIT, PRIOR>(LaunchArgs);   \
  template __global__ void w8_gemm<H, false, false, TL, SPLIT, PRIOR>(LaunchArgs); \
  template __global__ void w8_gemm<H, false, true, TL, SPLIT, PRIOR>(LaunchArgs);
MHG_W8_INST(HalfBF16, Tile256, false, false)
MHG_W8_INST(HalfF16, Tile256, false, false)
MHG_W8_INST(HalfBF16, Tile128, false, false)
MHG_W8_INST(HalfF16, Tile128, false, false)
MHG_W8_INST(HalfBF16, Tile64, false, false)
MHG_W8_INST(HalfF16, Tile64, false, false)
// Split-K only where the catalogue has it (the 64 x 64 and 128 x 128 tiles).
MHG_W8_INST(HalfBF16, Tile128, true, false)
MHG_W8_INST(HalfF16, Tile128, true, false)
MHG_W8_INST(HalfBF16, Tile64, true, false)
MHG_W8_INST(HalfF16, Tile64, true, false)
// The 256 x 256 tile with the prior C through LDS.
MHG_W8_INST(HalfBF16, Tile256, false, true)
MHG_W8_INST(HalfF16, Tile256, false, true)
#undef MHG_W8_INST

template <class H, class TL>
hipError_t launch_typed(const LaunchArgs &p, hipStream_t s) {
  const int split = p.split_k > 1 ? p.split_k : 1;
  if (split > 1 && (!p.workspace || p.k_chunk < TL::BK || p.k_chunk % TL::BK ||
                    p.ws_bytes < int64_t(split) * p.M * p.N * 4))
    return hipErrorInvalidValue;
  const dim3 grid(unsigned(p.gm) * unsigned(p.gn) * unsigned(split)), block(NT);
  if (split == 1) {
    // The 256 x 256 tile brings a 16-bit prior C into LDS with its last slab loads when
    // C's rows are whole 16-byte chunks (aligned base, ldc and N multiples of 8) and a
    // half-quarter (32 rows) spans less than 2^31 bytes.
    if constexpr (TL::BM == 256) {
      const bool prior = p.epi && p.beta != 0.0f && p.out_code != E_F32 && p.N % 8 == 0 && p.ldc % 8 == 0 &&
                         p.ldc < (int64_t(1) << 24) && (reinterpret_cast<uintptr_t>(p.C) & 15) == 0;
      if (prior) {
        if (!p.a_col && !p.b_col) hipLaunchKernelGGL((w8_gemm<H, true, false, TL, false, true>), grid, block, 0, s, p);
        else if (!p.a_col && p.b_col) hipLaunchKernelGGL((w8_gemm<H, true, true, TL, false, true>), grid, block, 0, s, p);
        else if (p.a_col && !p.b_col) hipLaunchKernelGGL((w8_gemm<H, false, false, TL, false, true>), grid, block, 0, s, p);
        else hipLaunchKernelGGL((w8_gemm<H, false, true, TL, false, true>), grid, block, 0, s, p);
        return hipGetLastError();
      }
    }
    if (!p.a_col && !p.b_col) hipLaunchKernelGGL((w8_gemm<H, true, false, TL, false, false>), grid, block, 0, s, p);
    else if (!p.a_col && p.b_col) hipLaunchKernelGGL((w8_gemm<H, true, true, TL, false, false>), grid, block, 0, s, p);
    else if (p.a_col && !p.b_col) hipLaunchKernelGGL((w8_gemm<H, false, false, TL, false, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((w8_gemm<H, false, true, TL, false, false>), grid, block, 0, s, p);
    return hipGetLastError();
  }
  if constexpr (TL::BM == 256) {
    return hipErrorInvalidValue;   // no split-K instantiation of the 256 x 256 tile
  } else {
    if (!p.a_col && !p.b_col) hipLaunchKernelGGL((w8_gemm<H, true, false, TL, true, false>), grid, block, 0, s, p);
    else if (!p.a_col && p.b_col) hipLaunchKernelGGL((w8_gemm<H, true, true, TL, true, false>), grid, block, 0, s, p);
    else if (p.a_col && !p.b_col) hipLaunchKernelGGL((w8_gemm<H, false, false, TL, true, false>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((w8_gemm<H, false, true, TL, true, false>), grid, block, 0, s, p);
  }
  {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t chunks = p.M * ((p.N + 3) / 4);
    hipLaunchKernelGGL(splitk_reduce, dim3(unsigned((chunks + 255) / 256)), dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <class TL>
hipError_t launch_tile(const LaunchArgs &p, hipStream_t s) {
  if (p.in_code == E_BF16) return launch_typed<HalfBF16, TL>(p, s);
  if (p.in_code == E_F16) return launch_typed<HalfF16, TL>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace w8

// bm: 256 (256 x 256 tiles, 32-deep slabs), 128 (128 x 128 tiles, 64-deep slabs) or
// 64 (64 x 64 tiles, 128-deep slabs).
hipError_t launch_w8(const LaunchArgs &p, int bm, hipStream_t s) {
  if (bm == 256) return w8::launch_tile<w8::Tile256>(p, s);
  if (bm == 128) return w8::launch_tile<w8::Tile128>(p, s);
  if (bm == 64) return w8::launch_tile<w8::Tile64>(p, s);
  return hipErrorInvalidValue;
}

}  // namespace mhg

// plan.cpp -- argument validation, the catalogue of compiled tile variants, the
// resource model and the shape-driven selector.  Host only, no HIP.
//
// The selector follows "Tiling 策略与内存层次优化" (constraints 1-3 and the
// autotuning section): enumerate the compiled variants, drop those that break the
// LDS budget (BM*BK + BK*BN) * elem * stages <= LDS per compute unit, then score
// the survivors.  The score multiplies three factors, each in [0, 1]:
//   * tile reuse: the tile intensity 2*BM*BN / ((BM+BN)*elem) from the same page,
//     relative to the largest tile in the catalogue;
//   * grid fill: how evenly the workgroups cover the compute units, in waves of
//     CUs x workgroups-per-CU ("GPU Kernel 的 Tile、Grid、Wave 与 Launch Overhead",
//     wave section: waves = CTAs / (SMs x CTAs per SM); its per-shape section
//     trades tile size against worker count the same way);
//   * useful work: the fraction of the padded grid area that lies inside C.
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cstdio>

#include "../../include/mhgemm.h"

namespace mhg {

namespace {

constexpr unsigned kF32 = 1u << E_F32;
constexpr unsigned kHalf = (1u << E_F16) | (1u << E_BF16);

// Registers per lane (VGPR + AGPR) each variant needs, from the compiler's
// resource report of the gfx950 build; used for the occupancy limit.
// Eight-wave variants come before the register-staged variant of the same tile so
// that they win ties; `fallback` names the register-staged variant run instead when
// the operands' alignment rules direct staging out at run time (a LauncherId; -1:
// none).
const Variant kCatalogue[] = {
    // kind            bm   bn   bk  wm wn st sk   thr  types  launcher           tm tn fallback
    {{GEMM_KIND_FMA, 32, 32, 32, 4, 1, 2, 1}, 256, kF32, L_FMA_32, 2, 2, -1},
    {{GEMM_KIND_FMA, 64, 64, 16, 4, 1, 2, 1}, 256, kF32, L_FMA_64, 4, 4, -1},
    // fp32 on the matrix cores (v_mfma_f32_32x32x2_f32); ahead of the FMA tile of the same size
    {{GEMM_KIND_MFMA, 128, 128, 16, 2, 2, 2, 1}, 256, kF32, L_MFMA32_128, 4, 4, -1},
    {{GEMM_KIND_FMA, 128, 128, 16, 4, 1, 2, 1}, 256, kF32, L_FMA_128, 8, 8, -1},
    {{GEMM_KIND_MFMA, 64, 64, 128, 2, 4, 5, 1}, 512, kHalf, L_W8_64, 2, 2, L_MFMA_64x64},
    {{GEMM_KIND_MFMA, 64, 64, 64, 2, 2, 2, 1}, 256, kHalf, L_MFMA_64x64, 2, 2, -1},
    {{GEMM_KIND_MFMA, 128, 128, 64, 2, 4, 5, 1}, 512, kHalf, L_W8_128, 4, 4, L_MFMA_128x128},
    {{GEMM_KIND_MFMA, 128, 128, 64, 2, 2, 2, 1}, 256, kHalf, L_MFMA_128x128, 4, 4, -1},
    {{GEMM_KIND_MFMA, 256, 128, 64, 2, 2, 2, 1}, 256, kHalf, L_MFMA_256x128, 8, 4, -1},
    {{GEMM_KIND_MFMA, 256, 256, 32, 2, 4, 5, 1}, 512, kHalf, L_W8_256, 8, 4, L_MFMA_256x256},
    {{GEMM_KIND_MFMA, 256, 256, 64, 2, 4, 2, 1}, 512, kHalf, L_MFMA_256x256, 8, 4, -1},
    // Eight-wave tiles with K split across workgroups: for grids of tiles that leave
    // most compute units idle (fp32 partials added in chunk order by a second kernel).
    {{GEMM_KIND_MFMA, 64, 64, 128, 2, 4, 5, 2}, 512, kHalf, L_W8_64, 2, 2, L_MFMA_64x64},
    {{GEMM_KIND_MFMA, 64, 64, 128, 2, 4, 5, 4}, 512, kHalf, L_W8_64, 2, 2, L_MFMA_64x64},
    {{GEMM_KIND_MFMA, 64, 64, 128, 2, 4, 5, 8}, 512, kHalf, L_W8_64, 2, 2, L_MFMA_64x64},
    {{GEMM_KIND_MFMA, 128, 128, 64, 2, 4, 5, 2}, 512, kHalf, L_W8_128, 4, 4, L_MFMA_128x128},
    {{GEMM_KIND_MFMA, 128, 128, 64, 2, 4, 5, 4}, 512, kHalf, L_W8_128, 4, 4, L_MFMA_128x128},
    {{GEMM_KIND_MFMA, 128, 128, 64, 2, 4, 5, 8}, 512, kHalf, L_W8_128, 4, 4, L_MFMA_128x128},
    // M <= 16: one workgroup per 128 columns and K chunk (split-K factor last).
    {{GEMM_KIND_SKINNY, 16, 128, 32, 1, 4, 2, 1}, 256, kHalf, L_SKINNY, 1, 8, L_MFMA_64x64},
    {{GEMM_KIND_SKINNY, 16, 128, 32, 1, 4, 2, 2}, 256, kHalf, L_SKINNY, 1, 8, L_MFMA_64x64},
    {{GEMM_KIND_SKINNY, 16, 128, 32, 1, 4, 2, 4}, 256, kHalf, L_SKINNY, 1, 8, L_MFMA_64x64},
    {{GEMM_KIND_SKINNY, 16, 128, 32, 1, 4, 2, 8}, 256, kHalf, L_SKINNY, 1, 8, L_MFMA_64x64},
    {{GEMM_KIND_SKINNY, 16, 128, 32, 1, 4, 2, 16}, 256, kHalf, L_SKINNY, 1, 8, L_MFMA_64x64},
};

// Largest tile intensity among the catalogue's tiles of an element size; the tile
// reuse factor is measured against it.
double best_intensity(int elem, unsigned mask) {
  double best = 0.0;
  for (const Variant &v : kCatalogue)
    if (v.in_mask & mask) best = std::max(best, tile_intensity(v.cfg.bm, v.cfg.bn, elem));
  return best;
}

// Registers per lane estimate: accumulators plus operand, staging and address
// registers.  FMA: TM*TN accumulators + TM + TN operands + staged elements.
// MFMA: 4 fp32 per 16x16 block + fragments + staged 16-byte chunks.
int regs_estimate(const Variant &v) {
  if (v.launcher == L_W8_256 || v.launcher == L_W8_128 || v.launcher == L_W8_64) return 256;   // two waves per SIMD
  if (v.launcher == L_SKINNY) return 128;    // 8 accumulators, two staged rounds, transposes
  if (v.launcher == L_MFMA32_128) return 128;   // 64 accumulators, 32 staged, fragments, addressing
  const TileConfig &c = v.cfg;
  if (c.kind == GEMM_KIND_FMA) {
    int staged = (c.bm * c.bk + c.bk * c.bn) / v.threads;
    return v.tm * v.tn + v.tm + v.tn + staged + 24;
  }
  int acc = v.tm * v.tn * 4;
  int frags = (v.tm + v.tn) * 4;
  int staged = (c.bm * c.bk + c.bk * c.bn) / 8 / v.threads * 4;
  return acc + frags + staged + 32;
}

}  // namespace

const Variant *catalogue(int *count) {
  *count = static_cast<int>(sizeof(kCatalogue) / sizeof(kCatalogue[0]));
  return kCatalogue;
}

const Variant *variant_of_launcher(int launcher) {
  for (const Variant &v : kCatalogue)
    if (v.launcher == launcher) return &v;
  return nullptr;
}

bool split_dtype(int dtype, int *in_code, int *out_code) {
  switch (dtype) {
    case GEMM_F32_F32: *in_code = E_F32; *out_code = E_F32; return true;
    case GEMM_F16_F16: *in_code = E_F16; *out_code = E_F16; return true;
    case GEMM_F16_F32: *in_code = E_F16; *out_code = E_F32; return true;
    case GEMM_BF16_BF16: *in_code = E_BF16; *out_code = E_BF16; return true;
    case GEMM_BF16_F32: *in_code = E_BF16; *out_code = E_F32; return true;
    default: return false;
  }
}

int elem_bytes(int code) { return code == E_F32 ? 4 : 2; }

int64_t lds_bytes_of(const TileConfig &c, int elem) {
  return (int64_t(c.bm) * c.bk + int64_t(c.bk) * c.bn) * elem * c.stages;
}

double tile_intensity(int bm, int bn, int elem) {
  return 2.0 * bm * bn / (double(bm + bn) * elem);
}

// LDS actually allocated: the MFMA tiles are swizzled (no padding); the FMA tiles
// pad each k-row by four elements.
static int64_t lds_allocated(const Variant &v, int elem) {
  const TileConfig &c = v.cfg;
  if (v.launcher == L_SKINNY) return int64_t(4) * 16 * c.bn * 4 + 16;   // wave partials, flag
  if (v.launcher == L_MFMA32_128)   // k-rows padded by 32 floats
    return (int64_t(c.bm + 32) * c.bk + int64_t(c.bn + 32) * c.bk) * elem * c.stages;
  if (c.kind == GEMM_KIND_FMA)
    return (int64_t(c.bm + 4) * c.bk + int64_t(c.bn + 4) * c.bk) * elem * c.stages;
  return lds_bytes_of(c, elem);
}

int workgroups_per_cu(const Variant &v, int elem, const Hardware &hw) {
  const int64_t lds = lds_allocated(v, elem);
  const int waves = v.threads / 64;
  int by_lds = lds > 0 ? int(hw.lds_bytes / lds) : 64;
  int by_waves = hw.simds_per_cu * hw.max_waves_per_simd / waves;
  int regs = regs_estimate(v);
  int waves_per_simd_by_regs = std::min(hw.max_waves_per_simd, hw.regs_per_lane / std::max(regs, 1));
  int by_regs = waves_per_simd_by_regs * hw.simds_per_cu / waves;
  return std::max(0, std::min(by_lds, std::min(by_waves, by_regs)));
}

double tail_efficiency(int64_t n_wg, int64_t slots) {
  if (n_wg <= 0 || slots <= 0) return 0.0;
  int64_t rounds = (n_wg + slots - 1) / slots;
  return double(n_wg) / double(rounds * slots);
}

bool validate(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
              int dtype, int layout, PlanData *p, std::string *err) {
  char buf[256];
  if (!split_dtype(dtype, &p->in_code, &p->out_code)) {
    std::snprintf(buf, sizeof buf, "gemm_plan: unknown dtype %d", dtype);
    *err = buf;
    return false;
  }
  if (layout < 0 || layout > (GEMM_A_COL | GEMM_B_COL)) {
    std::snprintf(buf, sizeof buf, "gemm_plan: unknown layout %d", layout);
    *err = buf;
    return false;
  }
  if (M < 0 || N < 0 || K < 0) {
    *err = "gemm_plan: negative extent";
    return false;
  }
  const int64_t kLimit = int64_t(1) << 31;
  if (M >= kLimit || N >= kLimit || K >= kLimit) {
    *err = "gemm_plan: extent of 2^31 or more";
    return false;
  }
  if (lda < 0 || ldb < 0 || ldc < 0) {
    *err = "gemm_plan: negative leading dimension";
    return false;
  }
  const bool a_col = layout & GEMM_A_COL, b_col = layout & GEMM_B_COL;
  if (M > 0 && K > 0 && lda < (a_col ? M : K)) {
    std::snprintf(buf, sizeof buf, "gemm_plan: lda=%lld below the contiguous extent %lld of A",
                  (long long)lda, (long long)(a_col ? M : K));
    *err = buf;
    return false;
  }
  if (K > 0 && N > 0 && ldb < (b_col ? K : N)) {
    std::snprintf(buf, sizeof buf, "gemm_plan: ldb=%lld below the contiguous extent %lld of B",
                  (long long)ldb, (long long)(b_col ? K : N));
    *err = buf;
    return false;
  }
  if (M > 0 && N > 0 && ldc < N) {
    std::snprintf(buf, sizeof buf, "gemm_plan: ldc=%lld below N=%lld", (long long)ldc, (long long)N);
    *err = buf;
    return false;
  }
  p->M = M; p->N = N; p->K = K;
  p->lda = lda; p->ldb = ldb; p->ldc = ldc;
  p->dtype = dtype; p->layout = layout;
  return true;
}

bool ring_shape_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, bool a_col, bool b_col,
                   int bm, int bn, int bk) {
  const int64_t a_ext = a_col ? M : K, b_ext = b_col ? K : N;
  if (a_ext % 8 || b_ext % 8 || lda % 8 || ldb % 8) return false;
  const int64_t a_span = (a_col ? bk : bm) * lda * 2, b_span = (b_col ? bn : bk) * ldb * 2;
  return a_span < (int64_t(1) << 31) && b_span < (int64_t(1) << 31);
}

bool needs_aligned_staging(int launcher) {
  return launcher == L_W8_256 || launcher == L_W8_128 || launcher == L_W8_64;
}

bool skinny_shape_ok(const PlanData &p, std::string *why) {
  const char *msg = nullptr;
  if (p.M > 16) msg = "variant for at most 16 rows of A";
  else if (p.layout & (GEMM_A_COL | GEMM_B_COL)) msg = "variant for at most 16 rows needs row-major A and B";
  else if (p.K % 8 || p.N % 8 || p.lda % 8 || p.ldb % 8)
    msg = "variant with direct 16-byte staging needs extents and leading dimensions that are multiples of 8";
  else if (p.K >= (int64_t(1) << 30) || p.lda >= (int64_t(1) << 25) || p.ldb >= (int64_t(1) << 25) ||
           (p.N + 127) / 128 * 16 * 128 * 4 * 16 >= (int64_t(1) << 31))
    msg = "variant for at most 16 rows needs K < 2^30, leading dimensions below 2^25 and N below 2^21";
  if (msg && why) *why = msg;
  return msg == nullptr;
}

int skinny_split(const PlanData &p, const Hardware &hw) {
  // More workgroups until every compute unit holds one (each keeps two rounds per
  // wave in flight, enough to cover the HBM latency; more chunks only add partials
  // to reduce), while each K chunk keeps at least 512 k (four rounds a wave).
  const int64_t gn = (p.N + 127) / 128;
  int s = 1;
  while (s < 16 && gn * s < int64_t(hw.cus) && p.K / (2 * s) >= 512) s *= 2;
  return s;
}

double score(const Variant &v, const PlanData &p, const Hardware &hw, std::string *why) {
  const int elem = elem_bytes(p.in_code);
  if (v.launcher == L_SKINNY && !skinny_shape_ok(p, why)) return -1.0;
  if (v.launcher != L_SKINNY && v.cfg.split_k > 1 && p.K < int64_t(2) * v.cfg.split_k * v.cfg.bk) {
    if (why) *why = "split-K variant needs at least two K slabs per chunk";
    return -1.0;
  }
  if (needs_aligned_staging(v.launcher) &&
      !ring_shape_ok(p.M, p.N, p.K, p.lda, p.ldb, p.layout & GEMM_A_COL, p.layout & GEMM_B_COL,
                     v.cfg.bm, v.cfg.bn, v.cfg.bk)) {
    if (why) *why = "variant with direct 16-byte staging needs extents and leading dimensions that are multiples of 8";
    return -1.0;
  }
  if (!(v.in_mask & (1u << p.in_code))) {
    if (why) *why = "variant does not take this input type";
    return -1.0;
  }
  if (lds_allocated(v, elem) > hw.lds_bytes) {
    if (why) *why = "LDS per workgroup exceeds the LDS of a compute unit";
    return -1.0;
  }
  const int per_cu = workgroups_per_cu(v, elem, hw);
  if (per_cu < 1) {
    if (why) *why = "no workgroup fits a compute unit";
    return -1.0;
  }
  const TileConfig &c = v.cfg;
  const int64_t gm = (p.M + c.bm - 1) / c.bm, gn = (p.N + c.bn - 1) / c.bn;
  const int64_t n_wg = gm * gn * c.split_k;
  if (n_wg >= (int64_t(1) << 31)) {
    if (why) *why = "grid too large";
    return -1.0;
  }
  const int64_t slots = int64_t(hw.cus) * per_cu;
  double fill = n_wg >= slots ? tail_efficiency(n_wg, slots)
                              : std::min(1.0, double(n_wg) / hw.cus);
  double useful = double(p.M) * double(p.N) / (double(gm * c.bm) * double(gn * c.bn));
  double reuse = tile_intensity(c.bm, c.bn, elem) / best_intensity(elem, 1u << p.in_code);
  return fill * useful * reuse;
}

static void fill_plan(PlanData *p, int idx, const Hardware &hw) {
  int n;
  const Variant *cat = catalogue(&n);
  const Variant &v = cat[idx];
  p->variant = idx;
  p->cfg = v.cfg;
  p->gm = int((p->M + v.cfg.bm - 1) / v.cfg.bm);
  p->gn = int((p->N + v.cfg.bn - 1) / v.cfg.bn);
  p->gz = v.cfg.split_k;
  p->threads = v.threads;
  p->lds_bytes = int(lds_allocated(v, elem_bytes(p->in_code)));
  p->cus = hw.cus;
  // Walk tiles in groups of rows so that workgroups running together share A
  // row-panels and B column-panels in L2.
  p->group_m = std::max(1, std::min(p->gm, 4));
  p->ws_bytes = 0;
  if (v.launcher == L_SKINNY && v.cfg.split_k > 1)   // arrival counters, then partials
    p->ws_bytes = (int64_t(p->gn) * 4 + 255) / 256 * 256 + int64_t(v.cfg.split_k) * p->gn * 16 * v.cfg.bn * 4;
  if (v.launcher != L_SKINNY && v.cfg.split_k > 1)   // one fp32 partial of C per K chunk
    p->ws_bytes = int64_t(v.cfg.split_k) * p->M * p->N * 4;
}

bool select(PlanData *p, const Hardware &hw, std::string *err) {
  if (p->M == 0 || p->N == 0 || p->K == 0) {
    p->variant = -1;
    p->cfg = TileConfig{GEMM_KIND_NONE, 0, 0, 0, 0, 0, 0, 1};
    p->gm = p->gn = 0;
    p->gz = 1;
    p->threads = 0;
    p->lds_bytes = 0;
    p->cus = hw.cus;
    return true;
  }
  int n;
  const Variant *cat = catalogue(&n);
  // At most 16 rows: the product streams B once and is bound by HBM, not by tile
  // reuse, so the split-K kernel is taken whenever it applies.
  if (p->M <= 16 && (1u << p->in_code) & kHalf && skinny_shape_ok(*p, nullptr)) {
    const int split = skinny_split(*p, hw);
    for (int i = 0; i < n; ++i)
      if (cat[i].launcher == L_SKINNY && cat[i].cfg.split_k == split && score(cat[i], *p, hw, nullptr) >= 0.0) {
        fill_plan(p, i, hw);
        return true;
      }
  }
  int best = -1;
  double best_score = -1.0;
  for (int i = 0; i < n; ++i) {
    if (cat[i].launcher == L_SKINNY || cat[i].cfg.split_k > 1) continue;
    double s = score(cat[i], *p, hw, nullptr);
    if (s > best_score + 1e-12) {
      best_score = s;
      best = i;
    }
  }
  if (best < 0 || best_score <= 0.0) {
    *err = "gemm_plan: no compiled variant fits this problem";
    return false;
  }
  // Too few workers ("GPU Kernel 的 Tile、Grid、Wave 与 Launch Overhead", per-shape
  // section): when the chosen eight-wave tile's grid covers at most half the compute
  // units, K is split across workgroups as well, by the smallest power of two (at
  // most 8) that covers three quarters of them, keeping at least four K slabs per
  // chunk.  (Measured: 768 x 512 x 4096, 96 tiles: split 2 18.0 us, split 4 20.9 us.)
  const Variant &b = cat[best];
  const int64_t tiles = ((p->M + b.cfg.bm - 1) / b.cfg.bm) * ((p->N + b.cfg.bn - 1) / b.cfg.bn);
  if ((b.launcher == L_W8_64 || b.launcher == L_W8_128) && 2 * tiles <= hw.cus) {
    int split = 1;
    while (split < 8 && 4 * tiles * split < 3 * int64_t(hw.cus) && p->K >= int64_t(4) * (2 * split) * b.cfg.bk)
      split *= 2;
    for (int i = 0; split > 1 && i < n; ++i)
      if (cat[i].launcher == b.launcher && cat[i].cfg.split_k == split && score(cat[i], *p, hw, nullptr) >= 0.0) {
        best = i;
        break;
      }
  }
  fill_plan(p, best, hw);
  return true;
}

bool force(PlanData *p, const Hardware &hw, const int32_t cfg[8], std::string *err) {
  if (p->M == 0 || p->N == 0 || p->K == 0) return select(p, hw, err);
  int n;
  const Variant *cat = catalogue(&n);
  for (int i = 0; i < n; ++i) {
    const TileConfig &c = cat[i].cfg;
    if (c.kind == cfg[0] && c.bm == cfg[1] && c.bn == cfg[2] && c.bk == cfg[3] &&
        c.waves_m == cfg[4] && c.waves_n == cfg[5] && c.stages == cfg[6] && c.split_k == cfg[7]) {
      std::string why;
      if (score(cat[i], *p, hw, &why) < 0.0) {
        *err = "gemm_plan_config: " + why;
        return false;
      }
      fill_plan(p, i, hw);
      return true;
    }
  }
  char buf[200];
  std::snprintf(buf, sizeof buf,
                "gemm_plan_config: no compiled variant kind=%d %dx%dx%d waves %dx%d stages %d split %d",
                cfg[0], cfg[1], cfg[2], cfg[3], cfg[4], cfg[5], cfg[6], cfg[7]);
  *err = buf;
  return false;
}

}  // namespace mhg

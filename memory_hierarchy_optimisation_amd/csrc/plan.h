// plan.h -- host-side plan, catalogue and launch arguments (no HIP types here, so the
// selector compiles and unit-tests on a machine without a GPU).
#pragma once

#include <cstddef>
#include <cstdint>
#include <string>

namespace mhg {

// Element codes of inputs and outputs.
enum Elem { E_F32 = 0, E_F16 = 1, E_BF16 = 2 };

// Launcher identities: one per compiled kernel variant family (capi.hip maps them).
enum LauncherId {
  L_FMA_32 = 0,
  L_FMA_64,
  L_FMA_128,
  L_MFMA_64x64,
  L_MFMA_128x128,
  L_MFMA_256x128,
  L_MFMA_256x256,
  L_SKINNY,
  L_W8_256,
  L_W8_128,
  L_W8_64,
  L_MFMA32_128,
  L_COUNT
};

// One tile configuration, in the vocabulary of the pages' tile-config tuple
// (BLOCK_M, BLOCK_N, BLOCK_K, warps, stages) plus the split-K factor.
struct TileConfig {
  int kind;      // gemm_kind
  int bm, bn, bk;
  int waves_m, waves_n;
  int stages;
  int split_k;
};

struct Variant {
  TileConfig cfg;
  int threads;
  unsigned in_mask;   // bit e set: input element code e supported
  int launcher;       // LauncherId
  int tm, tn;         // per-lane register tile (FMA) or per-wave 16x16 MFMA blocks (MFMA)
  int fallback;       // LauncherId run instead when run-time checks rule this one out (-1: none)
};

// Variants with direct global-to-LDS loads need 16-byte aligned operands whose
// contiguous extents and leading dimensions are multiples of 8 elements, and slab
// offsets below 2^31 bytes.
bool ring_shape_ok(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, bool a_col, bool b_col,
                   int bm, int bn, int bk);
// Variants with a fallback need direct 16-byte staging; the plan checks what it can see
// (extents and leading dimensions), gemm_run checks pointer alignment.
bool needs_aligned_staging(int launcher);
// The split-K variant for at most 16 rows: the shape rules, and the split factor the
// selector takes (powers of two up to 16, one workgroup per compute unit, K chunks of
// at least 512).
struct PlanData;
bool skinny_shape_ok(const PlanData &p, std::string *why);
struct Hardware;
int skinny_split(const PlanData &p, const Hardware &hw);

// Hardware description used by the resource model.
struct Hardware {
  int cus = 256;                 // compute units (MI355X: 8 XCDs x 32)
  int xcds = 8;
  int lds_bytes = 160 * 1024;    // LDS per compute unit
  int simds_per_cu = 4;
  int max_waves_per_simd = 8;
  int regs_per_lane = 512;       // VGPR + AGPR file per lane of a SIMD
};

// Arguments every kernel launcher takes (plain values; device pointers as void*).
struct LaunchArgs {
  const void *A;
  const void *B;
  void *C;
  int64_t M, N, K, lda, ldb, ldc;
  int in_code;     // Elem
  int out_code;    // Elem
  int a_col, b_col;
  int vec_a, vec_b;   // 1: 16-byte loads allowed (aligned base and leading dimension)
  int c_vec;          // 1: C's base and leading dimension allow 4-element vector stores
  int gm, gn;         // tiles along M and N
  int split_k;
  int group_m;        // rows of tiles walked together (L2 locality)
  void *workspace;
  int64_t ws_bytes;
  int64_t k_chunk;     // split-K of the eight-wave kernels: K per chunk (a multiple of BK)
  // Fused epilogue, C = act(alpha * product + beta * prior C + bias[column]); epi = 0 is
  // the plain product (alpha 1, beta 0, no bias, no activation) and skips all of it.
  int epi;
  float alpha, beta;
  const float *bias;   // N fp32 values or NULL
  int bias_vec;        // 1: bias is 16-byte aligned (four values a load)
  int act;             // gemm_activation
};

struct PlanData {
  int64_t M = 0, N = 0, K = 0, lda = 0, ldb = 0, ldc = 0;
  int dtype = 0, layout = 0;
  int in_code = 0, out_code = 0;
  int variant = -1;          // catalogue index; -1 when there is no product (kind NONE)
  TileConfig cfg{};
  int gm = 0, gn = 0, gz = 1;
  int threads = 0;
  int lds_bytes = 0;
  int cus = 256;
  int group_m = 1;
  int64_t ws_bytes = 0;
};

// Catalogue of compiled variants.
const Variant *catalogue(int *count);
const Variant *variant_of_launcher(int launcher);

// Input / output element codes of a gemm_dtype, or false when unknown.
bool split_dtype(int dtype, int *in_code, int *out_code);
int elem_bytes(int code);

// The pages' formulas the selector uses.
int64_t lds_bytes_of(const TileConfig &c, int elem);           // (BM*BK + BK*BN) * elem * stages
double tile_intensity(int bm, int bn, int elem);                // 2*BM*BN / ((BM+BN)*elem)
int workgroups_per_cu(const Variant &v, int elem, const Hardware &hw);
// Registers per lane (VGPR + AGPR) a wave of the variant holds, from the build's report.
int registers_of(const Variant &v);
double tail_efficiency(int64_t n_wg, int64_t slots);            // n / (ceil(n/slots) * slots)

// Validate arguments and fill the shape part of a plan.  Returns false and sets *err.
bool validate(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
              int dtype, int layout, PlanData *p, std::string *err);

// Score of a variant for the plan's shape (higher is better; < 0 means infeasible).
double score(const Variant &v, const PlanData &p, const Hardware &hw, std::string *why);

// Choose a variant (or kind NONE) and fill grid, threads, LDS and workspace fields.
bool select(PlanData *p, const Hardware &hw, std::string *err);

// Force a configuration; fails if it is not compiled or infeasible.
bool force(PlanData *p, const Hardware &hw, const int32_t cfg[8], std::string *err);

// Configuration recorded for exactly this problem by gemm_autotune or gemm_tune_load
// (tune.cpp); false when there is none.
bool tuned_lookup(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
                  int layout, int32_t cfg[8]);

}  // namespace mhg

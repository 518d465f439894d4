/*
 * mhgemm.h -- C ABI of the tiled dense matrix multiply for the AMD MI355X (gfx950).
 *
 * The operation (the element formula of the product in "CUDA tile", 2.1, and the
 * GEMM example of the roofline section of "Tiling 策略与内存层次优化"):
 *
 *     C[i][j] = sum over k in [0, K) of A(i,k) * B(k,j),   0 <= i < M, 0 <= j < N,
 *
 * with products of the input element type accumulated in fp32 and the sum written
 * once to C in the output element type (fp32 as is; fp16 / bf16 rounded to nearest,
 * ties to even).  C is overwritten: there is no alpha / beta scaling.
 *
 * Storage (elements, not bytes; every leading dimension counts elements):
 *     A row-major:    A(i,k) = A[i*lda + k]      requires lda >= K
 *     A column-major: A(i,k) = A[k*lda + i]      requires lda >= M
 *     B row-major:    B(k,j) = B[k*ldb + j]      requires ldb >= N
 *     B column-major: B(k,j) = B[j*ldb + k]      requires ldb >= K   ("K-contiguous")
 *     C row-major:    C(i,j) = C[i*ldc + j]      requires ldc >= N
 * A leading dimension is only checked against its extent when both extents of the
 * operand are non-zero.
 *
 * Work split (the three tiling levels of "Tiling 策略与内存层次优化", multi-level
 * tiling section): each workgroup owns one BM x BN tile of C, walks K in BK-deep
 * slabs staged through LDS, and each wave accumulates a register tile with matrix
 * (MFMA) instructions for fp16 / bf16 inputs or fused multiply-adds for fp32 inputs.
 * The launch grid is ceil(M/BM) x ceil(N/BN) workgroups (scheduling stage of the
 * same page), times the split-K factor where the plan splits K across workgroups.
 *
 * Ownership: A, B and C are device pointers owned by the caller.  A plan is an
 * immutable host object; it may own a device workspace (split-K partial sums), which
 * gemm_destroy frees.  Calls that run the same plan on different streams
 * concurrently must use distinct C; a plan with a workspace (see
 * gemm_plan_describe, field 15) must not run concurrently with itself.  C must not
 * alias A or B.
 *
 * Errors: gemm_plan and gemm_plan_config return NULL on invalid arguments and set a
 * thread-local message readable with gemm_last_error.  gemm_run returns GEMM_OK or
 * a negative GEMM_ERR_* code.  gemm_run is asynchronous on the given stream; a
 * device-side fault surfaces at the caller's next synchronisation of that stream.
 */
#ifndef MHGEMM_H
#define MHGEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gemm_plan_s *gemm_plan_t;

/* <input type>_<output type>; accumulation is always fp32. */
enum gemm_dtype {
    GEMM_F32_F32 = 0,
    GEMM_F16_F16 = 1,
    GEMM_F16_F32 = 2,
    GEMM_BF16_BF16 = 3,
    GEMM_BF16_F32 = 4
};

/* layout = (A flag) | (B flag).  C is always row-major. */
enum gemm_layout {
    GEMM_A_ROW = 0,
    GEMM_A_COL = 1,
    GEMM_B_ROW = 0,
    GEMM_B_COL = 2
};

enum gemm_status {
    GEMM_OK = 0,
    GEMM_ERR_INVALID_ARG = -1,
    GEMM_ERR_UNSUPPORTED = -2,
    GEMM_ERR_HIP = -3,
    GEMM_ERR_ALLOC = -4
};

/* Kernel families a plan can select (field 0 of gemm_plan_describe). */
enum gemm_kind {
    GEMM_KIND_NONE = 0,   /* M == 0, N == 0 or K == 0: no product to compute */
    GEMM_KIND_FMA = 1,    /* fp32: LDS-staged slabs, per-lane TM x TN register tile of FMAs */
    GEMM_KIND_MFMA = 2,   /* fp16 / bf16: LDS-staged slabs, per-wave MFMA register tiles */
    GEMM_KIND_SKINNY = 3  /* fp16 / bf16, M <= 16: K split across waves and workgroups */
};

/*
 * gemm_plan -- validate a problem and choose its tile configuration and grid.
 *
 * Host only; queries the current HIP device's compute-unit count once, and falls
 * back to the MI355X's 256 compute units when no device answers.  The choice
 * follows the pages' feasibility rules ("Tiling 策略与内存层次优化", constraints 1-3:
 * LDS bytes = (BM*BK + BK*BN) * elem * stages within the 160 KB LDS of a compute
 * unit, registers without spills, occupancy) and scores the survivors by tile
 * arithmetic intensity 2*BM*BN / ((BM+BN)*elem) (same page, how tiling raises
 * intensity) and by how evenly the workgroups fill the compute units ("GPU
 * Kernel 的 Tile、Grid、Wave 与 Launch Overhead", wave section and per-shape
 * choices).  M, N, K >= 0; dtype a gemm_dtype; layout a gemm_layout combination.
 * Returns NULL on invalid arguments (message via gemm_last_error).  A plan for
 * M == 0 or N == 0 runs as a no-op; a plan for K == 0 fills C with zeros (the
 * empty sum).
 *
 * M <= 16 (fp16 / bf16, row-major A and B, K, N, lda, ldb multiples of 8) selects
 * GEMM_KIND_SKINNY: such a product streams B once and is bound by HBM bandwidth
 * ("Tiling 策略与内存层次优化", roofline: intensity far left of the ridge), so K is
 * also split across workgroups until every compute unit holds one ("GPU Kernel 的
 * Tile、Grid、Wave 与 Launch Overhead", per-shape section: too few workers).  With a
 * split factor above 1 the plan owns a device workspace of arrival counters and fp32
 * partials (gemm_plan_describe field 15), allocated on the current device here when
 * one is present (otherwise on the first gemm_run) and freed by gemm_destroy; it
 * returns NULL (GEMM_ERR_ALLOC message) when that allocation fails.
 */
gemm_plan_t gemm_plan(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                      int dtype, int layout);

/*
 * gemm_plan_config -- like gemm_plan, but with the tile configuration forced.
 *
 * cfg[0..7] = { kind (gemm_kind), BM, BN, BK, waves along M, waves along N,
 * LDS stages, split-K factor }.  The configuration must be one of the compiled
 * variants for this input type (gemm_plan_describe of a gemm_plan result shows
 * valid ones) and must fit the LDS budget; otherwise NULL with a message.  For
 * sweeps of the tile space ("Tiling 策略与内存层次优化", autotuning section) and for
 * the pages' worked launch geometries (e.g. a 64 x 64 product as 2 x 2 tiles of
 * 32 x 32, "CUDA tile", 2.1).
 */
gemm_plan_t gemm_plan_config(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                             int64_t ldc, int dtype, int layout, const int32_t cfg[8]);

/*
 * gemm_run -- enqueue C = A x B on a HIP stream (hipStream_t passed as void *;
 * NULL is the null stream).  A, B, C: device pointers laid out as described at the
 * top of this file.  Pointers need only element alignment: operands whose base
 * address, leading dimension or contiguous extent is not a multiple of 16 bytes
 * are staged with narrower loads.  NULL operands are rejected when the operand has
 * elements to read or write.  Returns GEMM_OK, GEMM_ERR_INVALID_ARG, GEMM_ERR_HIP
 * when the launch itself fails, GEMM_ERR_ALLOC when a split-K workspace deferred from
 * gemm_plan cannot be allocated (that first run allocates; later runs do not), or
 * GEMM_ERR_UNSUPPORTED when the plan's workspace lives on another device than the
 * current one.  Never synchronises otherwise.  Split-K results are reproducible bit
 * for bit: partials are added in a fixed order whatever the workgroups' order.
 */
int gemm_run(gemm_plan_t plan, const void *A, const void *B, void *C, void *stream);

/* Activation of the fused epilogue. */
enum gemm_activation {
    GEMM_ACT_NONE = 0,
    GEMM_ACT_RELU = 1    /* max(t, 0); anything not above zero, NaN included, becomes +0 */
};

/* Fused epilogue: element-wise work on the product tile on its way to C. */
typedef struct gemm_epilogue {
    float alpha;         /* multiplies the accumulated product */
    float beta;          /* multiplies the prior contents of C; 0: C is only written */
    const float *bias;   /* device pointer to N fp32 values added to every row, or NULL */
    int32_t activation;  /* gemm_activation, applied last */
} gemm_epilogue_t;

/*
 * gemm_run_epilogue -- gemm_run with a fused epilogue ("Tiling 策略与内存层次优化",
 * fusion stage: element-wise post-processing such as bias add or ReLU done on the
 * GEMM tile's output before it is written back to HBM):
 *
 *     C[i][j] = act(alpha * sum_k A(i,k) B(k,j) + beta * C_prior[i][j] + bias[j])
 *
 * evaluated in fp32 (C_prior converted exactly from the output type), then rounded
 * once to the output type as in gemm_run.  beta == 0 reads nothing from C; bias may
 * be NULL; K == 0 gives act(beta * C_prior + bias).  epi == NULL, or alpha 1, beta 0,
 * no bias and no activation, is exactly gemm_run.  Same operands, stream semantics
 * and status codes as gemm_run; GEMM_ERR_INVALID_ARG also for an unknown activation
 * or a bias pointer that is not 4-byte aligned.  With beta != 0, C must hold valid
 * values of the output type, and C must not alias the bias.
 */
int gemm_run_epilogue(gemm_plan_t plan, const void *A, const void *B, void *C,
                      const gemm_epilogue_t *epi, void *stream);

/*
 * gemm_run_noalloc -- gemm_run_epilogue for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the problem is planned on the host as gemm_plan would plan it (tuned
 * table first, then the selector) and run at once, with no plan object.  A split-K
 * plan's workspace (arrival counters and fp32 partial sums) lives in a 16 MiB array
 * of device memory that the library holds on every GPU it runs on until the process
 * ends; nothing is allocated per call (the first call on a device looks up the
 * array's address there).  A plan whose workspace exceeds 16 MiB is rejected with
 * GEMM_ERR_UNSUPPORTED and a message.  All calls on one GPU share that array: calls
 * that may overlap in time on one GPU (different streams, or different threads) race
 * and give wrong results when their plans use split-K; serialise them.  Arguments
 * are those of gemm_plan followed by those of gemm_run_epilogue (epi may be NULL);
 * same results bit for bit as gemm_plan + gemm_run_epilogue, same status codes, plus
 * GEMM_ERR_INVALID_ARG for a problem gemm_plan rejects.  Asynchronous on `stream`.
 */
int gemm_run_noalloc(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
                     int layout, const void *A, const void *B, void *C, const gemm_epilogue_t *epi, void *stream);

/*
 * gemm_transpose -- out = transpose of in, the second tiled workload of "CUDA tile"
 * (applications section: a tile staged through shared memory makes both the reads
 * and the writes of a transpose coalesced):
 *
 *     out[c * ld_out + r] = in[r * ld_in + c],   0 <= r < rows, 0 <= c < cols.
 *
 * in: rows x cols, row-major, leading dimension ld_in >= cols; out: cols x rows,
 * row-major, ld_out >= rows; both device pointers of elem_bytes-byte elements
 * (2: fp16 / bf16, 4: fp32; the bytes are moved, not interpreted), aligned to the
 * element.  Elements of out outside the cols x rows block are not touched; out must
 * not overlap in.  Extents up to 2^31.  rows == 0 or cols == 0 is a no-op.
 * Asynchronous on `stream`.  Returns GEMM_OK, GEMM_ERR_INVALID_ARG (negative extent,
 * elem_bytes not 2 or 4, leading dimension too small, NULL or misaligned pointer) or
 * GEMM_ERR_HIP when the launch fails.
 */
int gemm_transpose(const void *in, void *out, int64_t rows, int64_t cols, int64_t ld_in, int64_t ld_out,
                   int32_t elem_bytes, void *stream);

/*
 * gemm_clock_probe -- a measurement helper beside the product (the pages' profiling
 * advice asks for the conditions a kernel ran under, and the clock of this part
 * moves with its load).  Launches one wave on `stream` that waits `ticks` periods of
 * the constant 100 MHz real-time counter and writes out[0] = shader-clock cycles and
 * out[1] = real-time ticks (>= ticks) elapsed over that window; the average shader
 * clock in MHz is 100 * out[0] / out[1].  Run on a second stream while GEMM calls run
 * on another, it reads the clock they run at.  out: device pointer to two uint64,
 * 8-byte aligned; 1 <= ticks <= 1e9 (ten seconds).  Asynchronous.  Returns GEMM_OK,
 * GEMM_ERR_INVALID_ARG or GEMM_ERR_HIP.
 */
int gemm_clock_probe(uint64_t *out, int64_t ticks, void *stream);

/* gemm_destroy -- release a plan and its workspace.  NULL is ignored. */
void gemm_destroy(gemm_plan_t plan);

/* gemm_last_error -- message of the last failure on this thread ("" if none). */
const char *gemm_last_error(void);

/*
 * gemm_plan_describe -- the chosen configuration, for tests and reports.
 * out[0..15] = { kind, BM, BN, BK, waves along M, waves along N, stages, split-K,
 *                grid x, grid y, grid z, threads per workgroup, LDS bytes per
 *                workgroup, compute units assumed, catalogue index,
 *                workspace bytes }.
 * Returns GEMM_OK, or GEMM_ERR_INVALID_ARG for a NULL plan or output.
 */
int gemm_plan_describe(gemm_plan_t plan, int32_t out[16]);

/*
 * gemm_catalogue -- the compiled variants, the candidate set of autotuning.
 * Writes min(count, max_cfgs) configurations as 8 int32 each (the layout of
 * gemm_plan_config's cfg) to cfgs (may be NULL) and returns the count.
 */
int gemm_catalogue(int32_t *cfgs, int32_t max_cfgs);

/*
 * gemm_catalogue_registers -- for each catalogue entry, the registers per lane (VGPR +
 * AGPR, in allocation granules) that the planner's occupancy filter assumes a wave of
 * it holds ("Tiling 策略与内存层次优化", constraint 2: the register budget decides how
 * many warps stay resident): the largest kernel of its family in the compiler's
 * resource report of this build.  Writes min(count, max_regs) values to regs (may be
 * NULL) in catalogue order and returns the count.
 */
int gemm_catalogue_registers(int32_t *regs, int32_t max_regs);

/*
 * gemm_autotune -- measure every compiled variant on one problem and keep the
 * fastest ("Tiling 策略与内存层次优化", autotuning section: enumerate the tile
 * configurations, filter out those that break the hardware limits, benchmark each
 * on the target, choose the best).
 *
 * The problem arguments are those of gemm_plan; A, B and C are the caller's device
 * operands in that layout (C is overwritten with the product).  Each variant that
 * gemm_plan_config accepts for the problem runs twice untimed, then twice `reps`
 * calls (1 <= reps <= 100000) between HIP events on `stream`; its time is the better
 * batch's mean per call.  The fastest configuration is stored in a process-wide
 * table that gemm_plan consults for this exact problem (all eight arguments equal)
 * before its heuristic; a plan already made is not changed.  Outputs, each optional:
 * best_cfg[8] (the gemm_plan_config layout), *best_us, and times_us[i] for catalogue
 * entry i < n_times (microseconds per call, -1 for a variant that does not fit).
 * Synchronises `stream`; allocates and frees split-K workspaces of the candidates.
 * Returns GEMM_OK, GEMM_ERR_INVALID_ARG (bad problem, empty product, NULL operand,
 * reps out of range, n_times > 0 with NULL times_us), GEMM_ERR_UNSUPPORTED (no variant
 * fits) or GEMM_ERR_HIP (a candidate failed to run; message names it).  Thread-safe
 * with respect to the table; do not run it concurrently on the same C.
 */
int gemm_autotune(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                  int dtype, int layout, const void *A, const void *B, void *C, void *stream,
                  int32_t reps, int32_t best_cfg[8], float *best_us, float *times_us, int32_t n_times);

/*
 * gemm_tune_save / gemm_tune_load / gemm_tune_clear -- the table of tuned choices.
 * The file is text: '#' comment lines, then one line per problem,
 *     M N K lda ldb ldc dtype layout | kind BM BN BK waves_m waves_n stages split_k | us
 * save writes the whole table and returns the number of entries; load checks every
 * line (a valid non-empty problem, a compiled configuration), then merges all of
 * them into the table (an entry replaces one for the same problem) and returns
 * their number; on any bad line it loads nothing and returns GEMM_ERR_INVALID_ARG
 * with the line number in gemm_last_error.  A stored configuration that no longer
 * fits when gemm_plan runs (for instance another compute-unit count) is ignored
 * there in favour of the heuristic.  clear empties the table.
 */
int gemm_tune_save(const char *path);
int gemm_tune_load(const char *path);
void gemm_tune_clear(void);

#ifdef __cplusplus
}
#endif

#endif /* MHGEMM_H */

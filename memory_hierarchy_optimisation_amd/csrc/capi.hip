// capi.hip -- the extern "C" boundary declared in include/mhgemm.h.
//
// gemm_plan validates and selects a tile configuration on the host; gemm_run checks
// pointers, decides per operand whether 16-byte loads are legal (aligned base and
// leading dimension), and enqueues one kernel on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "../../include/mhgemm.h"
#include "plan.h"

namespace mhg {
hipError_t launch_fma(int launcher, const LaunchArgs &p, hipStream_t s);
hipError_t launch_mfma(int launcher, const LaunchArgs &p, hipStream_t s);
hipError_t launch_fill(const LaunchArgs &p, hipStream_t s);
hipError_t launch_w8(const LaunchArgs &p, int bm, hipStream_t s);
hipError_t launch_skinny(const LaunchArgs &p, hipStream_t s);
hipError_t launch_mfma32(const LaunchArgs &p, hipStream_t s);
hipError_t launch_zero_words(void *w, int64_t n, hipStream_t s);
hipError_t launch_transpose(const void *in, void *out, int64_t rows, int64_t cols, int64_t ld_in, int64_t ld_out,
                            int elem_bytes, hipStream_t s);
hipError_t launch_clock_probe(uint64_t *out, uint64_t ticks, hipStream_t s);
}  // namespace mhg

struct gemm_plan_s {
  mhg::PlanData d;
  void *ws = nullptr;   // split-K workspace (device memory), or NULL
  int ws_dev = -1;      // device it lives on
};

namespace {

thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }

// Compute units of the current device; the MI355X's 256 when no device answers
// (planning is host-only and also runs where there is no GPU).
mhg::Hardware query_hardware() {
  mhg::Hardware hw;
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      hw.cus = cus;
  }
  (void)hipGetLastError();
  return hw;
}

// 32-bit arrival counters at the start of a split-K workspace (one per column block,
// padded to 256 bytes).
int64_t counter_words(const mhg::PlanData &d) { return (int64_t(d.gn) * 4 + 255) / 256 * 64; }

// Validate a problem and choose its configuration (forced, tuned or by the selector):
// host work only, nothing allocated on a device.  False with the message set.
bool choose_plan(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype, int layout,
                 const int32_t *cfg, mhg::PlanData *out) {
  mhg::PlanData d;
  std::string err;
  if (!mhg::validate(M, N, K, lda, ldb, ldc, dtype, layout, &d, &err)) {
    set_error(err);
    return false;
  }
  const mhg::Hardware hw = query_hardware();
  // A configuration measured fastest for exactly this problem (gemm_autotune, or a
  // table read by gemm_tune_load) wins over the heuristic while it still fits.
  bool ok;
  if (cfg) {
    ok = mhg::force(&d, hw, cfg, &err);
  } else {
    bool tuned_ok = false;
    int32_t tuned[8];
    if (M > 0 && N > 0 && K > 0 && mhg::tuned_lookup(M, N, K, lda, ldb, ldc, dtype, layout, tuned)) {
      mhg::PlanData t = d;
      std::string ignored;
      if (mhg::force(&t, hw, tuned, &ignored)) {
        d = t;
        tuned_ok = true;
      }
    }
    ok = tuned_ok || mhg::select(&d, hw, &err);
  }
  if (!ok) {
    set_error(err);
    return false;
  }
  *out = d;
  return true;
}

gemm_plan_t make_plan(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                      int dtype, int layout, const int32_t *cfg) {
  mhg::PlanData d;
  if (!choose_plan(M, N, K, lda, ldb, ldc, dtype, layout, cfg, &d)) return nullptr;
  gemm_plan_s *plan = new (std::nothrow) gemm_plan_s;
  if (!plan) {
    set_error("gemm_plan: out of host memory");
    return nullptr;
  }
  plan->d = d;
  // A workspace is allocated here when a device is present (its arrival counters
  // zeroed), else on the plan's first run.
  int dev = -1;
  if (d.ws_bytes > 0 && hipGetDevice(&dev) == hipSuccess) {
    if (hipMalloc(&plan->ws, size_t(d.ws_bytes)) != hipSuccess ||
        hipMemset(plan->ws, 0, size_t(counter_words(d)) * 4) != hipSuccess) {
      (void)hipGetLastError();
      if (plan->ws) (void)hipFree(plan->ws);
      delete plan;
      set_error("gemm_plan: cannot allocate the split-K workspace");
      return nullptr;
    }
    plan->ws_dev = dev;
  }
  (void)hipGetLastError();
  set_error("");
  return plan;
}

// Make sure the plan's workspace exists on the current device (first run of a plan
// made without a device).  Returns a gemm_status.
int ensure_workspace(gemm_plan_s *plan, hipStream_t s) {
  if (plan->d.ws_bytes == 0) return GEMM_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    set_error("gemm_run: no current HIP device");
    return GEMM_ERR_HIP;
  }
  if (plan->ws) {
    if (dev != plan->ws_dev) {
      set_error("gemm_run: the plan's split-K workspace lives on another device");
      return GEMM_ERR_UNSUPPORTED;
    }
    return GEMM_OK;
  }
  if (hipMalloc(&plan->ws, size_t(plan->d.ws_bytes)) != hipSuccess) {
    (void)hipGetLastError();
    plan->ws = nullptr;
    set_error("gemm_run: cannot allocate the split-K workspace");
    return GEMM_ERR_ALLOC;
  }
  plan->ws_dev = dev;
  if (mhg::launch_zero_words(plan->ws, counter_words(plan->d), s) != hipSuccess) {
    set_error("gemm_run: cannot clear the split-K workspace");
    return GEMM_ERR_HIP;
  }
  return GEMM_OK;
}

// Scratch memory of the allocation-free entry point (gemm_run_noalloc): the split-K
// workspaces its plans need, in a file-scope device array that each GPU holds from
// the library's load until the process ends.  Host code never passes the array's name
// to a kernel (on the host it is only a stand-in for the symbol): its address on each
// device is asked once, with that device current, and kept here.
constexpr int64_t kScratchBytes = int64_t(16) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, looked up on its first use.  Returns a gemm_status.
int scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    set_error("gemm_run_noalloc: no current HIP device");
    return GEMM_ERR_HIP;
  }
  if (dev >= kMaxDevices) {
    set_error("gemm_run_noalloc: device index beyond the 64 this library keeps scratch addresses for");
    return GEMM_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      set_error(std::string("gemm_run_noalloc: cannot find the scratch array on the device: ") +
                hipGetErrorString(e));
      return GEMM_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GEMM_OK;
}

// Enqueue a chosen plan.  The split-K workspace comes from `plan` (allocated on its
// first run when gemm_plan could not) or, with plan == NULL, from the device's scratch
// array, whose arrival counters are cleared first by a fill kernel.
int run_chosen(const mhg::PlanData &d, gemm_plan_s *plan, const void *A, const void *B, void *C,
               const gemm_epilogue_t *epi, hipStream_t s);

}  // namespace

namespace mhg {
void set_last_error(const std::string &msg) { set_error(msg); }
}  // namespace mhg

extern "C" {

gemm_plan_t gemm_plan(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                      int dtype, int layout) {
  return make_plan(M, N, K, lda, ldb, ldc, dtype, layout, nullptr);
}

gemm_plan_t gemm_plan_config(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                             int64_t ldc, int dtype, int layout, const int32_t cfg[8]) {
  if (!cfg) {
    set_error("gemm_plan_config: NULL configuration");
    return nullptr;
  }
  return make_plan(M, N, K, lda, ldb, ldc, dtype, layout, cfg);
}

int gemm_run(gemm_plan_t plan, const void *A, const void *B, void *C, void *stream) {
  return gemm_run_epilogue(plan, A, B, C, nullptr, stream);
}

}  // extern "C"

namespace {

int run_chosen(const mhg::PlanData &d, gemm_plan_s *plan, const void *A, const void *B, void *C,
               const gemm_epilogue_t *epi, hipStream_t s) {
  if (epi && epi->activation != GEMM_ACT_NONE && epi->activation != GEMM_ACT_RELU) {
    set_error("gemm_run_epilogue: unknown activation");
    return GEMM_ERR_INVALID_ARG;
  }
  if (epi && epi->bias && reinterpret_cast<uintptr_t>(epi->bias) % 4 != 0) {
    set_error("gemm_run_epilogue: bias must be 4-byte aligned fp32");
    return GEMM_ERR_INVALID_ARG;
  }
  if (d.M == 0 || d.N == 0) return GEMM_OK;
  if (!C) {
    set_error("gemm_run: NULL C");
    return GEMM_ERR_INVALID_ARG;
  }
  mhg::LaunchArgs a{};
  a.A = A;
  a.B = B;
  a.C = C;
  a.M = d.M; a.N = d.N; a.K = d.K;
  a.lda = d.lda; a.ldb = d.ldb; a.ldc = d.ldc;
  a.in_code = d.in_code;
  a.out_code = d.out_code;
  a.a_col = (d.layout & GEMM_A_COL) ? 1 : 0;
  a.b_col = (d.layout & GEMM_B_COL) ? 1 : 0;
  a.gm = d.gm;
  a.gn = d.gn;
  a.split_k = d.gz;
  a.group_m = d.group_m;
  // The identity epilogue is the plain product: the kernels then skip it entirely.
  a.alpha = 1.0f;
  a.beta = 0.0f;
  a.bias = nullptr;
  a.act = GEMM_ACT_NONE;
  if (epi) {
    a.alpha = epi->alpha;
    a.beta = epi->beta;
    a.bias = epi->bias;
    a.bias_vec = reinterpret_cast<uintptr_t>(epi->bias) % 16 == 0;
    a.act = epi->activation;
    a.epi = !(a.alpha == 1.0f && a.beta == 0.0f && !a.bias && a.act == GEMM_ACT_NONE);
  }
  hipError_t e;
  if (d.K == 0) {
    e = mhg::launch_fill(a, s);
  } else {
    if (!A || !B) {
      set_error("gemm_run: NULL A or B");
      return GEMM_ERR_INVALID_ARG;
    }
    const int elems16 = 16 / mhg::elem_bytes(d.in_code);
    a.vec_a = (reinterpret_cast<uintptr_t>(A) % 16 == 0) && (d.lda % elems16 == 0);
    a.vec_b = (reinterpret_cast<uintptr_t>(B) % 16 == 0) && (d.ldb % elems16 == 0);
    // four output elements per store: 16 bytes of fp32 or 8 bytes of fp16 / bf16
    const int out_bytes = mhg::elem_bytes(d.out_code);
    a.c_vec = (reinterpret_cast<uintptr_t>(C) % (4 * out_bytes) == 0) && (d.ldc % 4 == 0);
    int count;
    const mhg::Variant *cat = mhg::catalogue(&count);
    const mhg::Variant *v = &cat[d.variant];
    // Direct 16-byte staging: the plan checked extents, leading dimensions and slab
    // spans; what it cannot see is the alignment of the pointers.
    const bool direct_ok = a.vec_a && a.vec_b;
    if (v->fallback >= 0 && !direct_ok) {
      v = mhg::variant_of_launcher(v->fallback);   // register-staged: any alignment
      a.gm = int((d.M + v->cfg.bm - 1) / v->cfg.bm);
      a.gn = int((d.N + v->cfg.bn - 1) / v->cfg.bn);
      a.group_m = std::max(1, std::min(a.gm, 4));
      a.split_k = 1;
    }
    if (a.split_k > 1) {
      if (plan) {
        const int st = ensure_workspace(plan, s);
        if (st != GEMM_OK) return st;
        a.workspace = plan->ws;
      } else {
        if (d.ws_bytes > kScratchBytes) {
          set_error("gemm_run_noalloc: the plan's split-K workspace (" + std::to_string(d.ws_bytes) +
                    " bytes) exceeds the scratch array (" + std::to_string(kScratchBytes) + " bytes)");
          return GEMM_ERR_UNSUPPORTED;
        }
        const int st = scratch_of_current_device(&a.workspace);
        if (st != GEMM_OK) return st;
        // The skinny kernel's arrival counters must start at zero; the array keeps
        // whatever the previous call on this device left there.
        if (v->launcher == mhg::L_SKINNY && mhg::launch_zero_words(a.workspace, counter_words(d), s) != hipSuccess) {
          set_error("gemm_run_noalloc: cannot clear the arrival counters");
          return GEMM_ERR_HIP;
        }
      }
      a.ws_bytes = d.ws_bytes;
      // Eight-wave split-K: K per chunk, a whole number of slabs.
      const int64_t bk = v->cfg.bk, per = (d.K + a.split_k - 1) / a.split_k;
      a.k_chunk = (per + bk - 1) / bk * bk;
    }
    switch (v->launcher) {
      case mhg::L_FMA_32: case mhg::L_FMA_64: case mhg::L_FMA_128:
        e = mhg::launch_fma(v->launcher, a, s); break;
      case mhg::L_W8_256: case mhg::L_W8_128: case mhg::L_W8_64:
        e = mhg::launch_w8(a, v->cfg.bm, s); break;
      case mhg::L_SKINNY:
        e = mhg::launch_skinny(a, s); break;
      case mhg::L_MFMA32_128:
        e = mhg::launch_mfma32(a, s); break;
      default:
        e = mhg::launch_mfma(v->launcher, a, s); break;
    }
  }
  if (e != hipSuccess) {
    set_error(std::string("gemm_run: launch failed: ") + hipGetErrorString(e));
    return GEMM_ERR_HIP;
  }
  return GEMM_OK;
}

}  // namespace

extern "C" {

int gemm_run_epilogue(gemm_plan_t plan, const void *A, const void *B, void *C, const gemm_epilogue_t *epi,
                      void *stream) {
  if (!plan) {
    set_error("gemm_run: NULL plan");
    return GEMM_ERR_INVALID_ARG;
  }
  return run_chosen(plan->d, plan, A, B, C, epi, static_cast<hipStream_t>(stream));
}

int gemm_run_noalloc(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
                     int layout, const void *A, const void *B, void *C, const gemm_epilogue_t *epi, void *stream) {
  mhg::PlanData d;
  if (!choose_plan(M, N, K, lda, ldb, ldc, dtype, layout, nullptr, &d)) return GEMM_ERR_INVALID_ARG;
  return run_chosen(d, nullptr, A, B, C, epi, static_cast<hipStream_t>(stream));
}

void gemm_destroy(gemm_plan_t plan) {
  if (!plan) return;
  if (plan->ws) (void)hipFree(plan->ws);
  (void)hipGetLastError();
  delete plan;
}

const char *gemm_last_error(void) { return g_last_error.c_str(); }

int gemm_transpose(const void *in, void *out, int64_t rows, int64_t cols, int64_t ld_in, int64_t ld_out,
                   int32_t elem_bytes, void *stream) {
  if (rows < 0 || cols < 0) {
    set_error("gemm_transpose: negative extent");
    return GEMM_ERR_INVALID_ARG;
  }
  if (elem_bytes != 2 && elem_bytes != 4) {
    set_error("gemm_transpose: elem_bytes must be 2 or 4");
    return GEMM_ERR_INVALID_ARG;
  }
  if (rows == 0 || cols == 0) {
    set_error("");
    return GEMM_OK;
  }
  if (ld_in < cols || ld_out < rows) {
    set_error("gemm_transpose: ld_in must be >= cols and ld_out >= rows");
    return GEMM_ERR_INVALID_ARG;
  }
  if (rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31)) {
    set_error("gemm_transpose: extents above 2^31 are not supported");
    return GEMM_ERR_INVALID_ARG;
  }
  if (!in || !out || reinterpret_cast<uintptr_t>(in) % elem_bytes || reinterpret_cast<uintptr_t>(out) % elem_bytes) {
    set_error("gemm_transpose: NULL or misaligned (not element-aligned) pointer");
    return GEMM_ERR_INVALID_ARG;
  }
  const hipError_t e = mhg::launch_transpose(in, out, rows, cols, ld_in, ld_out, elem_bytes,
                                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_error(std::string("gemm_transpose: launch failed: ") + hipGetErrorString(e));
    return GEMM_ERR_HIP;
  }
  set_error("");
  return GEMM_OK;
}

int gemm_clock_probe(uint64_t *out, int64_t ticks, void *stream) {
  if (!out || reinterpret_cast<uintptr_t>(out) % 8 != 0) {
    set_error("gemm_clock_probe: NULL or misaligned output");
    return GEMM_ERR_INVALID_ARG;
  }
  if (ticks < 1 || ticks > 1000000000) {
    set_error("gemm_clock_probe: ticks must lie in [1, 1e9]");
    return GEMM_ERR_INVALID_ARG;
  }
  const hipError_t e = mhg::launch_clock_probe(out, uint64_t(ticks), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_error(std::string("gemm_clock_probe: launch failed: ") + hipGetErrorString(e));
    return GEMM_ERR_HIP;
  }
  set_error("");
  return GEMM_OK;
}

int gemm_plan_describe(gemm_plan_t plan, int32_t out[16]) {
  if (!plan || !out) {
    set_error("gemm_plan_describe: NULL argument");
    return GEMM_ERR_INVALID_ARG;
  }
  const mhg::PlanData &d = plan->d;
  const int32_t v[16] = {d.cfg.kind, d.cfg.bm, d.cfg.bn, d.cfg.bk, d.cfg.waves_m, d.cfg.waves_n,
                         d.cfg.stages, d.cfg.split_k, d.gm, d.gn, d.gz, d.threads, d.lds_bytes,
                         d.cus, d.variant, int32_t(d.ws_bytes)};
  std::memcpy(out, v, sizeof v);
  return GEMM_OK;
}

}  // extern "C"

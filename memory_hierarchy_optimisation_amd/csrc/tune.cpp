// tune.cpp -- autotuning of the tile configuration and the table of tuned choices.
//
// "Tiling 策略与内存层次优化" (autotuning section) finds the best tile size in four
// steps: enumerate the feasible tile configurations, drop those that break the
// hardware limits, benchmark every candidate on the target, keep the fastest.  Here
// the enumeration is the catalogue of compiled variants, the filter is the planner's
// feasibility test (gemm_plan_config refuses a variant whose LDS, alignment or
// operand-type needs the problem does not meet), and the benchmark times each
// candidate's own gemm_run calls with HIP events on the caller's stream, on the
// caller's operands.  The winner goes into a process-wide table keyed by the whole
// problem description; gemm_plan consults that table before its heuristic score, so
// the per-shape choices of "GPU Kernel 的 Tile、Grid、Wave 与 Launch Overhead"
// (different tiles for different shapes) come from measurement rather than from the
// model.  The table can be written to and read from a text file.
#include <hip/hip_runtime_api.h>

#include <cerrno>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/mhgemm.h"
#include "plan.h"

namespace mhg {

void set_last_error(const std::string &msg);   // capi.hip

namespace {

struct Key {
  int64_t M, N, K, lda, ldb, ldc;
  int dtype, layout;
  bool operator<(const Key &o) const {
    return std::tie(M, N, K, lda, ldb, ldc, dtype, layout) <
           std::tie(o.M, o.N, o.K, o.lda, o.ldb, o.ldc, o.dtype, o.layout);
  }
};

struct Entry {
  int32_t cfg[8];
  float us;
};

std::mutex g_mu;
std::map<Key, Entry> g_table;

void cfg_of(const TileConfig &c, int32_t out[8]) {
  const int32_t v[8] = {c.kind, c.bm, c.bn, c.bk, c.waves_m, c.waves_n, c.stages, c.split_k};
  std::memcpy(out, v, sizeof v);
}

bool in_catalogue(const int32_t cfg[8]) {
  int n;
  const Variant *cat = catalogue(&n);
  for (int i = 0; i < n; ++i) {
    int32_t c[8];
    cfg_of(cat[i].cfg, c);
    if (std::memcmp(c, cfg, sizeof c) == 0) return true;
  }
  return false;
}

// Mean time per call of `reps` back-to-back runs of one plan, in microseconds; the
// better of two batches.  Returns < 0 (message set) when a run or an event fails.
float time_plan(gemm_plan_t plan, const void *A, const void *B, void *C, hipStream_t s, int reps) {
  for (int i = 0; i < 2; ++i)
    if (gemm_run(plan, A, B, C, s) != GEMM_OK) return -1.0f;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    (void)hipGetLastError();
    set_last_error("gemm_autotune: cannot create HIP events");
    return -1.0f;
  }
  float best = -1.0f;
  for (int batch = 0; batch < 2 && best != -2.0f; ++batch) {
    if (hipEventRecord(e0, s) != hipSuccess) { best = -2.0f; break; }
    for (int i = 0; i < reps; ++i)
      if (gemm_run(plan, A, B, C, s) != GEMM_OK) { best = -2.0f; break; }
    if (best == -2.0f) break;
    float ms = 0.0f;
    if (hipEventRecord(e1, s) != hipSuccess || hipEventSynchronize(e1) != hipSuccess ||
        hipEventElapsedTime(&ms, e0, e1) != hipSuccess) {
      set_last_error("gemm_autotune: timing with HIP events failed");
      best = -2.0f;
      break;
    }
    const float us = ms * 1000.0f / float(reps);
    if (best < 0.0f || us < best) best = us;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  (void)hipGetLastError();
  return best < 0.0f ? -1.0f : best;
}

}  // namespace

bool tuned_lookup(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
                  int layout, int32_t cfg[8]) {
  std::lock_guard<std::mutex> lock(g_mu);
  const auto it = g_table.find(Key{M, N, K, lda, ldb, ldc, dtype, layout});
  if (it == g_table.end()) return false;
  std::memcpy(cfg, it->second.cfg, sizeof it->second.cfg);
  return true;
}

}  // namespace mhg

extern "C" {

int gemm_catalogue(int32_t *cfgs, int32_t max_cfgs) {
  int n;
  const mhg::Variant *cat = mhg::catalogue(&n);
  if (cfgs)
    for (int i = 0; i < n && i < max_cfgs; ++i) mhg::cfg_of(cat[i].cfg, cfgs + 8 * i);
  return n;
}

int gemm_catalogue_registers(int32_t *regs, int32_t max_regs) {
  int n;
  const mhg::Variant *cat = mhg::catalogue(&n);
  if (regs)
    for (int i = 0; i < n && i < max_regs; ++i) regs[i] = mhg::registers_of(cat[i]);
  return n;
}

int gemm_autotune(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dtype,
                  int layout, const void *A, const void *B, void *C, void *stream, int32_t reps,
                  int32_t best_cfg[8], float *best_us, float *times_us, int32_t n_times) {
  mhg::PlanData d;
  std::string err;
  if (!mhg::validate(M, N, K, lda, ldb, ldc, dtype, layout, &d, &err)) {
    mhg::set_last_error("gemm_autotune: " + err);
    return GEMM_ERR_INVALID_ARG;
  }
  if (M == 0 || N == 0 || K == 0) {
    mhg::set_last_error("gemm_autotune: an empty product has no tile configuration to tune");
    return GEMM_ERR_INVALID_ARG;
  }
  if (!A || !B || !C || reps < 1 || reps > 100000 || (n_times > 0 && !times_us)) {
    mhg::set_last_error("gemm_autotune: NULL operand, reps outside [1, 100000] or NULL times_us");
    return GEMM_ERR_INVALID_ARG;
  }
  int n;
  const mhg::Variant *cat = mhg::catalogue(&n);
  for (int i = 0; i < n_times; ++i) times_us[i] = -1.0f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int best = -1;
  float best_time = 0.0f;
  for (int i = 0; i < n; ++i) {
    int32_t cfg[8];
    mhg::cfg_of(cat[i].cfg, cfg);
    gemm_plan_t plan = gemm_plan_config(M, N, K, lda, ldb, ldc, dtype, layout, cfg);
    if (!plan) continue;   // filtered out: this variant does not fit the problem
    int32_t desc[16];
    gemm_plan_describe(plan, desc);
    // A configuration listed twice maps to its first catalogue entry; time it once.
    if (desc[14] != i) {
      gemm_destroy(plan);
      continue;
    }
    const float us = mhg::time_plan(plan, A, B, C, s, reps);
    gemm_destroy(plan);
    if (us < 0.0f) {
      std::string msg = gemm_last_error();
      mhg::set_last_error("gemm_autotune: candidate " + std::to_string(i) + " failed: " + msg);
      return GEMM_ERR_HIP;
    }
    if (i < n_times) times_us[i] = us;
    if (best < 0 || us < best_time) {
      best = i;
      best_time = us;
    }
  }
  if (best < 0) {
    mhg::set_last_error("gemm_autotune: no compiled variant fits this problem");
    return GEMM_ERR_UNSUPPORTED;
  }
  mhg::Entry e;
  mhg::cfg_of(cat[best].cfg, e.cfg);
  e.us = best_time;
  {
    std::lock_guard<std::mutex> lock(mhg::g_mu);
    mhg::g_table[mhg::Key{M, N, K, lda, ldb, ldc, dtype, layout}] = e;
  }
  if (best_cfg) std::memcpy(best_cfg, e.cfg, sizeof e.cfg);
  if (best_us) *best_us = best_time;
  mhg::set_last_error("");
  return GEMM_OK;
}

int gemm_tune_save(const char *path) {
  if (!path) {
    mhg::set_last_error("gemm_tune_save: NULL path");
    return GEMM_ERR_INVALID_ARG;
  }
  std::vector<std::pair<mhg::Key, mhg::Entry>> rows;
  {
    std::lock_guard<std::mutex> lock(mhg::g_mu);
    rows.assign(mhg::g_table.begin(), mhg::g_table.end());
  }
  FILE *f = std::fopen(path, "w");
  if (!f) {
    mhg::set_last_error(std::string("gemm_tune_save: cannot open ") + path + ": " + std::strerror(errno));
    return GEMM_ERR_INVALID_ARG;
  }
  std::fprintf(f, "# mhgemm tuned configurations v1\n"
                  "# M N K lda ldb ldc dtype layout | kind BM BN BK waves_m waves_n stages split_k | us\n");
  for (const auto &r : rows) {
    const mhg::Key &k = r.first;
    const int32_t *c = r.second.cfg;
    std::fprintf(f, "%lld %lld %lld %lld %lld %lld %d %d | %d %d %d %d %d %d %d %d | %.3f\n",
                 (long long)k.M, (long long)k.N, (long long)k.K, (long long)k.lda, (long long)k.ldb,
                 (long long)k.ldc, k.dtype, k.layout, c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7],
                 double(r.second.us));
  }
  const bool ok = std::fclose(f) == 0;
  if (!ok) {
    mhg::set_last_error(std::string("gemm_tune_save: write failed: ") + path);
    return GEMM_ERR_INVALID_ARG;
  }
  mhg::set_last_error("");
  return int(rows.size());
}

int gemm_tune_load(const char *path) {
  if (!path) {
    mhg::set_last_error("gemm_tune_load: NULL path");
    return GEMM_ERR_INVALID_ARG;
  }
  FILE *f = std::fopen(path, "r");
  if (!f) {
    mhg::set_last_error(std::string("gemm_tune_load: cannot open ") + path + ": " + std::strerror(errno));
    return GEMM_ERR_INVALID_ARG;
  }
  std::map<mhg::Key, mhg::Entry> parsed;
  char line[512];
  int lineno = 0;
  std::string bad;
  while (std::fgets(line, sizeof line, f)) {
    ++lineno;
    if (!std::strchr(line, '\n') && !std::feof(f)) {
      bad = "line too long";
      break;
    }
    const char *p = line;
    while (*p == ' ' || *p == '\t') ++p;
    if (*p == '#' || *p == '\n' || *p == '\r' || *p == '\0') continue;
    long long m, nn, k, lda, ldb, ldc;
    int dtype, layout;
    int32_t c[8];
    float us;
    char tail;
    const int got = std::sscanf(p, "%lld %lld %lld %lld %lld %lld %d %d | %d %d %d %d %d %d %d %d | %f %c",
                                &m, &nn, &k, &lda, &ldb, &ldc, &dtype, &layout, &c[0], &c[1], &c[2], &c[3],
                                &c[4], &c[5], &c[6], &c[7], &us, &tail);
    if (got != 17) {
      bad = "expected 8 problem fields, 8 configuration fields and a time";
      break;
    }
    mhg::PlanData d;
    std::string err;
    if (!mhg::validate(m, nn, k, lda, ldb, ldc, dtype, layout, &d, &err) || m == 0 || nn == 0 || k == 0) {
      bad = err.empty() ? std::string("empty product") : err;
      break;
    }
    if (!mhg::in_catalogue(c)) {
      bad = "configuration is not a compiled variant";
      break;
    }
    mhg::Entry e;
    std::memcpy(e.cfg, c, sizeof c);
    e.us = us;
    parsed[mhg::Key{m, nn, k, lda, ldb, ldc, dtype, layout}] = e;
  }
  std::fclose(f);
  if (!bad.empty()) {
    mhg::set_last_error(std::string("gemm_tune_load: ") + path + ", line " + std::to_string(lineno) + ": " + bad);
    return GEMM_ERR_INVALID_ARG;
  }
  {
    std::lock_guard<std::mutex> lock(mhg::g_mu);
    for (const auto &r : parsed) mhg::g_table[r.first] = r.second;
  }
  mhg::set_last_error("");
  return int(parsed.size());
}

void gemm_tune_clear(void) {
  std::lock_guard<std::mutex> lock(mhg::g_mu);
  mhg::g_table.clear();
}

}  // extern "C"

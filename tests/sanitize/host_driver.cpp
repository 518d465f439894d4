// Sanitizer run of the library's host code (tests/test_sanitizers.py builds capi.hip,
// plan.cpp and tune.cpp with ASan and UBSan on the host side, against launcher stubs,
// and runs this on the CPU): planning over a grid of shapes, types and layouts with
// valid and invalid arguments, every catalogue configuration forced, plan
// descriptions, the tuned-table text format (valid, malformed and oversized lines),
// and the argument checks of the run calls.  Prints "host sanitizer run ok" at the end.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "mhgemm.h"

static int g_plans = 0;

static void plan_and_describe(int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, int dt,
                              int lay) {
  gemm_plan_t p = gemm_plan(M, N, K, lda, ldb, ldc, dt, lay);
  int32_t d[16];
  if (p) {
    gemm_plan_describe(p, d);
    ++g_plans;
    // argument checks of the run calls: NULL operands, bad epilogue (no launch happens)
    gemm_run(p, nullptr, nullptr, nullptr, nullptr);
    gemm_epilogue_t e{1.0f, 0.0f, reinterpret_cast<const float *>(2), 0};
    gemm_run_epilogue(p, nullptr, nullptr, reinterpret_cast<void *>(256), &e, nullptr);
    e.activation = 7;
    gemm_run_epilogue(p, nullptr, nullptr, reinterpret_cast<void *>(256), &e, nullptr);
    gemm_destroy(p);
  }
  (void)strlen(gemm_last_error());
}

int main(int argc, char **argv) {
  const char *dir = argc > 1 ? argv[1] : ".";
  const int64_t ext[] = {0, 1, 7, 8, 16, 17, 64, 100, 256, 1000, 4096};
  for (int dt = -1; dt <= 5; ++dt)
    for (int lay = -1; lay <= 4; ++lay)
      for (int64_t M : ext)
        for (int64_t N : ext)
          for (int64_t K : {int64_t(0), int64_t(8), int64_t(1000), int64_t(8192)}) {
            const int64_t lda = (lay & 1) ? M : K, ldb = (lay & 2) ? K : N;
            plan_and_describe(M, N, K, lda, ldb, N, dt, lay);
            plan_and_describe(M, N, K, lda + 8, ldb + 8, N + 8, dt, lay);
            plan_and_describe(M, N, K, lda - 1, ldb, N, dt, lay);
          }
  plan_and_describe(int64_t(1) << 31, 16, 16, 16, 16, 16, 0, 0);
  plan_and_describe(16, 16, -1, 16, 16, 16, 0, 0);
  plan_and_describe(16, 8192, int64_t(1) << 30, int64_t(1) << 30, 8192, 8192, GEMM_BF16_F32, 0);
  // every compiled configuration forced on a few shapes
  const int n = gemm_catalogue(nullptr, 0);
  std::vector<int32_t> cfgs(8 * size_t(n));
  std::vector<int32_t> regs(static_cast<size_t>(n));
  gemm_catalogue(cfgs.data(), n);
  gemm_catalogue_registers(regs.data(), n);
  for (int i = 0; i < n; ++i)
    for (int64_t s : {int64_t(1), int64_t(16), int64_t(300), int64_t(304), int64_t(4096)})
      for (int dt = 0; dt < 5; ++dt)
        for (int lay = 0; lay < 4; ++lay) {
          gemm_plan_t p = gemm_plan_config(s, s, s, s, s, s, dt, lay, &cfgs[8 * size_t(i)]);
          if (p) {
            int32_t d[16];
            gemm_plan_describe(p, d);
            gemm_destroy(p);
            ++g_plans;
          }
        }
  gemm_plan_config(64, 64, 64, 64, 64, 64, 0, 0, nullptr);
  // the tuned table: a valid file, then malformed ones
  const std::string path = std::string(dir) + "/tune.txt";
  const char *files[] = {
      "# comment\n64 64 64 64 64 64 0 0 | 1 32 32 32 4 1 2 1 | 3.5\n"
      "4096 4096 4096 4096 4096 4096 3 0 | 2 256 256 32 2 4 5 1 | 100\n",
      "64 64 64 64 64 64 0 0 | 1 32 32 32 4 1 2\n",
      "64 64 64 64 64 64 0 0 | 9 9 9 9 9 9 9 9 | 1\n",
      "-1 64 64 64 64 64 0 0 | 1 32 32 32 4 1 2 1 | 1\n",
      "garbage\n",
      "",
  };
  for (const char *text : files) {
    FILE *f = std::fopen(path.c_str(), "w");
    std::fputs(text, f);
    std::fclose(f);
    gemm_tune_load(path.c_str());
    (void)strlen(gemm_last_error());
  }
  {
    std::string big(100000, '7');
    FILE *f = std::fopen(path.c_str(), "w");
    std::fputs(big.c_str(), f);
    std::fclose(f);
    gemm_tune_load(path.c_str());
  }
  gemm_tune_load((std::string(dir) + "/does_not_exist.txt").c_str());
  gemm_tune_save(path.c_str());
  gemm_tune_load(path.c_str());
  plan_and_describe(4096, 4096, 4096, 4096, 4096, 4096, 3, 0);
  gemm_tune_clear();
  // argument checks that need no device
  gemm_run(nullptr, nullptr, nullptr, nullptr, nullptr);
  gemm_plan_describe(nullptr, nullptr);
  gemm_transpose(nullptr, nullptr, -1, 4, 4, 4, 4, nullptr);
  gemm_transpose(nullptr, nullptr, 4, 4, 4, 4, 3, nullptr);
  gemm_transpose(nullptr, nullptr, 4, 4, 3, 4, 4, nullptr);
  gemm_transpose(nullptr, nullptr, 0, 4, 4, 4, 4, nullptr);
  gemm_clock_probe(nullptr, 10, nullptr);
  gemm_clock_probe(reinterpret_cast<uint64_t *>(16), 0, nullptr);
  gemm_run_noalloc(-1, 4, 4, 4, 4, 4, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr);
  gemm_run_noalloc(0, 4, 4, 4, 4, 4, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr);
  std::printf("host sanitizer run ok (%d plans)\n", g_plans);
  return 0;
}

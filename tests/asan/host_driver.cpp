// Exercises every host-only entry point of the library (argument checks of every region entry
// point, the path decision, both pipeline schedules, the threshold search, tuning tables, CU
// splits and files) on many inputs,
// including invalid ones.  Built together with the host source under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_asan.py; a sanitizer report fails the test.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "../../include/proj_add_rmsnorm.h"

namespace pr {
// The device query lives in the runtime (not built here): a fixed key stands in for it.
int current_device_key(std::string* key) {
  *key = "host-driver:1";
  return PR_OK;
}
}  // namespace pr

int main(int argc, char** argv) {
  const char* tune_path = argc > 1 ? argv[1] : "host_driver_tuning.txt";
  std::vector<char> arena(1 << 16);
  char* a = arena.data();
  char* b = a + 4096;
  char* c = a + 8192;
  char* d = a + 12288;
  char* e = a + 16384;
  long checks = 0;
  const int Ts[] = {-1, 0, 1, 17, 64, 1000, 4096, 5000, 32768};
  const int Ks[] = {-64, 0, 63, 64, 512, 4096, 16384};
  const int Hs[] = {0, 64, 320, 512, 3072, 4096, 8192};
  const int mcs[] = {-3, -2, -1, 0, 1, 16, 512, 4096, 4097};
  for (int T : Ts)
    for (int K : Ks)
      for (int H : Hs)
        for (int mc : mcs) {
          pr_decision dec;
          checks += pr_select(T, K, H, mc, &dec) == PR_OK;
          for (int kind = -1; kind <= 2; ++kind)
            checks += pr_validate(a, b, c, d, 1e-5f, T, K, H, mc, kind, e) == PR_OK;
          checks += pr_validate(nullptr, b, c, d, 1e-5f, T, K, H, mc, 0, e) == PR_OK;
          checks += pr_validate(a, b, c, d, -1.0f, T, K, H, mc, 0, nullptr) == PR_OK;
          checks += pr_validate(a + 1, b, c, d, 1e-5f, T, K, H, mc, 0, e) == PR_OK;  // misaligned
          checks += pr_validate(a, b, a, d, 1e-5f, T, K, H, mc, 0, e) == PR_OK;      // aliasing
        }
  // The fused-SiluAndMul and FP8 argument checks (gate_up: 4 bytes per element of x; FP8:
  // byte operands and two scale pointers, including misaligned and overlapping ones).
  char* f = a + 20480;
  char* g = a + 24576;
  for (int T : Ts)
    for (int K : Ks)
      for (int H : Hs) {
        for (int kind = -1; kind <= 2; ++kind)
          checks += pr_validate_silu(a, b, c, d, 1e-5f, T, K, H, kind, e) == PR_OK;
        checks += pr_validate_silu(a, b, a + 16, d, 1e-5f, T, K, H, 0, e) == PR_OK;
        for (int sr : {-1, 0, 1, 7, 256, 1 << 30}) {
          checks += pr_validate_fp8(a, f, sr, b, g, c, d, 1e-5f, T, K, H, 0, e) == PR_OK;
          checks += pr_validate_fp8(a, f + 2, sr, b, g, c, d, 1e-5f, T, K, H, 0, e) == PR_OK;
          checks += pr_validate_fp8(a, nullptr, sr, b, g, c, d, 1e-5f, T, K, H, 1, e) == PR_OK;
          checks += pr_validate_fp8(a, c, sr, b, c + 8, c, d, 1e-5f, T, K, H, 0, e) == PR_OK;
        }
      }
  for (int T : Ts)
    for (int mc : mcs) {
      const int n = pr_plan_cu_split(T, mc, nullptr, 0);
      if (n < 0) continue;
      std::vector<pr_plan_op> ops(n > 0 ? n : 1);
      checks += pr_plan_cu_split(T, mc, ops.data(), n) == n;
      if (n > 2) checks += pr_plan_cu_split(T, mc, ops.data(), n / 2) >= 0;
    }
  for (int n : {-8, 0, 7, 8, 32, 64, 128, 136, 1 << 30})
    for (int mc : mcs) checks += pr_set_cu_split(4096, 4096, mc, n) == PR_OK;
  pr_clear_tuning();
  for (int T : Ts)
    for (int mc : mcs) {
      const int n = pr_plan(T, mc, nullptr, 0);
      if (n < 0) continue;
      std::vector<pr_plan_op> ops(n > 0 ? n : 1);
      checks += pr_plan(T, mc, ops.data(), n) == n;
      if (n > 2) checks += pr_plan(T, mc, ops.data(), n / 2) >= 0;  // truncated output
    }
  {
    const int grid[] = {128, 512, 2048, 8192, 32768};
    std::vector<double> conv(2 * 5), fused(2 * 5), spread(2 * 5);
    for (int i = 0; i < 10; ++i) {
      conv[i] = 1e-4 * (1 + i % 5);
      fused[i] = (i % 3 == 0) ? -1.0 : 0.9e-4 * (1 + i % 5);
      spread[i] = 1e-6 * i;
    }
    int thr = 0;
    checks += pr_threshold_from_timings(2, 5, grid, conv.data(), fused.data(), spread.data(),
                                        &thr) == PR_OK;
    checks += pr_threshold_from_timings(2, 5, grid, conv.data(), fused.data(), nullptr, &thr) ==
              PR_OK;
    checks += pr_threshold_from_timings(0, 5, grid, conv.data(), fused.data(), nullptr, &thr) ==
              PR_OK;
    checks += pr_threshold_from_timings(2, 5, nullptr, conv.data(), fused.data(), nullptr, &thr) ==
              PR_OK;
  }
  {
    const int grid[] = {128, 1024, 4096};
    const int mc[] = {128, 512, PR_SINGLE_LAUNCH};
    const int bad_mc[] = {128, 0, 9999};
    checks += pr_set_tuning(4096, 4096, 1024, 8192, grid, mc, 3) == PR_OK;
    checks += pr_set_tuning(4096, 4096, 1024, 8192, grid, bad_mc, 3) == PR_OK;
    checks += pr_set_tuning(4096, 4096, 1024, 8192, nullptr, mc, 3) == PR_OK;
    checks += pr_set_chunk_config(4096, 4096, 512, 128, 128, 2, 8) == PR_OK;
    checks += pr_set_chunk_config(4096, 4096, 512, 100, 128, 2, 8) == PR_OK;
    checks += pr_set_chunk_config(4096, 4096, 512, 128, 128, 3, 8) == PR_OK;
    for (int T : Ts) {
      pr_decision dec;
      checks += pr_select(T, 4096, 4096, 0, &dec) == PR_OK;
    }
    checks += pr_tuning_save(tune_path, nullptr) == PR_OK;
    pr_clear_tuning();
    checks += pr_tuning_load(tune_path, nullptr) == PR_OK;
    checks += pr_tuning_load(tune_path, "other:2") == PR_OK;
    checks += pr_tuning_save(tune_path, "with space") == PR_OK;
    checks += pr_tuning_load("/nonexistent/dir/file", "k") == PR_OK;
    FILE* f = std::fopen(tune_path, "w");
    if (f != nullptr) {
      std::fputs("pr_tuning 1 1 host-driver:1\ntuning 1 2 3\nchunk 99999999999 1 2 3 4 5 6\n"
                 "tuning 64 64 1 1 1000000 1 1\n \n\n", f);
      std::fclose(f);
    }
    checks += pr_tuning_load(tune_path, nullptr) == PR_OK;
    pr_clear_tuning();
  }
  for (int code = 1; code >= -8; --code) checks += pr_strerror(code) != nullptr;
  checks += pr_last_error() != nullptr;
  std::printf("host driver: %ld calls succeeded\n", checks);
  return 0;
}

// Kernel-choice log. With FP8BQ_LOG=1 in the environment, every distinct
// (entry point, M, N, K) -> kernel decision is printed once to stderr, e.g.
//   fp8bq: gemm M=3 N=17408 K=5120 -> gemm_rows_kernel MT=16 act=codes TILES=5 GMAX=5 rows/wg=68 grid=256
// so that a run shows which instance each shape took (there is no lookup
// by nearest size: the instance follows from M's range and from N and K).
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <set>
#include <string>
#include <tuple>

#include "launch.h"

namespace fp8bq {

namespace {

bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("FP8BQ_LOG");
    return v != nullptr && v[0] != '\0' && v[0] != '0';
  }();
  return on;
}

}  // namespace

void dispatch_log(const char* entry, int64_t m, int64_t n, int64_t k, const char* kernel) {
  if (!log_enabled()) return;
  static std::mutex mu;
  static std::set<std::tuple<std::string, int64_t, int64_t, int64_t>> seen;
  std::lock_guard<std::mutex> lock(mu);
  if (!seen.emplace(entry, m, n, k).second) return;
  std::fprintf(stderr, "fp8bq: %s M=%lld N=%lld K=%lld -> %s\n", entry, static_cast<long long>(m),
               static_cast<long long>(n), static_cast<long long>(k), kernel);
}

}  // namespace fp8bq

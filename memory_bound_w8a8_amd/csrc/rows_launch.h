// Launch plumbing shared by the translation units that instantiate the
// row-range streaming kernel (gemm.hip: W8A8 and W8A16 entry points;
// gemm_fused.hip: quantisation fused into the GEMM).
#pragma once

#include <array>
#include <utility>

#include "device_common.h"
#include "gemm_rows.h"

namespace fp8bq {

namespace {

constexpr int kNumCUs = 256;   // MI355X
constexpr int kRowsWaves = 8;  // waves per workgroup in the row-range kernel
constexpr int kMaxTiles = 5;
constexpr int kMaxGroupsPerWave = 9;

struct GemmArgs {
  int64_t m, n, k;
  const void* aq;
  const float* as;
  const void* wq;
  const float* ws;
  void* c;
  hipStream_t stream;
};

using Launch = hipError_t (*)(const GemmArgs&, int64_t rows_per_wg);

// Row-range launch shape for (N, K): rows per workgroup, tiles, groups
// per wave. Returns false when the shape is outside the compiled table.
inline bool rows_shape(int64_t n, int64_t k, int64_t* rows_per_wg, int* tiles, int* gmax) {
  const int64_t groups = k / kGroup;
  const int64_t g = (groups + kRowsWaves - 1) / kRowsWaves;
  if (g < 1 || g > kMaxGroupsPerWave) return false;
  // Rows per workgroup: N spread over one round of kNumCUs workgroups, or,
  // when that would exceed the largest tile count, over the fewest whole
  // rounds that fit (e.g. a vocabulary projection of 152064 rows: 8 rounds
  // of 76 rows instead of 7.4 rounds of 80, whose last round would leave
  // most CUs idle).
  const int64_t max_rows = 16 * kMaxTiles;
  const int64_t rounds = (n + kNumCUs * max_rows - 1) / (kNumCUs * max_rows);
  int64_t r = (n + kNumCUs * rounds - 1) / (kNumCUs * rounds);
  r = (r + 3) / 4 * 4;
  if (r > max_rows) r = max_rows;
  *rows_per_wg = r;
  *tiles = static_cast<int>((r + 15) / 16);
  *gmax = static_cast<int>(g);
  return true;
}


template <int MT, int AF, int TILES, int GMAX, int TOK = 16>
hipError_t rows_instance(const GemmArgs& a, int64_t rows_per_wg) {
  // chunks of weight loads kept in flight per wave (fewer where the held
  // activation of a 32-token tile, or the bf16 activation awaiting
  // quantisation, already takes most registers; and at 8..9 groups per wave
  // with the activation codes held for every group: on (5120, 8704) at
  // M = 1..8, 2 in flight measured 2-4% faster than 6, 1, 3 or 4)
  constexpr int PD = AF == kActBf16 ? (GMAX >= 8 ? 2 : (GMAX >= 7 ? 4 : 6))
                                    : (MT == 16 ? (AF == kActCodes && GMAX >= 8 ? 2 : 6) : 4);
  const unsigned grid = static_cast<unsigned>((a.n + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL((gemm_rows_kernel<MT, kRowsWaves, GMAX, TILES, PD, AF, TOK>), dim3(grid), dim3(64 * kRowsWaves),
                     0, a.stream, static_cast<int>(a.m), a.n, a.k, rows_per_wg,
                     static_cast<const unsigned char*>(a.aq), a.as, static_cast<const unsigned char*>(a.wq), a.ws,
                     static_cast<unsigned short*>(a.c));
  return hipGetLastError();
}

}  // namespace

}  // namespace fp8bq

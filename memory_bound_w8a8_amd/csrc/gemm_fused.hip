// Instances and launcher of the activation quantisation fused into the
// streaming block-FP8 GEMM (fp8bq_gemm_fused; page 1, SmartX blog,
// "single-stream optimisation": the W8A8 backend's per-call activation
// quantisation).
//
// The launch shape follows from (N, K) as for fp8bq_gemm (rows_shape). M
// selects the quantisation layout: 1, 2, 3..4 and 5..8 tokens spread each
// group's values over the whole wave (TOK = 1, 2, 4, 8: 64 / TOK lanes per
// token, 2 TOK values per lane) and exchange the codes through LDS. Every M
// inside a class runs the same instruction stream. Up to 8 tokens only:
// every workgroup quantises the whole activation (there is no memory shared
// between workgroups to quantise it once), and at 9..16 tokens that work no
// longer hides under the weight stream of the narrower logged weights
// (N = 5120 .. 8192), where quantisation + GEMM as two launches measured
// faster.
#include <array>
#include <string>
#include <utility>

#include "launch.h"
#include "rows_launch.h"

namespace fp8bq {

namespace {

template <int TOK, int TILES, int... G>
constexpr std::array<Launch, sizeof...(G)> fused_row(std::integer_sequence<int, G...>) {
  return {&rows_instance<16, kActBf16, TILES, G + 1, TOK>...};
}

template <int TOK, int... T>
constexpr std::array<std::array<Launch, kMaxGroupsPerWave>, sizeof...(T)> fused_table(std::integer_sequence<int, T...>) {
  return {fused_row<TOK, T + 1>(std::make_integer_sequence<int, kMaxGroupsPerWave>{})...};
}

constexpr auto kFused1 = fused_table<1>(std::make_integer_sequence<int, kMaxTiles>{});
constexpr auto kFused2 = fused_table<2>(std::make_integer_sequence<int, kMaxTiles>{});
constexpr auto kFused4 = fused_table<4>(std::make_integer_sequence<int, kMaxTiles>{});
constexpr auto kFused8 = fused_table<8>(std::make_integer_sequence<int, kMaxTiles>{});

}  // namespace

hipError_t launch_gemm_fused(int64_t m, int64_t n, int64_t k, const void* a, const void* wq, const float* ws, void* c,
                             hipStream_t stream) {
  const GemmArgs args{m, n, k, a, nullptr, wq, ws, c, stream};
  int64_t rows_per_wg;
  int tiles, gmax;
  if (m < 1 || m > 8 || !rows_shape(n, k, &rows_per_wg, &tiles, &gmax)) return hipErrorInvalidValue;
  const auto& table = m == 1 ? kFused1 : m == 2 ? kFused2 : m <= 4 ? kFused4 : kFused8;
  const int tok = m == 1 ? 1 : m == 2 ? 2 : m <= 4 ? 4 : 8;
  dispatch_log("gemm_fused", m, n, k,
               ("gemm_rows_kernel MT=16 act=bf16 TOK=" + std::to_string(tok) + " TILES=" + std::to_string(tiles) +
                " GMAX=" + std::to_string(gmax) + " rows/wg=" + std::to_string(rows_per_wg) +
                " grid=" + std::to_string((n + rows_per_wg - 1) / rows_per_wg))
                   .c_str());
  return table[tiles - 1][gmax - 1](args, rows_per_wg);
}

}  // namespace fp8bq

// Kernel instances and launch configuration of the block-FP8 GEMM.
//
// Streaming path (M <= 64, and 65..80 where the registers allow: at most 2
// row tiles per workgroup and 5 groups per wave). The launch shape follows
// from (N, K) alone:
//   rows per workgroup R = N / 256 rounded up to a multiple of 4 (one
//   workgroup per CU; at most 16 * kMaxTiles rows, beyond that more
//   workgroups), TILES = ceil(R / 16), and with S = 8 waves splitting the
//   K / 128 groups, GMAX = ceil(groups / 8).
// M only selects a token class (1..8, 9..16, 17..32, 33..48, 49..64, 65..80;
// see rows_entry), so every M inside a class runs the same instruction
// stream. Each (TILES, GMAX)
// pair has its own compiled instance, looked up exactly; shapes outside the
// table (very large K) run the generic streaming kernel, which handles any
// size with runtime loops.
#include <array>
#include <cstdint>
#include <string>
#include <utility>

#include "device_common.h"
#include "gemm_rows.h"
#include "gemm_rows64.h"
#include "gemm_stream.h"
#include "gemm_tiled.h"
#include "gemm_w8a16.h"
#include "launch.h"
#include "rows_launch.h"

namespace fp8bq {

namespace {

// 65..80 tokens stream only where a workgroup holds at most this many row
// tiles and a wave at most this many groups (both limits by register use)
constexpr int kWideMaxTiles = 2;
constexpr int kWideMaxGroups = 5;

template <int TILES, int GMAX, int MSX = 4>
hipError_t rows64_instance(const GemmArgs& a, int64_t rows_per_wg) {
  // with one row tile the activation fragments in flight dominate the
  // register budget: keep fewer weight chunks ahead
  constexpr int PD = TILES == 1 ? 2 : 3;
  const unsigned grid = static_cast<unsigned>((a.n + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL((gemm_rows64_kernel<GMAX, TILES, PD, MSX>), dim3(grid), dim3(64 * kRowsWaves), 0, a.stream,
                     static_cast<int>(a.m), a.n, a.k, rows_per_wg, static_cast<const unsigned char*>(a.aq), a.as,
                     static_cast<const unsigned char*>(a.wq), a.ws, static_cast<unsigned short*>(a.c));
  return hipGetLastError();
}

// Token classes: up to 8 tokens (16-token tile, operand loaded directly),
// 9..16 and 17..32 (16- and 32-token tiles, activation read as whole lines
// and transposed; the 32-token tile walks the chunks group-major when a
// wave has more than 6 groups, so that only the groups in use are held --
// with up to 2 row tiles; with more, those registers still do not fit and
// the 64-token kernel serves), and 33..48, 49..64 and 65..80 tokens
// (gemm_rows64.h with three, four or five 16-token sub-tiles: at M = 33..48
// the three cost 3-10% less than four on the five logged shapes; five at
// 65..80 cost 7-12% less than the tiled kernel where they fit).
template <int TT, int TILES, int GMAX>
constexpr Launch rows_entry() {
  if constexpr (TT == 80) {
    // 65..80 tokens, five sub-tiles: only where a workgroup has at most 2
    // row tiles and a wave at most 5 groups (beyond, the accumulators and
    // the held activation no longer fit in registers and spill)
    if constexpr (TILES <= kWideMaxTiles && GMAX <= kWideMaxGroups)
      return &rows64_instance<TILES, GMAX, 5>;
    else
      return nullptr;
  } else if constexpr (TT == 48)
    return &rows64_instance<TILES, GMAX, 3>;
  else if constexpr (TT == 64 || (TT == 32 && GMAX > 6 && TILES > 2))
    return &rows64_instance<TILES, GMAX>;
  else if constexpr (TT == 8)
    return &rows_instance<16, kActCodes, TILES, GMAX>;
  else
    return &rows_instance<TT, kActCodeLines, TILES, GMAX>;
}

template <int TT, int TILES, int... G>
constexpr std::array<Launch, sizeof...(G)> rows_row(std::integer_sequence<int, G...>) {
  return {rows_entry<TT, TILES, G + 1>()...};
}

template <int TT, int... T>
constexpr std::array<std::array<Launch, kMaxGroupsPerWave>, sizeof...(T)> rows_table(std::integer_sequence<int, T...>) {
  return {rows_row<TT, T + 1>(std::make_integer_sequence<int, kMaxGroupsPerWave>{})...};
}

// Weight-only (bf16 activation) instances, up to 16 tokens.
template <int TILES, int GMAX>
hipError_t w8a16_instance(const GemmArgs& a, int64_t rows_per_wg) {
  // 16 activation registers per group: keep fewer chunks ahead at large K
  constexpr int PD = GMAX >= 8 ? 2 : (GMAX >= 7 ? 4 : 6);
  const unsigned grid = static_cast<unsigned>((a.n + rows_per_wg - 1) / rows_per_wg);
  hipLaunchKernelGGL((gemm_w8a16_kernel<GMAX, TILES, PD>), dim3(grid), dim3(64 * kRowsWaves), 0, a.stream,
                     static_cast<int>(a.m), a.n, a.k, rows_per_wg, static_cast<const unsigned short*>(a.aq),
                     static_cast<const unsigned char*>(a.wq), a.ws, static_cast<unsigned short*>(a.c));
  return hipGetLastError();
}

template <int TILES, int... G>
constexpr std::array<Launch, sizeof...(G)> w8a16_row(std::integer_sequence<int, G...>) {
  return {&w8a16_instance<TILES, G + 1>...};
}

template <int... T>
constexpr std::array<std::array<Launch, kMaxGroupsPerWave>, sizeof...(T)> w8a16_table(std::integer_sequence<int, T...>) {
  return {w8a16_row<T + 1>(std::make_integer_sequence<int, kMaxGroupsPerWave>{})...};
}

constexpr auto kW8A16 = w8a16_table(std::make_integer_sequence<int, kMaxTiles>{});

constexpr auto kRows8 = rows_table<8>(std::make_integer_sequence<int, kMaxTiles>{});
constexpr auto kRows16 = rows_table<16>(std::make_integer_sequence<int, kMaxTiles>{});
constexpr auto kRows32 = rows_table<32>(std::make_integer_sequence<int, kMaxTiles>{});
constexpr auto kRows48 = rows_table<48>(std::make_integer_sequence<int, kMaxTiles>{});
constexpr auto kRows80 = rows_table<80>(std::make_integer_sequence<int, kMaxTiles>{});
constexpr auto kRows64 = rows_table<64>(std::make_integer_sequence<int, kMaxTiles>{});

template <int MT, int R, int S, int U>
hipError_t stream_instance(const GemmArgs& a) {
  hipLaunchKernelGGL((gemm_stream_kernel<MT, R, S, U>), dim3(stream_grid<R>(a.n)), dim3(64 * S), 0, a.stream,
                     static_cast<int>(a.m), a.n, a.k, static_cast<const unsigned char*>(a.aq), a.as,
                     static_cast<const unsigned char*>(a.wq), a.ws, static_cast<unsigned short*>(a.c));
  return hipGetLastError();
}

// C = bf16_rne(part[0] + part[1] + ... + part[split - 1]) elementwise, the
// parts added in that order (deterministic): the K-split tiled path's second
// launch. count = M * N; four outputs per thread when count % 4 == 0 (part
// and c 16-byte aligned). S > 0: the number of parts as a compile-time
// constant (all S loads in flight together); S = 0: any `split`.
template <int S>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int split, int64_t count,
                                                           unsigned short* __restrict__ c) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  const int64_t first = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int parts = S > 0 ? S : split;
  if ((count & 3) == 0) {
    const v4f* p = reinterpret_cast<const v4f*>(part);
    const int64_t q4 = count >> 2;
    for (int64_t q = first; q < q4; q += stride) {
      v4f sum;
      if constexpr (S > 0) {
        v4f t[S];
#pragma unroll
        for (int u = 0; u < S; ++u) t[u] = __builtin_nontemporal_load(p + u * q4 + q);
        sum = t[0];
#pragma unroll
        for (int u = 1; u < S; ++u) sum += t[u];
      } else {
        sum = p[q];
        for (int u = 1; u < parts; ++u) sum += __builtin_nontemporal_load(p + u * q4 + q);
      }
      v2u packed;
      packed[0] = pack_bf16x2(sum[0], sum[1]);
      packed[1] = pack_bf16x2(sum[2], sum[3]);
      reinterpret_cast<v2u*>(c)[q] = packed;
    }
  } else {
    for (int64_t i = first; i < count; i += stride) {
      float sum = part[i];
      for (int u = 1; u < parts; ++u) sum += part[u * count + i];
      c[i] = static_cast<unsigned short>(pack_bf16x2(sum, 0.f) & 0xffffu);
    }
  }
}

template <int... S>
constexpr std::array<void (*)(const float*, int, int64_t, unsigned short*), sizeof...(S)> reduce_table(
    std::integer_sequence<int, S...>) {
  return {&split_reduce_kernel<S>...};
}
// split_reduce_kernel<S> for S = 0 (any split) .. 16
constexpr auto kSplitReduce = reduce_table(std::make_integer_sequence<int, 17>{});

__global__ void fill_zero_kernel(unsigned short* __restrict__ c, int64_t count) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count; i += stride) c[i] = 0;
}

}  // namespace

// Description of a row-range launch for the kernel-choice log.
static std::string rows_desc(const char* kernel, int64_t n, int64_t rows_per_wg, int tiles, int gmax) {
  return std::string(kernel) + " TILES=" + std::to_string(tiles) + " GMAX=" + std::to_string(gmax) +
         " rows/wg=" + std::to_string(rows_per_wg) + " grid=" + std::to_string((n + rows_per_wg - 1) / rows_per_wg);
}

hipError_t launch_gemm_stream(int64_t m, int64_t n, int64_t k, const void* aq, const float* as,
                              const void* wq, const float* ws, void* c, hipStream_t stream) {
  const GemmArgs a{m, n, k, aq, as, wq, ws, c, stream};
  int64_t rows_per_wg;
  int tiles, gmax;
  if (m > 64) {  // 65..80 tokens, only where stream_wide_serves
    if (!stream_wide_serves(m, n, k)) return hipErrorInvalidValue;
    rows_shape(n, k, &rows_per_wg, &tiles, &gmax);
    dispatch_log("gemm(stream)", m, n, k,
                 rows_desc("gemm_rows64_kernel MS=5", n, rows_per_wg, tiles, gmax).c_str());
    return kRows80[tiles - 1][gmax - 1](a, rows_per_wg);
  }
  if (rows_shape(n, k, &rows_per_wg, &tiles, &gmax)) {
    const auto& table = m <= 8 ? kRows8 : m <= 16 ? kRows16 : m <= 32 ? kRows32 : m <= 48 ? kRows48 : kRows64;
    const char* kernel = m <= 8    ? "gemm_rows_kernel MT=16 act=codes"
                         : m <= 16 ? "gemm_rows_kernel MT=16 act=lines"
                         : m <= 32 ? (gmax > 6 && tiles > 2 ? "gemm_rows64_kernel" : "gemm_rows_kernel MT=32 act=lines")
                                   : "gemm_rows64_kernel";
    dispatch_log("gemm(stream)", m, n, k, rows_desc(kernel, n, rows_per_wg, tiles, gmax).c_str());
    return table[tiles - 1][gmax - 1](a, rows_per_wg);
  }
  // Generic streaming kernel: any N and K, 16-row slabs, runtime K loop.
  dispatch_log("gemm(stream)", m, n, k, "gemm_stream_kernel (generic: K beyond the instance table)");
  if (m <= 16) return stream_instance<16, 1, 8, 5>(a);
  if (m <= 32) return stream_instance<32, 1, 8, 4>(a);
  return stream_instance<64, 1, 8, 2>(a);
}

// 33..64 tokens where each wave of the streaming kernel walks a long K
// range (8 or 9 groups) over a short row range (2 row tiles, N = 4097..8192;
// a single row tile was not measured): there
// the wave's serial chain, not HBM, sets the streaming time, and the
// K-split tiled plan of fp8bq_gemm_ws measured faster: on (5120, 8704)
// 16.1 / 17.5 us against 19.7 / 23.8 at M = 48 / 64 (64 x 128 tiles in 6
// parts), while on the other logged shapes streaming stayed ahead.
bool stream_deep_k(int64_t m, int64_t n, int64_t k) {
  int64_t rows_per_wg;
  int tiles, gmax;
  return m > 32 && m <= 64 && rows_shape(n, k, &rows_per_wg, &tiles, &gmax) && tiles == 2 && gmax >= 8;
}

bool stream_wide_serves(int64_t m, int64_t n, int64_t k) {
  int64_t rows_per_wg;
  int tiles, gmax;
  return m > 64 && m <= 80 && rows_shape(n, k, &rows_per_wg, &tiles, &gmax) && tiles <= kWideMaxTiles &&
         gmax <= kWideMaxGroups;
}

bool small_m_supported(int64_t m, int64_t n, int64_t k) {
  int64_t rows_per_wg;
  int tiles, gmax;
  return m >= 1 && m <= 16 && rows_shape(n, k, &rows_per_wg, &tiles, &gmax);
}

hipError_t launch_gemm_w8a16(int64_t m, int64_t n, int64_t k, const void* a, const void* wq, const float* ws, void* c,
                             hipStream_t stream) {
  const GemmArgs args{m, n, k, a, nullptr, wq, ws, c, stream};
  int64_t rows_per_wg;
  int tiles, gmax;
  if (m < 1 || m > 16 || !rows_shape(n, k, &rows_per_wg, &tiles, &gmax)) return hipErrorInvalidValue;
  dispatch_log("gemm_w8a16", m, n, k, rows_desc("gemm_w8a16_kernel", n, rows_per_wg, tiles, gmax).c_str());
  return kW8A16[tiles - 1][gmax - 1](args, rows_per_wg);
}

// One launch of gemm_tiled_kernel: the whole K range per tile into C, or
// (split > 1) `split` K parts per tile into the fp32 partial tiles `part`.
template <int BM, int BN, int WM, int WN, int STAGES>
hipError_t tiled_instance(int64_t m, int64_t n, int64_t k, const void* aq, const float* as, const void* wq,
                          const float* ws, void* c, hipStream_t stream, int split = 1, float* part = nullptr) {
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN, WM, WN, STAGES>), dim3(static_cast<unsigned>(tiles * split)),
                     dim3(64 * WM * WN), 0, stream, m, n, k, split, static_cast<const unsigned char*>(aq), as,
                     static_cast<const unsigned char*>(wq), ws, static_cast<unsigned short*>(c), part);
  return hipGetLastError();
}

// The 8-wave two-stage tiles (192 x 256, 256 x 256): gemm_tiled2_kernel,
// unclamped when every row of every tile exists once the last token tile is
// shifted back (M >= BM, N a multiple of BN, a tile's rows within 32-bit
// copy offsets). A last round of at most 128 tiles after whole rounds
// (e.g. M = 3465 on (5120, 8704): 380 tiles of 192 x 256 = 256 + 124) runs
// as a second launch of column halves, 2 x 124 workgroups of 192 x 128 in
// one round (measured at 0.66 of a whole round's time), instead of 124
// whole tiles leaving half the CUs idle.
template <int BM, int BN, bool CLAMP>
void tiled2_launch(int64_t m, int64_t n, int64_t k, int64_t t0, int split, int64_t grid, const void* aq,
                   const float* as, const void* wq, const float* ws, void* c, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_tiled2_kernel<BM, BN, 2, 4, CLAMP>), dim3(static_cast<unsigned>(grid)), dim3(512), 0, stream,
                     m, n, k, t0, split, static_cast<const unsigned char*>(aq), as,
                     static_cast<const unsigned char*>(wq), ws, static_cast<unsigned short*>(c));
}

template <int BM, int BN>
struct Tiled2Plan {
  int64_t tiles, whole, halves;  // tiles of BM x BN; whole tiles launched first; then column halves
  Tiled2Plan(int64_t m, int64_t n) {
    tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
    const int64_t rem = tiles % kNumCUs;
    const bool split = tiles > kNumCUs && rem > 0 && 2 * rem <= kNumCUs;
    whole = split ? tiles - rem : tiles;
    halves = split ? 2 * rem : 0;
  }
};

template <int BM, int BN>
hipError_t tiled2_instance(int64_t m, int64_t n, int64_t k, const void* aq, const float* as, const void* wq,
                           const float* ws, void* c, hipStream_t stream) {
  const Tiled2Plan<BM, BN> plan(m, n);
  const bool exact = m >= BM && n % BN == 0 && k < (int64_t(1) << 23);
  if (plan.whole > 0) {
    if (exact)
      tiled2_launch<BM, BN, false>(m, n, k, 0, 1, plan.whole, aq, as, wq, ws, c, stream);
    else
      tiled2_launch<BM, BN, true>(m, n, k, 0, 1, plan.whole, aq, as, wq, ws, c, stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (plan.halves > 0) {
    if (exact)
      tiled2_launch<BM, BN / 2, false>(m, n, k, plan.whole, 2, plan.halves, aq, as, wq, ws, c, stream);
    else
      tiled2_launch<BM, BN / 2, true>(m, n, k, plan.whole, 2, plan.halves, aq, as, wq, ws, c, stream);
  }
  return hipGetLastError();
}

namespace {

struct TileShape {
  int bm, bn;
  int per_cu;  // workgroups one CU holds at once (LDS: 1 for 8-wave and 128 x 128 tiles, 2 for the halves, 3 for 64 x 64)
  // measured time of one K step of one round of resident workgroups,
  // 1/100 us (MI355X, Gaussian data): with at most one workgroup per CU,
  // and with two or three on some CUs (per_cu > 1, grids of more than 256
  // tiles)
  int step_cost, step_cost2;
  const char* desc;
  bool halves_last = false;  // 8-wave tiles: a last round of <= 128 tiles as column halves
  int step_cost_halves = 0;  // ... at this measured cost (1/100 us per K step)
};
// Indexed as the forced tile-shape paths of fp8bq_gemm_forced (0..6 =
// FP8BQ_PATH_TILED_128x128 .. FP8BQ_PATH_TILED_64x64).
constexpr TileShape kTileShapes[] = {
    {128, 128, 1, 85, 85, "gemm_tiled_kernel BM=128 BN=128 4 waves 3 stages"},
    {128, 256, 1, 115, 115, "gemm_tiled_kernel BM=128 BN=256 8 waves 3 stages"},
    {192, 256, 1, 150, 150, "gemm_tiled2_kernel BM=192 BN=256 8 waves 2 stages", true, 126},
    {256, 256, 1, 178, 178, "gemm_tiled2_kernel BM=256 BN=256 8 waves 2 stages", true, 140},
    {64, 128, 2, 60, 100, "gemm_tiled_kernel BM=64 BN=128 4 waves 3 stages"},
    {128, 64, 2, 60, 100, "gemm_tiled_kernel BM=128 BN=64 4 waves 3 stages"},
    {64, 64, 3, 52, 90, "gemm_tiled_kernel BM=64 BN=64 4 waves 3 stages"},
};
constexpr int kNumTileShapes = sizeof(kTileShapes) / sizeof(kTileShapes[0]);

int64_t tile_count(int64_t m, int64_t n, const TileShape& t) { return ((m + t.bm - 1) / t.bm) * ((n + t.bn - 1) / t.bn); }

}  // namespace

// Tile shape for the tiled kernel: the one with the least rounds x step
// cost. A grid runs in ceil(tiles / (256 x workgroups per CU)) rounds, each
// as long as its K loop; the step costs are measured.
//  - Larger tiles re-read fewer LDS and L2 bytes per MFMA (a step of a
//    256 x 256 tile does twice the work of a 128 x 256 one at 1.65x its
//    time) but make fewer tiles, so a grid just past a whole number of
//    rounds takes the smaller tile that stays within them (M = 3465:
//    (17408, 5120) takes 256 x 256, 4 rounds; (5120, 8704) 192 x 256, 2
//    rounds instead of 256 x 256's 1.09).
//  - Few tokens leave most CUs idle with large tiles: the 4-wave halves
//    (64 x 128, 128 x 64; two fit in one CU's LDS) and quarters (64 x 64,
//    three per CU) fill them, e.g. 160 tiles instead of 40 at M = 65..128
//    on N = 5120 (M = 128 at (5120, 8704): 32 us against 59 with 128 x 128
//    tiles and 48 streaming the weights twice). Once their grid outgrows
//    one workgroup per CU the smaller tiles lose their edge (64 x 64 at
//    M = 192 on N = 8192: 35 us against 26 for 128 x 64).
//  - The 8-wave tiles run a last round of at most 128 tiles (after whole
//    rounds) as column halves, which measured 0.84 of a whole round (a half
//    tile's K step is bound by its copies' latency more than by its MFMAs):
//    M = 3465 on (5120, 8704), 380 tiles of 192 x 256, 189 -> 173 us.
// Equal costs go to the grid with more tiles (the better-filled machine),
// then to the earlier shape in the order 64x64, 64x128, 128x64, 128x128,
// 128x256, 192x256, 256x256.
int tiled_shape(int64_t m, int64_t n, int64_t* step_cost) {
  constexpr int kOrder[kNumTileShapes] = {6, 4, 5, 0, 1, 2, 3};
  int best = 0;
  int64_t best_cost = INT64_MAX, best_tiles = 0;
  for (int i : kOrder) {
    const TileShape& t = kTileShapes[i];
    const int64_t tiles = tile_count(m, n, t);
    const int64_t cap = static_cast<int64_t>(kNumCUs) * t.per_cu;
    const int64_t rounds = (tiles + cap - 1) / cap;
    int64_t cost = rounds * (tiles > kNumCUs ? t.step_cost2 : t.step_cost);
    if (t.halves_last) {  // a last round of <= 128 tiles runs as column halves
      const int64_t rem = tiles % kNumCUs;
      if (tiles > kNumCUs && rem > 0 && 2 * rem <= kNumCUs) cost = (rounds - 1) * t.step_cost + t.step_cost_halves;
    }
    if (cost < best_cost || (cost == best_cost && tiles > best_tiles)) {
      best = i;
      best_cost = cost;
      best_tiles = tiles;
    }
  }
  if (step_cost != nullptr) *step_cost = best_cost;
  return best;
}

// K-split plan for the tiled path when the caller gives a workspace
// (fp8bq_gemm_ws). With few tiles (M = 65..~256 tokens: 20..136 tiles on
// the logged shapes) most CUs sit idle while each tile walks all K/128
// groups; splitting every tile's groups into `split` parts fills the CUs,
// each part writing an fp32 partial tile, and a second launch adds the
// parts in a fixed order. Costs in 1/100 us, fitted to measured times
// (MI355X, the five logged shapes at M = 81, 128, 256, every splittable
// shape x 2..24 parts; least squares, mean error 7%):
//   split:   0.965 x rounds(tiles x split) x ceil(groups / split) x step
//            cost + 0.418 us per MB of partial tiles (written once, read
//            once) + 7.9 us (the second launch, the pipeline's fill and
//            drain at short K ranges);
//   unsplit: 1.146 x rounds(tiles) x groups x step cost - 1.8 us.
// The split runs where its cost is the lower: e.g. M = 81 on (5120, 8704)
// 128 x 128 tiles in 6 parts, 19.6 us against 29.5; on (17408, 5120)
// 128 x 256 tiles in 3 parts, 31.7 against 37.3; not on (5120, 3072),
// whose 24 groups leave too little K per part. Only the gemm_tiled_kernel
// shapes split (not the two-stage 192 x 256 / 256 x 256 tiles).
constexpr int64_t kSplitStepPerMille = 965;
constexpr int64_t kSplitPerByteE7 = 418;  // 1/100 us per 10^7 bytes of partial tiles
constexpr int64_t kSplitFixed = 790;
constexpr int64_t kUnsplitPerMille = 1146;
constexpr int64_t kUnsplitOffset = -178;
constexpr int kMaxSplit = 64;

int64_t tile_grid(int64_t m, int64_t n, int shape) {
  return shape >= 0 && shape < kNumTileShapes ? tile_count(m, n, kTileShapes[shape]) : 0;
}

SplitPlan split_plan(int64_t m, int64_t n, int64_t k) {
  SplitPlan plan;
  const int64_t groups = k / kGroup;
  if (m < 1 || n < 1 || groups < 2) return plan;
  int64_t step;
  plan.shape = tiled_shape(m, n, &step);
  plan.cost = kUnsplitPerMille * step * groups / 1000 + kUnsplitOffset;
  constexpr int kSplitShapes[] = {6, 4, 5, 0, 1};
  for (int i : kSplitShapes) {
    const TileShape& t = kTileShapes[i];
    const int64_t tiles = tile_count(m, n, t);
    const int64_t cap = static_cast<int64_t>(kNumCUs) * t.per_cu;
    for (int64_t sp = 2; sp <= groups && sp <= kMaxSplit; ++sp) {
      const int64_t items = tiles * sp;
      if (items > 4 * cap) break;
      const int64_t rounds = (items + cap - 1) / cap;
      const int64_t steps = (groups + sp - 1) / sp;
      const int64_t compute = rounds * steps * (items > kNumCUs ? t.step_cost2 : t.step_cost);
      const int64_t cost = kSplitStepPerMille * compute / 1000 + kSplitPerByteE7 * (sp * m * n * 4) / 10000000 +
                           kSplitFixed;
      if (cost < plan.cost) {
        plan.shape = i;
        plan.split = static_cast<int>(sp);
        plan.cost = cost;
      }
    }
  }
  return plan;
}

hipError_t launch_gemm_split(int64_t m, int64_t n, int64_t k, const void* aq, const float* as, const void* wq,
                             const float* ws, void* c, float* part, int shape, int split, hipStream_t stream) {
  if (split < 2 || split > k / kGroup || (shape != 0 && shape != 1 && shape != 4 && shape != 5 && shape != 6))
    return hipErrorInvalidValue;
  const std::string desc = std::string(kTileShapes[shape].desc) + " grid=" +
                           std::to_string(tile_count(m, n, kTileShapes[shape]) * split) + " (K in " +
                           std::to_string(split) + " parts) + split_reduce_kernel";
  dispatch_log("gemm(tiled, split K)", m, n, k, desc.c_str());
  hipError_t e;
  switch (shape) {
    case 0: e = tiled_instance<128, 128, 2, 2, 3>(m, n, k, aq, as, wq, ws, c, stream, split, part); break;
    case 1: e = tiled_instance<128, 256, 2, 4, 3>(m, n, k, aq, as, wq, ws, c, stream, split, part); break;
    case 4: e = tiled_instance<64, 128, 1, 4, 3>(m, n, k, aq, as, wq, ws, c, stream, split, part); break;
    case 5: e = tiled_instance<128, 64, 2, 2, 3>(m, n, k, aq, as, wq, ws, c, stream, split, part); break;
    default: e = tiled_instance<64, 64, 2, 2, 3>(m, n, k, aq, as, wq, ws, c, stream, split, part); break;
  }
  if (e != hipSuccess) return e;
  const int64_t count = m * n;
  const int64_t per = (count & 3) == 0 ? count / 4 : count;
  int64_t blocks = (per + 255) / 256;
  blocks = blocks < 2048 ? blocks : 2048;
  hipLaunchKernelGGL(kSplitReduce[split < static_cast<int>(kSplitReduce.size()) ? split : 0],
                     dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, part, split, count,
                     static_cast<unsigned short*>(c));
  return hipGetLastError();
}

hipError_t launch_gemm_tiled(int64_t m, int64_t n, int64_t k, const void* aq, const float* as,
                             const void* wq, const float* ws, void* c, hipStream_t stream, int shape) {
  if (shape < 0) shape = tiled_shape(m, n, nullptr);
  if (shape >= kNumTileShapes) return hipErrorInvalidValue;
  std::string desc = std::string(kTileShapes[shape].desc) + " grid=" + std::to_string(tile_count(m, n, kTileShapes[shape]));
  if (shape == 2 || shape == 3) {
    const int64_t whole = shape == 2 ? Tiled2Plan<192, 256>(m, n).whole : Tiled2Plan<256, 256>(m, n).whole;
    const int64_t halves = shape == 2 ? Tiled2Plan<192, 256>(m, n).halves : Tiled2Plan<256, 256>(m, n).halves;
    if (halves > 0)
      desc += " (" + std::to_string(whole) + " whole + " + std::to_string(halves) + " column halves)";
  }
  dispatch_log("gemm(tiled)", m, n, k, desc.c_str());
  switch (shape) {
    case 0:
      return tiled_instance<128, 128, 2, 2, 3>(m, n, k, aq, as, wq, ws, c, stream);
    case 1:
      return tiled_instance<128, 256, 2, 4, 3>(m, n, k, aq, as, wq, ws, c, stream);
    case 2:
      return tiled2_instance<192, 256>(m, n, k, aq, as, wq, ws, c, stream);
    case 3:
      return tiled2_instance<256, 256>(m, n, k, aq, as, wq, ws, c, stream);
    case 4:
      return tiled_instance<64, 128, 1, 4, 3>(m, n, k, aq, as, wq, ws, c, stream);
    case 5:
      return tiled_instance<128, 64, 2, 2, 3>(m, n, k, aq, as, wq, ws, c, stream);
    default:
      return tiled_instance<64, 64, 2, 2, 3>(m, n, k, aq, as, wq, ws, c, stream);
  }
}

hipError_t launch_fill_zero_bf16(int64_t count, void* c, hipStream_t stream) {
  int64_t blocks = (count + 255) / 256;
  blocks = blocks < 65536 ? blocks : 65536;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<unsigned short*>(c), count);
  return hipGetLastError();
}

}  // namespace fp8bq

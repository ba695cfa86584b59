// LDS-tiled FP8 MFMA block-scaled GEMM for large M (batches, prefill),
// gfx950.
//
// At M in the thousands (page 2, ownding.com L20 report, section 4.2: a
// 3,465-token prompt; section 8: prefill forced onto an M=1 config regressed)
// the op is a dense contraction well above the FP8 ridge, so it runs on the
// matrix cores. A workgroup of 4 waves computes a BM x BN tile of C (tokens x
// weight rows) and walks K one 128-wide scale group at a time:
//   1. the group's A tile (BM x 128 codes) and W tile (BN x 128 codes) are
//      copied global -> registers -> LDS, double-buffered so the next
//      group's copy overlaps this group's MFMAs;
//   2. each wave multiplies its (BN/2) x (BM/2) sub-tile with 16x16x128 FP8
//      MFMAs into fresh fp32 accumulators (one instruction per 16x16 tile per
//      group, weight rows as the first operand);
//   3. the fresh result is scaled by A_scale[m, g] * W_scale[n / 128, g] and
//      added to the running fp32 tile (BN = 128 keeps one weight block per
//      tile, so the weight scale is uniform over the workgroup).
// LDS rows are padded from 128 to 144 bytes so that the 16-byte operand
// reads of 8 consecutive lanes (8 different rows, same column) hit 32
// distinct banks. Rows past M or N are clamped onto the last valid row for
// loading and masked at the store.
#pragma once

#include "device_common.h"

namespace fp8bq {

constexpr int kTileLdsStride = 144;  // bytes per LDS row (128 + 16 pad)

template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(int64_t m_rows, int64_t n, int64_t k,
                                                         const unsigned char* __restrict__ aq,
                                                         const float* __restrict__ as,
                                                         const unsigned char* __restrict__ wq,
                                                         const float* __restrict__ ws,
                                                         unsigned short* __restrict__ c) {
  static_assert(BN == 128, "one weight scale block per tile");
  static_assert(BM % 32 == 0 && BM <= 128, "BM");
  constexpr int WM = BM / 2;  // tokens per wave
  constexpr int WN = BN / 2;  // weight rows per wave
  constexpr int TM = WM / 16; // 16-token sub-tiles per wave
  constexpr int TN = WN / 16; // 16-row sub-tiles per wave
  constexpr int A_LOADS = BM * 8 / 256;  // 16-byte chunks per thread for A
  constexpr int W_LOADS = BN * 8 / 256;

  __shared__ __attribute__((aligned(16))) unsigned char lds_a[2][BM * kTileLdsStride];
  __shared__ __attribute__((aligned(16))) unsigned char lds_w[2][BN * kTileLdsStride];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int lrow = lane & 15;
  const int quarter = lane >> 4;
  const int wave_n = wave & 1;   // which half of the BN rows
  const int wave_m = wave >> 1;  // which half of the BM tokens
  const int64_t groups = k >> 7;
  // Linear tile id -> (weight-row tile, token tile), token tile fastest so
  // that consecutive workgroups share one weight tile.
  const int64_t m_tiles = (m_rows + BM - 1) / BM;
  const int64_t tile = blockIdx.x;
  const int64_t n0 = (tile / m_tiles) * BN;
  const int64_t m0 = (tile % m_tiles) * BM;

  // Global -> LDS copy assignment: thread t moves 16-byte chunk t % 8 of
  // rows t / 8 + 32 j.
  const int chunk = t & 7;
  const unsigned char* a_src[A_LOADS];
  const unsigned char* w_src[W_LOADS];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    int64_t row = m0 + (t >> 3) + 32 * j;
    row = row < m_rows ? row : m_rows - 1;
    a_src[j] = aq + row * k + chunk * 16;
  }
#pragma unroll
  for (int j = 0; j < W_LOADS; ++j) {
    int64_t row = n0 + (t >> 3) + 32 * j;
    row = row < n ? row : n - 1;
    w_src[j] = wq + row * k + chunk * 16;
  }
  const float* sw_row = ws + ((n0 < n ? n0 : n - 1) >> 7) * groups;
  // Activation scale rows of this lane's tokens (one per 16-token sub-tile).
  const float* sa_row[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    int64_t m = m0 + wave_m * WM + 16 * i + lrow;
    m = m < m_rows ? m : m_rows - 1;
    sa_row[i] = as + m * groups;
  }

  v4u a_stage[A_LOADS];
  v4u w_stage[W_LOADS];
  auto fetch = [&](int64_t g) {
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j) a_stage[j] = *reinterpret_cast<const v4u*>(a_src[j] + g * kGroup);
#pragma unroll
    for (int j = 0; j < W_LOADS; ++j) w_stage[j] = *reinterpret_cast<const v4u*>(w_src[j] + g * kGroup);
  };
  auto park = [&](int buf) {
#pragma unroll
    for (int j = 0; j < A_LOADS; ++j)
      *reinterpret_cast<v4u*>(&lds_a[buf][((t >> 3) + 32 * j) * kTileLdsStride + chunk * 16]) = a_stage[j];
#pragma unroll
    for (int j = 0; j < W_LOADS; ++j)
      *reinterpret_cast<v4u*>(&lds_w[buf][((t >> 3) + 32 * j) * kTileLdsStride + chunk * 16]) = w_stage[j];
  };

  v4f acc[TN][TM];
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  fetch(0);
  park(0);
  __syncthreads();

  for (int64_t g = 0; g < groups; ++g) {
    const int buf = static_cast<int>(g & 1);
    if (g + 1 < groups) fetch(g + 1);

    // Operand reads: lane l takes row l % 16 of a sub-tile, bytes
    // 16 (l / 16) .. +15 and 64 + 16 (l / 16) .. +15.
    v8i wop[TN];
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const unsigned char* p = &lds_w[buf][(wave_n * WN + 16 * i + lrow) * kTileLdsStride + quarter * 16];
      const v4u lo = *reinterpret_cast<const v4u*>(p);
      const v4u hi = *reinterpret_cast<const v4u*>(p + 64);
      wop[i] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    v8i aop[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const unsigned char* p = &lds_a[buf][(wave_m * WM + 16 * j + lrow) * kTileLdsStride + quarter * 16];
      const v4u lo = *reinterpret_cast<const v4u*>(p);
      const v4u hi = *reinterpret_cast<const v4u*>(p + 64);
      aop[j] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    const float sw = sw_row[g];
    float sc[TM];
#pragma unroll
    for (int j = 0; j < TM; ++j) sc[j] = sa_row[j][g] * sw;

#pragma unroll
    for (int i = 0; i < TN; ++i) {
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const v4f p = mfma_16x16x128_e4m3(wop[i], aop[j]);
        acc[i][j][0] = fmaf(sc[j], p[0], acc[i][j][0]);
        acc[i][j][1] = fmaf(sc[j], p[1], acc[i][j][1]);
        acc[i][j][2] = fmaf(sc[j], p[2], acc[i][j][2]);
        acc[i][j][3] = fmaf(sc[j], p[3], acc[i][j][3]);
      }
    }
    if (g + 1 < groups) park(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: lane holds, for each sub-tile, rows n = 4 (l / 16) + 0..3 of
  // token m = l % 16: four consecutive outputs of C's row m.
#pragma unroll
  for (int j = 0; j < TM; ++j) {
    const int64_t m = m0 + wave_m * WM + 16 * j + lrow;
    if (m >= m_rows) continue;
#pragma unroll
    for (int i = 0; i < TN; ++i) {
      const int64_t col = n0 + wave_n * WN + 16 * i + 4 * quarter;
      unsigned short* dst = c + m * n + col;
      const v4f v = acc[i][j];
      if ((n & 3) == 0 && col + 3 < n) {
        v2u packed;
        packed[0] = pack_bf16x2(v[0], v[1]);
        packed[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<v2u*>(dst) = packed;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e < n) dst[e] = static_cast<unsigned short>(pack_bf16x2(v[e], 0.f) & 0xffffu);
      }
    }
  }
}

}  // namespace fp8bq

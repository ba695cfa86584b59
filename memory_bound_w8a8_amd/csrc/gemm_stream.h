// Weight-streaming split-K block-FP8 GEMM for small M (decode, speculative
// verification, small batches), gfx950.
//
// The pages put about 89% of each decode step in weight-reading matmuls that
// already sit near the bandwidth floor (page 1, SmartX blog, section
// "operator optimisation"); at M = 1..64 the op reads each weight byte once
// and does 2M flops per byte, far below the FP8 MFMA ridge, so this kernel is
// organised around HBM: every weight byte is fetched exactly once with
// 16-byte loads, many loads are in flight per wave, and arithmetic is kept
// off the critical path.
//
// Work decomposition. A workgroup owns R slabs of 16 consecutive weight rows
// and all of K; its S waves split the K/128 scale groups into S contiguous
// ranges (split-K). Per group, a wave loads for each slab 16 rows x 128
// bytes of W (lane l: row l % 16, bytes 16 (l / 16) .. +15 and 64 + 16 (l /
// 16) .. +15, so each load instruction covers 64 contiguous bytes of 16
// rows) and the matching bytes of up to MT activation rows, and issues one
// 16x16x128 FP8 MFMA per (slab, 16-token tile). The MFMA does the 128-long
// inner products; its fresh fp32 result is scaled by A_scale[m, g] *
// W_scale[n / 128, g] (the weight scale is uniform over the 16 rows, one
// activation scale per lane) and added to the running fp32 sum. Waves then
// sum their partial 16x16 tiles through LDS in a fixed order (deterministic,
// no atomics) and the result is rounded to bf16 and stored, 4 consecutive
// outputs (8 bytes) per lane.
//
// Template parameters: MT = token tile (16, 32 or 64; M <= MT), R = slabs per
// workgroup, S = waves per workgroup (split-K factor), U = groups whose loads
// are issued together before their MFMAs.
#pragma once

#include "device_common.h"

namespace fp8bq {

template <int MT, int R, int S, int U>
__global__ __launch_bounds__(64 * S) void gemm_stream_kernel(int m_rows, int64_t n, int64_t k,
                                                            const unsigned char* __restrict__ aq,
                                                            const float* __restrict__ as,
                                                            const unsigned char* __restrict__ wq,
                                                            const float* __restrict__ ws,
                                                            unsigned short* __restrict__ c) {
  constexpr int MS = MT / 16;  // 16-token tiles
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lrow = lane & 15;
  const int quarter = lane >> 4;
  const int groups = static_cast<int>(k >> 7);
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * (16 * R);

  // This wave's contiguous range of K groups.
  const int per = groups / S;
  const int rem = groups - per * S;
  const int gbeg = wave * per + (wave < rem ? wave : rem);
  const int gcnt = per + (wave < rem ? 1 : 0);

  // Weight rows (clamped into [0, N) for a short last slab; those outputs
  // are never stored) and the row index of each slab's scale block.
  const unsigned char* wp[R];
  const float* swp[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t row = n0 + 16 * r + lrow;
    row = row < n ? row : n - 1;
    wp[r] = wq + row * k + quarter * 16;
    int64_t first = n0 + 16 * r;
    first = first < n ? first : n - 1;
    swp[r] = ws + (first >> 7) * groups;
  }
  // Activation rows of each token tile; lanes past M load nothing.
  const unsigned char* ap[MS];
  const float* sap[MS];
  bool aval[MS];
#pragma unroll
  for (int s = 0; s < MS; ++s) {
    const int m = 16 * s + lrow;
    aval[s] = m < m_rows;
    const int mc = aval[s] ? m : m_rows - 1;
    ap[s] = aq + static_cast<int64_t>(mc) * k + quarter * 16;
    sap[s] = as + static_cast<int64_t>(mc) * groups;
  }

  v4f acc[R][MS];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < MS; ++s) acc[r][s] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int gi = 0; gi < gcnt; gi += U) {
    v8i wv[U][R];
    v8i bv[U][MS];
    float sa[U][MS];
    float sw[U][R];
    bool live[U];
    // Issue every load of the batch first. Groups past this wave's range are
    // clamped onto its last group (a cache hit) and weighted by zero.
#pragma unroll
    for (int u = 0; u < U; ++u) {
      live[u] = gi + u < gcnt;
      const int g = gbeg + (live[u] ? gi + u : gcnt - 1);
      const int64_t off = static_cast<int64_t>(g) * kGroup;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const v4u lo = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wp[r] + off));
        const v4u hi = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wp[r] + off + 64));
        wv[u][r] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sw[u][r] = swp[r][g];
      }
#pragma unroll
      for (int s = 0; s < MS; ++s) {
        v4u lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
        float scale = 0.f;
        if (aval[s]) {
          lo = *reinterpret_cast<const v4u*>(ap[s] + off);
          hi = *reinterpret_cast<const v4u*>(ap[s] + off + 64);
          scale = sap[s][g];
        }
        bv[u][s] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        sa[u][s] = scale;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int s = 0; s < MS; ++s) {
          const v4f p = mfma_16x16x128_e4m3(wv[u][r], bv[u][s]);
          const float sc = live[u] ? sa[u][s] * sw[u][r] : 0.f;
          acc[r][s][0] = fmaf(sc, p[0], acc[r][s][0]);
          acc[r][s][1] = fmaf(sc, p[1], acc[r][s][1]);
          acc[r][s][2] = fmaf(sc, p[2], acc[r][s][2]);
          acc[r][s][3] = fmaf(sc, p[3], acc[r][s][3]);
        }
      }
    }
  }

  // Split-K reduction: every wave parks its tiles in LDS, then the tiles are
  // shared out over the waves and summed in wave order 0..S-1.
  __shared__ v4f red[S][R * MS][64];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int s = 0; s < MS; ++s) red[wave][r * MS + s][lane] = acc[r][s];
  __syncthreads();

  for (int t = wave; t < R * MS; t += S) {
    v4f sum = red[0][t][lane];
#pragma unroll
    for (int w = 1; w < S; ++w) sum += red[w][t][lane];
    const int r = t / MS;
    const int s = t - r * MS;
    const int m = 16 * s + lrow;
    const int64_t col = n0 + 16 * r + 4 * quarter;  // first of 4 consecutive outputs
    if (m < m_rows) {
      unsigned short* dst = c + static_cast<int64_t>(m) * n + col;
      if ((n & 3) == 0 && col + 3 < n) {
        v2u packed;
        packed[0] = pack_bf16x2(sum[0], sum[1]);
        packed[1] = pack_bf16x2(sum[2], sum[3]);
        *reinterpret_cast<v2u*>(dst) = packed;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (col + i < n) dst[i] = static_cast<unsigned short>(pack_bf16x2(sum[i], 0.f) & 0xffffu);
      }
    }
  }
}

// Workgroups needed to cover n rows with R slabs of 16 rows each.
template <int R>
inline unsigned stream_grid(int64_t n) {
  return static_cast<unsigned>((n + 16 * R - 1) / (16 * R));
}

}  // namespace fp8bq

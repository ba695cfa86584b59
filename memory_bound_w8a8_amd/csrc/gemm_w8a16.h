// Weight-only block-FP8 GEMM (bf16 activation x block-FP8 weight) for up to
// 16 tokens, gfx950.
//
// Page 1 (SmartX blog, "Qwen3.8-27B performance optimisation"), section
// "single-stream optimisation": a W8A16 backend keeps the activation in 16
// bits and skips the per-call activation quantisation, which made it the
// faster choice at one stream (and the slower one at high concurrency, so it
// is offered for small M only). Same weights as the W8A8 path; the output is
//   C[m, n] = sum_g sw[n / 128, g] * sum_{k in g} A[m, k] * dec(W[n, k]).
//
// The weight side is the decode kernel's (gemm_rows.h): one workgroup per
// CU streams a balanced row range with whole-line loads, 8 waves split the
// K groups, each 16-row x 128-byte chunk goes through a per-wave
// XOR-swizzled LDS transpose into MFMA operand order (lane l: row l % 16,
// bytes 16 q .. 16 q + 15 and 64 + 16 q .. 64 + 16 q + 15 of the group,
// q = l / 16). Here those 32 fp8 bytes are converted to bf16 in registers
// (V_CVT_SCALEF32_PK_BF16_FP8 with scale 1: exact, every e4m3fn value is a
// bf16 value) and fed to four V_MFMA_F32_16X16X32_BF16, each covering 8
// bytes' worth of K; the activation operand of each is the matching 8 bf16
// of the lane's token, loaded directly (token lane % 16, clamped to M - 1).
// The four products chain through the MFMA accumulator, so one FMA per
// output applies the group's weight scale: acc += sw * group_sum.
#pragma once

#include "device_common.h"

namespace fp8bq {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// 8 e4m3fn codes (two dwords, byte i = element i) -> 8 bf16, exactly.
__device__ __forceinline__ v8bf e4m3x8_to_bf16(int d0, int d1) {
  const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, false);
  const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d0, 1.0f, true);
  const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, false);
  const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d1, 1.0f, true);
  return v8bf{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

template <int GMAX, int TILES, int PD>
__global__ __launch_bounds__(512) void gemm_w8a16_kernel(int m_rows, int64_t n, int64_t k, int64_t rows_per_wg,
                                                         const unsigned short* __restrict__ a,
                                                         const unsigned char* __restrict__ wq,
                                                         const float* __restrict__ ws,
                                                         unsigned short* __restrict__ c) {
  constexpr int S = 8;  // waves
  constexpr int CH = TILES * GMAX;
  constexpr int RING = PD + 1;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lrow = lane & 15;
  const int quarter = lane >> 4;
  const int groups = static_cast<int>(k >> 7);

  const int64_t r_begin = static_cast<int64_t>(blockIdx.x) * rows_per_wg;
  int64_t r_end = r_begin + rows_per_wg;
  r_end = r_end < n ? r_end : n;
  const int64_t r_last = r_end - 1;  // the grid never holds an empty range

  // This wave's contiguous range of K groups (gcnt may be < GMAX, even 0).
  const int per = groups / S;
  const int rem = groups - per * S;
  const int gbeg = wave * per + (wave < rem ? wave : rem);
  const int gcnt = per + (wave < rem ? 1 : 0);
  const int glast = gcnt > 0 ? gbeg + gcnt - 1 : 0;

  __shared__ v4u stage[S][2][128];
  __shared__ v4f red[S][TILES][64];

  // Activation operand of the lane's token for this wave's groups: bf16
  // elements 16 q .. 16 q + 15 and 64 + 16 q .. 64 + 16 q + 15 of each group
  // (four 16-byte pieces, one per MFMA). Groups past the wave's range
  // re-read its last group and get weight 0 (gw).
  const int tok = lrow < m_rows ? lrow : m_rows - 1;
  const unsigned short* arow = a + static_cast<int64_t>(tok) * k + 16 * quarter;
  v4u av[GMAX][4];
  float gw[GMAX];
#pragma unroll
  for (int u = 0; u < GMAX; ++u) {
    const bool live = u < gcnt;
    const int g = live ? gbeg + u : glast;
    const unsigned short* p = arow + static_cast<int64_t>(g) * kGroup;
    av[u][0] = *reinterpret_cast<const v4u*>(p);
    av[u][1] = *reinterpret_cast<const v4u*>(p + 8);
    av[u][2] = *reinterpret_cast<const v4u*>(p + 64);
    av[u][3] = *reinterpret_cast<const v4u*>(p + 72);
    gw[u] = live ? 1.f : 0.f;
  }

  // Weight chunks: rows 8 j + lane / 8 of each 16-row tile (j = 0, 1),
  // 16-byte piece lane % 8; rows past the range clamped onto its last row.
  const int lr8 = lane >> 3;
  const int piece = lane & 7;
  v8i wv[RING];
  float sw[RING];
  auto load_chunk = [&](int ci, int slot) {
    const int t = ci / GMAX;
    const int u = ci - t * GMAX;
    const int g = u < gcnt ? gbeg + u : glast;
    const int64_t off = static_cast<int64_t>(g) * kGroup + piece * 16;
    int64_t row0 = r_begin + 16 * t + lr8;
    int64_t row1 = row0 + 8;
    row0 = row0 < r_end ? row0 : r_last;
    row1 = row1 < r_end ? row1 : r_last;
    const v4u lo = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wq + row0 * k + off));
    const v4u hi = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wq + row1 * k + off));
    wv[slot] = join8(lo, hi);
    int64_t quad = r_begin + 16 * t + 4 * quarter;
    quad = quad < r_end ? quad : r_last;
    sw[slot] = ws[(quad >> 7) * groups + g];
  };

  // Pieces this lane loaded (rows lr8 and lr8 + 8, piece `piece`) -> the
  // operand bytes of row lrow (pieces quarter and quarter + 4).
  auto transpose = [&](const v8i& raw, int st) -> v8i {
    v4u* slot = stage[wave][st];
    slot[8 * lr8 + (piece ^ lr8)] = v4u{(unsigned)raw[0], (unsigned)raw[1], (unsigned)raw[2], (unsigned)raw[3]};
    slot[8 * (lr8 + 8) + (piece ^ lr8)] = v4u{(unsigned)raw[4], (unsigned)raw[5], (unsigned)raw[6], (unsigned)raw[7]};
    __builtin_amdgcn_wave_barrier();
    const int x = lrow & 7;
    const v4u lo = slot[8 * lrow + (quarter ^ x)];
    const v4u hi = slot[8 * lrow + ((quarter + 4) ^ x)];
    __builtin_amdgcn_wave_barrier();
    return join8(lo, hi);
  };

  v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ci = 0; ci < PD && ci < CH; ++ci) load_chunk(ci, ci % RING);
#pragma unroll
  for (int ci = 0; ci < CH; ++ci) {
    const int t = ci / GMAX;
    const int u = ci - t * GMAX;
    if (ci + PD < CH) load_chunk(ci + PD, (ci + PD) % RING);
    if (u == 0) acc = v4f{0.f, 0.f, 0.f, 0.f};
    const v8i wop = transpose(wv[ci % RING], ci & 1);
    v4f p = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(wop[2 * j], wop[2 * j + 1]),
                                                  __builtin_bit_cast(v8bf, av[u][j]), p, 0, 0, 0);
    // lane: rows 16 t + 4 quarter + i (one aligned quad, one weight block),
    // token lrow
    const float sc = sw[ci % RING] * gw[u];
    acc[0] = fmaf(sc, p[0], acc[0]);
    acc[1] = fmaf(sc, p[1], acc[1]);
    acc[2] = fmaf(sc, p[2], acc[2]);
    acc[3] = fmaf(sc, p[3], acc[3]);
    if (u == GMAX - 1) red[wave][t][lane] = acc;
  }
  __syncthreads();

  // Sum the S partials of every tile in wave order and store.
#pragma unroll
  for (int t0 = 0; t0 < TILES; t0 += S) {
    const int t = t0 + wave;
    if (t < TILES) {
      v4f sum = red[0][t][lane];
#pragma unroll
      for (int w = 1; w < S; ++w) sum += red[w][t][lane];
      const int m = lrow;
      const int64_t col = r_begin + 16 * t + 4 * quarter;  // first of 4 consecutive outputs
      if (m < m_rows && col < r_end) {
        unsigned short* dst = c + static_cast<int64_t>(m) * n + col;
        if ((n & 3) == 0 && col + 3 < r_end) {
          v2u packed;
          packed[0] = pack_bf16x2(sum[0], sum[1]);
          packed[1] = pack_bf16x2(sum[2], sum[3]);
          *reinterpret_cast<v2u*>(dst) = packed;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (col + i < r_end) dst[i] = static_cast<unsigned short>(pack_bf16x2(sum[i], 0.f) & 0xffffu);
        }
      }
    }
  }
}

}  // namespace fp8bq

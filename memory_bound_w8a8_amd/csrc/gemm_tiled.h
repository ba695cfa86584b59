// LDS-tiled FP8 MFMA block-scaled GEMM for large M (batches, prefill),
// gfx950.
//
// At M in the thousands (page 2, ownding.com L20 report, section 4.2: a
// 3,465-token prompt; section 8: prefill forced onto an M=1 config regressed)
// the op is a dense contraction far above the FP8 ridge, so it runs on the
// matrix cores at the largest register tile that fits.
//
// Tiling. A workgroup of WM x WN waves computes a BM x BN tile of C (tokens x
// weight rows); each wave owns a (BM / WM) x (BN / WN) sub-tile held in fp32
// registers. K is walked one 128-wide scale group per step:
//   1. the step's A slice (BM x 128 codes) and W slice (BN x 128 codes) are
//      copied global -> LDS with direct-to-LDS loads (no registers), STAGES
//      deep: steps g + 1 .. g + STAGES - 1 are in flight while step g
//      computes (three stages where they fit in the 160 KB of LDS, two for
//      the 192- and 256-token tiles); the copies go out spread over a
//      sub-tile's MFMAs rather than in one burst. The BM activation scales
//      come 8 groups at a time (a BM x 8 block every 8 steps, 8 rows per
//      copy instruction) into a two-buffer array of their own;
//   2. each wave reads its W fragments once per step and streams its token
//      fragments; one 16x16x128 FP8 MFMA per 16 x 16 sub-tile gives the
//      group's exact products into a fresh accumulator (weight rows first
//      operand, tokens second);
//   3. acc += (A_scale[m, g] * W_scale[n / 128, g]) * mfma in fp32: one FMA
//      per output per group, which the VALU issues while the matrix core runs
//      the next MFMAs (4 FMAs per 32-cycle MFMA).
// LDS layout: each tile row is 128 bytes, its 16-byte chunk c stored at
// position c ^ (row & 7). A direct-to-LDS load writes lane i's 16 bytes at
// base + 16 i, so lane i of the load covering rows 8 q .. 8 q + 7 fetches
// chunk (i % 8) ^ (row & 7) of row 8 q + i / 8; the fragment reads (8 lanes =
// 8 rows, one chunk each) then hit 8 distinct 16-byte bank groups.
// Workgroups are mapped to tiles XCD by XCD (hardware places workgroup b on
// XCD b % 8): each XCD gets a contiguous run of the tile order, which walks
// bands of 8 token tiles with the token tile fastest, so the ~32 tiles
// resident on one XCD form a compact block sharing A and W slices in L2.
// Rows past M or N are clamped onto the last valid row for loading and masked
// at the store.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "wave_prio.h"

namespace fp8bq {

typedef __attribute__((address_space(3))) const void lds_void;

// Direct global -> LDS copies (lane i's bytes land at base + size * i; the
// LDS base goes through M0 and must be uniform across the wave, which
// readfirstlane states to the compiler). Issued as
// inline assembly so that the compiler does not track them: it cannot tell
// which stage a copy writes and would otherwise wait for every copy in
// flight before each LDS read. The kernel orders them itself (explicit
// vmcnt wait + barrier before a stage is read or rewritten).
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>((const lds_void*)p));
}
// Global address = uniform 64-bit base (scalar registers) + per-lane 32-bit
// offset, so a copy needs one vector register per lane and no 64-bit
// address arithmetic. `sbase` must be the same in every lane; uniform()
// states that to the compiler where it cannot prove it.
__device__ __forceinline__ const void* uniform(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v & 0xffffffffu)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(v >> 32)));
  return reinterpret_cast<const void*>(lo | (hi << 32));
}
__device__ __forceinline__ void dma16(const void* sbase, unsigned voff, void* lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_base)))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* sbase, unsigned voff, void* lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase),
               "s"(__builtin_amdgcn_readfirstlane(lds_addr(lds_base)))
               : "memory", "m0");
}

template <int BM, int BN, int WM, int WN, int STAGES>
struct TiledKernel {
  static constexpr int kWaves = WM * WN;
  static constexpr int kTM = BM / WM;  // tokens per wave
  static constexpr int kTN = BN / WN;  // weight rows per wave
  static constexpr int kJ = kTM / 16;  // token sub-tiles per wave
  static constexpr int kI = kTN / 16;  // weight-row sub-tiles per wave
  // A codes, then W codes (the activation scales sit in a separate
  // two-buffer array, 8 groups at a time)
  static constexpr int kStageBytes = (BM + BN) * 128;
  static constexpr int kScaleBytes = 2 * BM * 8 * 4;
  static constexpr int kLdsBytes = STAGES * kStageBytes + kScaleBytes;
  // direct-to-LDS loads one wave issues per K step (plus kScaleLoadsPerWave
  // every 8 steps)
  static constexpr int kTileLoadsPerWave = BM / 8 / kWaves + BN / 8 / kWaves;
  static constexpr int kScaleLoadsPerWave = BM / 8 / kWaves;
};

// Wait until at most N of this wave's vector-memory operations are
// outstanding, then barrier the workgroup. Written out because
// __syncthreads() carries a workgroup memory fence, which would also wait
// for the tile copies still in flight (direct-to-LDS loads count as LDS
// stores) and so drain the pipeline at every step. The memory clobber keeps
// the compiler from moving memory operations across it. Ordering this
// relies on: every LDS read of a step is consumed by that step's MFMAs, so
// it has completed before the barrier.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Tile index of workgroup b: XCD-contiguous runs of the tile space.
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t tiles) {
  const int64_t x = b & 7, s = b >> 3;
  const int64_t per = tiles >> 3, rem = tiles & 7;
  const int64_t start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return start + s;
}

// Tile t -> (token tile, weight tile) in bands of `band` token tiles: inside
// a band the token tile runs fastest, so any run of consecutive tiles covers
// a compact block (e.g. 32 tiles = 8 token x 4 weight tiles) whose A and W
// slices are shared through L2. A last, narrower band takes the remainder.
__device__ __forceinline__ void band_tile(int64_t t, int64_t m_tiles, int64_t n_tiles, int64_t band, int64_t* tm,
                                          int64_t* tn) {
  const int64_t full_bands = m_tiles / band;
  const int64_t in_full = full_bands * band * n_tiles;
  if (t < in_full) {
    const int64_t b = t / (band * n_tiles);
    const int64_t w = t - b * band * n_tiles;
    *tn = w / band;
    *tm = b * band + (w - *tn * band);
  } else {
    const int64_t last = m_tiles - full_bands * band;  // > 0 whenever this branch runs
    const int64_t w = t - in_full;
    *tn = w / last;
    *tm = full_bands * band + (w - *tn * last);
  }
}

template <int BM, int BN, int WM, int WN, int STAGES>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tiled_kernel(int64_t m_rows, int64_t n, int64_t k, int split,
                                                                  const unsigned char* __restrict__ aq,
                                                                  const float* __restrict__ as,
                                                                  const unsigned char* __restrict__ wq,
                                                                  const float* __restrict__ ws,
                                                                  unsigned short* __restrict__ c,
                                                                  float* __restrict__ part) {
  using KC = TiledKernel<BM, BN, WM, WN, STAGES>;
  constexpr int WAVES = KC::kWaves;
  constexpr int TM = KC::kTM, TN = KC::kTN, J = KC::kJ, I = KC::kI;
  static_assert(TN <= 128 && 128 % TN == 0, "a wave's weight rows must sit in one 128-row scale block");
  static_assert(BM % (8 * WAVES) == 0 && BN % (8 * WAVES) == 0, "8-row load chunks spread over the waves");
  static_assert(BM % 64 == 0 && BM <= 64 * WAVES, "scales: one dword per token, 64 tokens per wave");
  static_assert(STAGES == 2 || STAGES == 3, "STAGES");

  // One LDS object per stage: the compiler then sees that the copies into
  // one stage cannot alias the fragment reads of another, and does not wait
  // for the in-flight copies before every read.
  __shared__ __attribute__((aligned(16))) unsigned char lds0[KC::kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[KC::kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds2[STAGES > 2 ? KC::kStageBytes : 16];
  // token scales of 8 groups at a time, [token][8], two buffers (groups
  // 8c .. 8c + 7 of this workgroup's K range in buffer c % 2)
  __shared__ __attribute__((aligned(16))) float lds_scales[2 * BM * 8];

  const int lane = threadIdx.x & 63;
  // wave index as a provably uniform value: per-wave pointers (the weight
  // scale row) then live in scalar registers and their loads go through the
  // scalar cache, outside the in-order vector-memory counter that tracks the
  // in-flight tile copies
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 15;
  const int quarter = lane >> 4;
  const int wave_m = wave % WM;
  const int wave_n = wave / WM;
  const int64_t gstride = k >> 7;  // scale groups per row of the scale arrays

  // Workgroup -> (tile, K part): with split > 1 the grid is tiles x split
  // workgroups, part s of a tile summing groups [G s / split, G (s + 1) /
  // split) into an fp32 partial tile of `part` (split x M x N); the parts
  // of one K range run next to each other, so an XCD's run of workgroups
  // shares A and W slices as in the unsplit grid.
  const int64_t m_tiles = (m_rows + BM - 1) / BM;
  const int64_t n_tiles = (n + BN - 1) / BN;
  const int64_t n_units = m_tiles * n_tiles;
  const int64_t unit = xcd_tile(blockIdx.x, n_units * split);
  const int64_t tile = unit % n_units;
  const int64_t ks = unit / n_units;
  const int64_t g_lo = gstride * ks / split;
  const int64_t groups = gstride * (ks + 1) / split - g_lo;  // this workgroup's K steps (>= 1)
  int64_t tm, tn;
  band_tile(tile, m_tiles, n_tiles, 8, &tm, &tn);
  const int64_t m0 = tm * BM;
  const int64_t n0 = tn * BN;

  // ---- global -> LDS copy plan (per wave: chunks of 8 rows x 128 bytes) ----
  constexpr int A_CHUNKS = BM / 8 / WAVES;  // per wave
  constexpr int W_CHUNKS = BN / 8 / WAVES;
  const int cr = lane >> 3;                 // row within the 8-row chunk
  // Per-lane 32-bit offsets from the tile's first row (which sits in scalar
  // registers); a tile spans at most 256 rows of K bytes.
  const unsigned char* a_base = aq + m0 * k + g_lo * kGroup;
  const unsigned char* w_base = wq + n0 * k + g_lo * kGroup;
  unsigned a_off[A_CHUNKS];
  unsigned w_off[W_CHUNKS];
#pragma unroll
  for (int q = 0; q < A_CHUNKS; ++q) {
    const int r = 8 * (wave + WAVES * q) + cr;  // tile row
    const int64_t row = m0 + r < m_rows ? r : m_rows - 1 - m0;
    a_off[q] = static_cast<unsigned>(row * k + 16 * ((lane & 7) ^ (r & 7)));
  }
#pragma unroll
  for (int q = 0; q < W_CHUNKS; ++q) {
    const int r = 8 * (wave + WAVES * q) + cr;
    const int64_t row = n0 + r < n ? r : n - 1 - n0;
    w_off[q] = static_cast<unsigned>(row * k + 16 * ((lane & 7) ^ (r & 7)));
  }
  // Activation scales of the tile's tokens: every 8 groups the BM x 8 block,
  // one dword copy per lane (lane l: token 8 u + l / 8, group 8 c + l % 8 of
  // the wave's u-th 8-token chunk), so a copy touches 8 rows' lines rather
  // than the 64 of a per-group gather.
  constexpr int S_CHUNKS = KC::kScaleLoadsPerWave;
  const float* sa_base = as + m0 * gstride;
  int64_t wblock = n0 + TN * wave_n;
  wblock = wblock < n ? wblock : n - 1;
  const float* sw_src = ws + (wblock >> 7) * gstride + g_lo;

  auto stage_base = [&](auto st) -> unsigned char* {
    if constexpr (decltype(st)::value == 0) return lds0;
    else if constexpr (decltype(st)::value == 1) return lds1;
    else return lds2;
  };

  // The copies of group g into stage st: this wave's 8-row chunks c = 0 ..
  // A_CHUNKS - 1 of the token tile, then A_CHUNKS .. CHUNKS - 1 of the
  // weight tile; every 8 groups also the scales.
  constexpr int CHUNKS = A_CHUNKS + W_CHUNKS;
  constexpr bool kSpread = I * J >= 8;
  auto issue_chunk = [&](int64_t g, auto st, int c) {
    unsigned char* base = stage_base(st);
    if (c < A_CHUNKS)
      dma16(uniform(a_base + g * kGroup), a_off[c], base + 1024 * (wave + WAVES * c));
    else
      dma16(uniform(w_base + g * kGroup), w_off[c - A_CHUNKS], base + BM * 128 + 1024 * (wave + WAVES * (c - A_CHUNKS)));
  };
  auto issue_scales = [&](int64_t g) {
    if ((g & 7) == 0) {  // the scales of groups g .. g + 7
      const int64_t col = g_lo + g + (lane & 7) < gstride ? g_lo + g + (lane & 7) : gstride - 1;
#pragma unroll
      for (int q = 0; q < S_CHUNKS; ++q) {
        const int u = wave + WAVES * q;
        const int r = 8 * u + cr;
        const int64_t row = m0 + r < m_rows ? r : m_rows - 1 - m0;
        dma4(uniform(sa_base), static_cast<unsigned>(4 * (row * gstride + col)),
             reinterpret_cast<unsigned char*>(lds_scales) + 4 * BM * 8 * ((g >> 3) & 1) + 256 * u);
      }
    }
  };
  auto issue = [&](int64_t g, auto st) {
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) issue_chunk(g, st, c);
    issue_scales(g);
  };

  // Fragment read: lane's row `r` of a 128-byte-row tile, chunks quarter and
  // quarter + 4 (un-swizzled through c ^ (r & 7)).
  auto frag = [&](const unsigned char* base, int r) -> v8i {
    const int x = r & 7;
    const v4u lo = *reinterpret_cast<const v4u*>(base + r * 128 + 16 * (quarter ^ x));
    const v4u hi = *reinterpret_cast<const v4u*>(base + r * 128 + 16 * ((quarter + 4) ^ x));
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  v4f acc[I][J];
#pragma unroll
  for (int i = 0; i < I; ++i)
#pragma unroll
    for (int j = 0; j < J; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Pipeline: step g computes from stage g % STAGES while the copies of the
  // next STAGES - 1 steps are in flight. Copies are issued unconditionally
  // (steps past the end re-copy the last step into a stage that is never
  // read again, and its scales unchanged), so the wait after a step is
  // constant but for the scale copies: step g + 1 must have landed, the
  // STAGES - 2 later ones (with 8-group scale copies when their group is a
  // multiple of 8) may not.
  constexpr int kInFlight = (STAGES - 2) * KC::kTileLoadsPerWave;
  constexpr int kInFlightScales = kInFlight + (STAGES - 2) * S_CHUNKS;
  auto wait_step = [&](bool scales_in_flight) {
    if (STAGES > 2 && scales_in_flight) wait_vm_barrier<kInFlightScales>();
    else wait_vm_barrier<kInFlight>();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  issue(0, S0{});
  if constexpr (STAGES == 3) issue(groups > 1 ? 1 : 0, S1{});
  wait_step(false);

  auto step = [&](int64_t g, auto st) {
    constexpr int cur = decltype(st)::value;
    constexpr int nxt = (cur + STAGES - 1) % STAGES;  // stage of step g + STAGES - 1
    using SN = std::integral_constant<int, nxt>;
    const int64_t gn = g + STAGES - 1 < groups ? g + STAGES - 1 : groups - 1;
    // The tile chunks now where a wave's step is short (4 MFMAs: 64 x 64
    // tiles), else spread over sub-tile 0's MFMAs, and the scales: a burst of
    // copies at the step's start holds up the MFMAs (M = 512..1024 on the
    // logged shapes: 128 x 128 and 128 x 256 tiles 6-10% faster; 64 x 64
    // tiles 9-11% slower spread).
    if constexpr (!kSpread) {
#pragma unroll
      for (int c = 0; c < CHUNKS; ++c) issue_chunk(gn, SN{}, c);
    }
    issue_scales(gn);

    const unsigned char* la = stage_base(st);
    const unsigned char* lw = la + BM * 128;
    const float* ls = lds_scales + BM * 8 * ((g >> 3) & 1) + (g & 7);
    const float sw = sw_src[g];

    v8i wf[I];
#pragma unroll
    for (int i = 0; i < I; ++i) wf[i] = frag(lw, TN * wave_n + 16 * i + lrow);

    // Token sub-tile j's MFMAs are issued before sub-tile j - 1's scale FMAs,
    // so no FMA waits on the MFMA just issued.
    v4f p_prev[I];
    float sc_prev = 0.f;
    v8i af = frag(la, TM * wave_m + lrow);
    float sc = ls[8 * (TM * wave_m + lrow)] * sw;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      v8i af_next = af;
      float sc_next = sc;
      if (j + 1 < J) {
        const int tr = TM * wave_m + 16 * (j + 1) + lrow;
        af_next = frag(la, tr);
        sc_next = ls[8 * tr] * sw;
      }
      // MFMA (i, j), then the scale FMAs of (i, j - 1), whose MFMA was issued
      // I MFMAs earlier: at most I + 1 fresh results are live.
      v4f p_cur[I];
#pragma unroll
      for (int i = 0; i < I; ++i) {
        p_cur[i] = mfma_16x16x128_e4m3(wf[i], af);
        if (kSpread && j == 0) {
#pragma unroll
          for (int c = i * CHUNKS / I; c < (i + 1) * CHUNKS / I; ++c) issue_chunk(gn, SN{}, c);
        }
        if (j > 0) {
          acc[i][j - 1][0] = fmaf(sc_prev, p_prev[i][0], acc[i][j - 1][0]);
          acc[i][j - 1][1] = fmaf(sc_prev, p_prev[i][1], acc[i][j - 1][1]);
          acc[i][j - 1][2] = fmaf(sc_prev, p_prev[i][2], acc[i][j - 1][2]);
          acc[i][j - 1][3] = fmaf(sc_prev, p_prev[i][3], acc[i][j - 1][3]);
          // Pin the update here: left free, the compiler sinks every FMA of
          // the step below the step's closing barrier, where both waves of
          // a SIMD run them at once while the matrix core idles.
          asm volatile("" : "+v"(acc[i][j - 1]));
        }
        // Keep this order: left alone, the compiler issues all MFMAs of the
        // step first and all FMAs afterwards, so that the matrix core and
        // the VALU never overlap.
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < I; ++i) p_prev[i] = p_cur[i];
      sc_prev = sc;
      af = af_next;
      sc = sc_next;
    }
#pragma unroll
    for (int i = 0; i < I; ++i) {
      acc[i][J - 1][0] = fmaf(sc_prev, p_prev[i][0], acc[i][J - 1][0]);
      acc[i][J - 1][1] = fmaf(sc_prev, p_prev[i][1], acc[i][J - 1][1]);
      acc[i][J - 1][2] = fmaf(sc_prev, p_prev[i][2], acc[i][J - 1][2]);
      acc[i][J - 1][3] = fmaf(sc_prev, p_prev[i][3], acc[i][J - 1][3]);
      asm volatile("" : "+v"(acc[i][J - 1]));
    }

    // Step g + 1's copies must have landed, and every wave must be done
    // reading this stage before the next step's copies overwrite it.
    wait_step((gn & 7) == 0);
  };

  for (int64_t g = 0; g < groups; g += STAGES) {
    step(g, S0{});
    if (g + 1 < groups) step(g + 1, S1{});
    if constexpr (STAGES == 3) {
      if (g + 2 < groups) step(g + 2, S2{});
    }
  }
  // The copies issued past the last step must land before this workgroup's
  // LDS can be handed to another one.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue: lane holds, per sub-tile, weight rows 4 (l / 16) .. +3 of token
  // l % 16: four consecutive outputs in C's row (or in the partial tile's).
  if (part != nullptr) {
    float* pdst = part + ks * m_rows * n;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int64_t m = m0 + TM * wave_m + 16 * j + lrow;
      if (m >= m_rows) continue;
#pragma unroll
      for (int i = 0; i < I; ++i) {
        const int64_t col = n0 + TN * wave_n + 16 * i + 4 * quarter;
        float* dst = pdst + m * n + col;
        const v4f v = acc[i][j];
        if ((n & 3) == 0 && col + 3 < n) {
          *reinterpret_cast<v4f*>(dst) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < n) dst[e] = v[e];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t m = m0 + TM * wave_m + 16 * j + lrow;
    if (m >= m_rows) continue;
#pragma unroll
    for (int i = 0; i < I; ++i) {
      const int64_t col = n0 + TN * wave_n + 16 * i + 4 * quarter;
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

// Two-stage variant for the tiles whose two LDS stages take most of the
// 160 KB (192 x 256 and 256 x 256 tokens x weight rows, 8 waves). Same
// tiling, copies, swizzle and per-group summation order as
// gemm_tiled_kernel (results are bitwise equal), with the K step arranged
// around what its profile showed to be the cost: LDS latency in front of the
// MFMAs.
//  - The token fragment of sub-tile j + 1 is read while sub-tile j's MFMAs
//    run (registers freed for it: one DMA lane offset instead of one per
//    chunk, the chunk bases in scalar registers; weight scales fetched 64
//    groups at a time with a vector load and picked per step with
//    v_readlane, so no scalar load shares the LDS wait counter in the loop).
//  - The last token sub-tile's MFMAs are deferred across the step barrier:
//    after the barrier a wave issues the next step's copies and fragment
//    reads, then those MFMAs (operands already in registers), which cover
//    the latency of the new reads; each weight fragment is refilled right
//    after the MFMA that last uses it. Where no row is clamped, half of
//    step g + 2's copies go out there and the other half with step g + 1's
//    first sub-tile (the clamped instance has no registers left for the
//    second set of lane offsets and issues them all after the barrier).
//  - The two waves that share a SIMD would otherwise take the matrix core in
//    age order (a per-wave timestamp trace showed the older wave finishing
//    its K step about 1,000 cycles before the younger one, which then ran
//    alone); the wave's priority steps down from 3 to 0 over the step's
//    sub-tiles, so whichever wave is behind in the step is preferred, and
//    the barrier resets it (M = 3465: 2-3% less time on (17408, 5120) and
//    (5120, 8704); issuing the copies two sub-tiles after the barrier
//    instead helped the first and cost the second 5%).
//  - CLAMP = false (every row of the tile exists: M >= BM, N a multiple of
//    BN): the last token tile is shifted back to end at row M - 1 and stores
//    only the rows the previous tile does not, so no row is clamped and one
//    lane offset serves every copy. CLAMP = true keeps the per-chunk clamped
//    offsets of gemm_tiled_kernel.
//  - A launch covers the tiles t0 .. t0 + gridDim.x / split - 1 of the grid of
//    BM x (split BN) tiles, each as `split` workgroups of BN columns (split
//    = 1: whole tiles; split = 2: the two column halves of a tile, so that a
//    last, partly filled round of whole tiles can run as one round of
//    halves, each output still summed over its groups in the same order).
template <int BM, int BN, int WM, int WN, bool CLAMP>
__global__ __launch_bounds__(64 * WM * WN) void gemm_tiled2_kernel(int64_t m_rows, int64_t n, int64_t k, int64_t t0,
                                                                   int split, const unsigned char* __restrict__ aq,
                                                                   const float* __restrict__ as,
                                                                   const unsigned char* __restrict__ wq,
                                                                   const float* __restrict__ ws,
                                                                   unsigned short* __restrict__ c) {
  constexpr int WAVES = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN, J = TM / 16, I = TN / 16;
  static_assert(TN <= 128 && 128 % TN == 0, "a wave's weight rows must sit in one 128-row scale block");
  static_assert(BM % (8 * WAVES) == 0 && BN % (8 * WAVES) == 0, "8-row load chunks spread over the waves");
  static_assert(BM % 64 == 0 && BM <= 64 * WAVES, "scales: one dword per token, 64 tokens per wave");
  static_assert(J >= 2, "at least two token sub-tiles per wave");
  constexpr int kStageBytes = (BM + BN) * 128;
  __shared__ __attribute__((aligned(16))) unsigned char lds0[kStageBytes];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[kStageBytes];
  // token scales of 8 groups at a time, [token][8], two buffers (groups
  // 8c .. 8c + 7 in buffer c % 2)
  __shared__ __attribute__((aligned(16))) float lds_scales[2 * BM * 8];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 15;
  const int quarter = lane >> 4;
  const int wave_m = wave % WM;
  const int wave_n = wave / WM;
  const int64_t groups = k >> 7;

  const int64_t m_tiles = (m_rows + BM - 1) / BM;
  const int64_t n_tiles = (n + split * BN - 1) / (split * BN);  // tiles of split * BN columns
  int64_t tm, tn;
  const int64_t u = xcd_tile(blockIdx.x, gridDim.x);
  band_tile(t0 + u / split, m_tiles, n_tiles, 8, &tm, &tn);
  const int64_t m_own = tm * BM;  // first token row this tile stores
  int64_t m0 = m_own;
  if (!CLAMP && m0 + BM > m_rows) m0 = m_rows - BM;  // last token tile shifted back: every row valid
  const int64_t n0 = (tn * split + u % split) * BN;
  if (n0 >= n) return;  // a column half wholly past N (whole workgroup, before any barrier)

  constexpr int A_CHUNKS = BM / 8 / WAVES;
  constexpr int W_CHUNKS = BN / 8 / WAVES;
  const int cr = lane >> 3;
  const unsigned char* a_base = aq + m0 * k;
  const unsigned char* w_base = wq + n0 * k;
  // DMA lane offsets. Without clamping every chunk q uses the same lane
  // offset (row cr of its 8-row chunk, 16-byte piece (lane % 8) ^ cr); the
  // chunk's first row goes into the scalar base.
  unsigned a_off[CLAMP ? A_CHUNKS : 1];
  unsigned w_off[CLAMP ? W_CHUNKS : 1];
  if constexpr (CLAMP) {
#pragma unroll
    for (int q = 0; q < A_CHUNKS; ++q) {
      const int r = 8 * (wave + WAVES * q) + cr;
      const int64_t row = m0 + r < m_rows ? r : m_rows - 1 - m0;
      a_off[q] = static_cast<unsigned>(row * k + 16 * ((lane & 7) ^ (r & 7)));
    }
#pragma unroll
    for (int q = 0; q < W_CHUNKS; ++q) {
      const int r = 8 * (wave + WAVES * q) + cr;
      const int64_t row = n0 + r < n ? r : n - 1 - n0;
      w_off[q] = static_cast<unsigned>(row * k + 16 * ((lane & 7) ^ (r & 7)));
    }
  } else {
    a_off[0] = static_cast<unsigned>(cr * k + 16 * ((lane & 7) ^ cr));
    w_off[0] = a_off[0];
  }
  // Token scales: every 8 groups, the tile's BM x 8 block, one dword copy
  // per lane (lane l: token 8 u + l / 8, group 8 c + l % 8 of the wave's
  // u-th 8-token chunk), so a copy touches 8 rows' lines instead of the 64
  // of a per-group gather (which cost 4% of the K step).
  constexpr int S_CHUNKS = BM / 8 / WAVES;
  const float* sa_base = as + m0 * groups;
  int64_t wblock = n0 + TN * wave_n;
  if (CLAMP) wblock = wblock < n ? wblock : n - 1;
  const float* sw_src = ws + (wblock >> 7) * groups;
  // The wave's weight scales, 64 groups at a time: lane l holds group
  // 64 c + l (a vector load; steps read theirs with v_readlane, so no
  // scalar load shares the LDS wait counter inside the K loop).
  auto sw_chunk = [&](int64_t g0) -> float {
    const int64_t gl = g0 + lane < groups ? g0 + lane : groups - 1;
    float v = sw_src[gl];
    asm volatile("" : "+v"(v));  // a per-lane vector value, not a scalar load
    return v;
  };

  // Without clamping: the first row of every 8-row chunk this wave copies,
  // as uniform pointers computed once (the per-step address is then one
  // scalar add).
  const unsigned char* a_chunk[CLAMP ? 1 : A_CHUNKS];
  const unsigned char* w_chunk[CLAMP ? 1 : W_CHUNKS];
  if constexpr (!CLAMP) {
#pragma unroll
    for (int q = 0; q < A_CHUNKS; ++q)
      a_chunk[q] = static_cast<const unsigned char*>(uniform(a_base + static_cast<int64_t>(8 * (wave + WAVES * q)) * k));
#pragma unroll
    for (int q = 0; q < W_CHUNKS; ++q)
      w_chunk[q] = static_cast<const unsigned char*>(uniform(w_base + static_cast<int64_t>(8 * (wave + WAVES * q)) * k));
  }

  auto stage_base = [&](auto st) -> unsigned char* {
    if constexpr (decltype(st)::value == 0) return lds0;
    else return lds1;
  };
  // The copies of group g into stage st: this wave's 8-row chunks c = 0 ..
  // A_CHUNKS - 1 of the token tile, then A_CHUNKS .. CHUNKS - 1 of the
  // weight tile, and (waves 0 .. BM / 64 - 1) the token scales.
  constexpr int CHUNKS = A_CHUNKS + W_CHUNKS;
  constexpr bool kSplitCopies = !CLAMP;
  constexpr int HALF = kSplitCopies ? CHUNKS / 2 : CHUNKS;  // chunks issued with the deferred sub-tile
  auto issue_chunk = [&](int64_t g, auto st, int c) {
    unsigned char* base = stage_base(st);
    if (c < A_CHUNKS) {
      if constexpr (CLAMP)
        dma16(uniform(a_base + g * kGroup), a_off[c], base + 1024 * (wave + WAVES * c));
      else
        dma16(a_chunk[c] + g * kGroup, a_off[0], base + 1024 * (wave + WAVES * c));
    } else {
      const int q = c - A_CHUNKS;
      if constexpr (CLAMP)
        dma16(uniform(w_base + g * kGroup), w_off[q], base + BM * 128 + 1024 * (wave + WAVES * q));
      else
        dma16(w_chunk[q] + g * kGroup, w_off[0], base + BM * 128 + 1024 * (wave + WAVES * q));
    }
  };
  auto issue_scales = [&](int64_t g) {  // g a multiple of 8
    const int64_t col = g + (lane & 7) < groups ? g + (lane & 7) : groups - 1;
#pragma unroll
    for (int q = 0; q < S_CHUNKS; ++q) {
      const int u = wave + WAVES * q;
      const int r = 8 * u + cr;
      const int64_t row = (!CLAMP || m0 + r < m_rows) ? r : m_rows - 1 - m0;
      dma4(uniform(sa_base), static_cast<unsigned>(4 * (row * groups + col)),
           reinterpret_cast<unsigned char*>(lds_scales) + 4 * BM * 8 * ((g >> 3) & 1) + 256 * u);
    }
  };
  auto issue = [&](int64_t g, auto st) {
#pragma unroll
    for (int c = 0; c < CHUNKS; ++c) issue_chunk(g, st, c);
    if ((g & 7) == 0) issue_scales(g);
  };
  auto frag = [&](const unsigned char* base, int r) -> v8i {
    const int x = r & 7;
    const v4u lo = *reinterpret_cast<const v4u*>(base + r * 128 + 16 * (quarter ^ x));
    const v4u hi = *reinterpret_cast<const v4u*>(base + r * 128 + 16 * ((quarter + 4) ^ x));
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto a_frag = [&](auto st, int j) -> v8i { return frag(stage_base(st), TM * wave_m + 16 * j + lrow); };
  auto a_scale = [&](int64_t g, int j) -> float {
    return lds_scales[BM * 8 * ((g >> 3) & 1) + 8 * (TM * wave_m + 16 * j + lrow) + (g & 7)];
  };
  auto w_frag = [&](auto st, int i) -> v8i { return frag(stage_base(st) + BM * 128, TN * wave_n + 16 * i + lrow); };

  v4f acc[I][J];
#pragma unroll
  for (int i = 0; i < I; ++i)
#pragma unroll
    for (int j = 0; j < J; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;

  // Prologue: step 0's tiles land, then step 1's copies go out and step 0's
  // fragments come in.
  issue(0, S0{});
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  issue(groups > 1 ? 1 : 0, S1{});
  v8i wf[I];
#pragma unroll
  for (int i = 0; i < I; ++i) wf[i] = w_frag(S0{}, i);
  v8i af = a_frag(S0{}, 0);
  float sa = a_scale(0, 0);
  float sw_lanes = sw_chunk(0);
  float sw = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sw_lanes), 0));
  // results of the previous token sub-tile awaiting their scale FMA (zeros
  // before the first: adding 0 * 0 leaves the +0 running sums unchanged)
  v4f p_prev[I];
#pragma unroll
  for (int i = 0; i < I; ++i) p_prev[i] = v4f{0.f, 0.f, 0.f, 0.f};
  float sc_prev = 0.f;

  // MFMAs of token sub-tile j (fragment af, scale sc) while the FMAs of the
  // previous sub-tile's results (into acc[.][jp]) retire one per MFMA;
  // `between(i)` runs after MFMA i (used to refill the weight fragments).
  auto mfma_row = [&](int jp, float sc, auto between) {
    v4f p_cur[I];
#pragma unroll
    for (int i = 0; i < I; ++i) {
      p_cur[i] = mfma_16x16x128_e4m3(wf[i], af);
      acc[i][jp][0] = fmaf(sc_prev, p_prev[i][0], acc[i][jp][0]);
      acc[i][jp][1] = fmaf(sc_prev, p_prev[i][1], acc[i][jp][1]);
      acc[i][jp][2] = fmaf(sc_prev, p_prev[i][2], acc[i][jp][2]);
      acc[i][jp][3] = fmaf(sc_prev, p_prev[i][3], acc[i][jp][3]);
      asm volatile("" : "+v"(acc[i][jp]));
      between(i);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < I; ++i) p_prev[i] = p_cur[i];
    sc_prev = sc;
  };
  auto nothing = [](int) {};

  // Step g from stage st: sub-tiles 0 .. J - 2 with the next fragment in
  // flight; sub-tile J - 1 either across the barrier into step g + 1 (its
  // MFMAs hide the latency of step g + 1's first fragment reads) or, at the
  // last step, as a final drain.
  auto step = [&](int64_t g, auto st) {
    constexpr int cur = decltype(st)::value;
    using SN = std::integral_constant<int, cur ^ 1>;
    // Unclamped, the second half of step g + 1's copies (into the other
    // stage) go out with sub-tile 0 (the first went out with step g - 1's
    // deferred sub-tile; the prologue copied group 1 whole); clamped, its
    // per-copy lane offsets leave no registers for that and all go out with
    // the deferred sub-tile.
    const bool second_half = kSplitCopies && g >= 1 && g + 1 < groups;
#pragma unroll
    for (int j = 0; j < J - 1; ++j) {
      const v8i af_n = a_frag(st, j + 1);
      const float sa_n = a_scale(g, j + 1);
      set_prio(3 - (3 * (j + 1)) / (J - 1));
      mfma_row((j + J - 1) % J, sa * sw, [&](int i) {
        if (j == 0 && second_half) {
#pragma unroll
          for (int c = HALF + i * (CHUNKS - HALF) / I; c < HALF + (i + 1) * (CHUNKS - HALF) / I; ++c)
            issue_chunk(g + 1, SN{}, c);
        }
      });
      af = af_n;
      sa = sa_n;
    }
    // The same code at every step, the last included (its fragment reads
    // after the barrier fetch a stage that holds nothing of use, and are
    // not used): with a separate branch for the last step the compiler
    // renamed the running sums across the two paths and moved them back,
    // about 30 register moves per step.
    const bool more = g + 1 < groups;
    if (more && ((g + 1) & 63) == 0) sw_lanes = sw_chunk(g + 1);
    const float sw_n = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sw_lanes),
                                                                           static_cast<int>((g + 1) & 63)));
    // every LDS read of this stage has completed and step g + 1's tiles
    // have landed (own copies: vmcnt; everyone's: the barrier)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    set_prio(3);
    // step g + 2's copies, spread over the deferred sub-tile's MFMAs
    // (issued at once after the barrier, every wave's burst of copies
    // held up its MFMAs: 3.5% more cycles per K step); past the last group
    // a copy of it into the stage just consumed, never read
    const int64_t g2 = g + 2 < groups ? g + 2 : groups - 1;
    if (g + 2 < groups && (g2 & 7) == 0) issue_scales(g2);
    const v8i af_n = a_frag(SN{}, 0);
    const float sa_n = a_scale(g + 1, 0);
    mfma_row(J - 2, sa * sw, [&](int i) {
      wf[i] = w_frag(SN{}, i);
#pragma unroll
      for (int c = i * HALF / I; c < (i + 1) * HALF / I; ++c) issue_chunk(g2, st, c);
    });
    af = af_n;
    sa = sa_n;
    sw = sw_n;
  };

  for (int64_t g = 0; g < groups; g += 2) {
    step(g, S0{});
    if (g + 1 < groups) step(g + 1, S1{});
  }
  // last sub-tile's results
#pragma unroll
  for (int i = 0; i < I; ++i) {
    acc[i][J - 1][0] = fmaf(sc_prev, p_prev[i][0], acc[i][J - 1][0]);
    acc[i][J - 1][1] = fmaf(sc_prev, p_prev[i][1], acc[i][J - 1][1]);
    acc[i][J - 1][2] = fmaf(sc_prev, p_prev[i][2], acc[i][J - 1][2]);
    acc[i][J - 1][3] = fmaf(sc_prev, p_prev[i][3], acc[i][J - 1][3]);
  }
  // copies issued past the last step must land before the LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t m = m0 + TM * wave_m + 16 * j + lrow;
    if (m >= m_rows || m < m_own) continue;
#pragma unroll
    for (int i = 0; i < I; ++i) {
      const int64_t col = n0 + TN * wave_n + 16 * i + 4 * quarter;
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

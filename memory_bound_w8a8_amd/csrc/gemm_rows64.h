// Weight-streaming split-K block-FP8 GEMM for 33..80 tokens, gfx950: 33..48
// tokens as three 16-token sub-tiles (MSX = 3), 49..64 as four, 65..80 as
// five (only with at most 2 row tiles and 5 groups per wave, where the
// accumulators and activation fragments still fit in registers).
//
// Still HBM-bound (about 2 M flop per weight byte, far below the FP8 MFMA
// ridge), so the design is the row-range streaming one of gemm_rows.h: one
// workgroup per CU owns a balanced range of weight rows, its 8 waves split
// the K/128 scale groups, every load instruction reads eight whole 128-byte
// lines, and a branch-free, fully unrolled chunk sequence keeps PD chunks of
// weight loads in flight per wave.
//
// What changes at 64 tokens is the activation operand: 64 tokens x 32 bytes
// per lane and group is 32 registers, so a wave cannot hold it for all its
// groups. The chunk order is therefore group-major: a wave walks its groups,
// and within a group all row tiles, keeping the fp32 accumulators of every
// (row tile, 16-token sub-tile) pair live (16 x TILES registers) and the
// activation operand of only the groups in flight. Each group's activation
// fragment (L2-resident: every workgroup reads the same 64 x K bytes) is
// loaded in the same step as the group's first weight chunk, so the in-order
// load counter never makes a wait cover loads issued later than needed.
//
// Reduction: after the last chunk every wave holds fp32 partials of all its
// tiles. Two row tiles at a time, the 8 waves park them in LDS; the 2 * MS
// (tile, sub-tile) items of the round go to the waves in turn (item i to
// wave i mod 8: with three sub-tiles waves 6 and 7 sit out, with five waves
// 0 and 1 take a second item), and each sums its item over the waves in
// order 0..7 (deterministic, no atomics), rounds to bf16 (RNE) and stores 4
// consecutive outputs per lane.
#pragma once

#include "device_common.h"
#include "wave_prio.h"

namespace fp8bq {

template <int GMAX, int TILES, int PD, int MSX = 4>
struct Rows64Kernel {
  static constexpr int kWaves = 8;
  static constexpr int kMS = MSX;                              // 16-token sub-tiles (3, 4 or 5)
  static constexpr int kChunks = TILES * GMAX;
  static constexpr int kRing = PD + 1;                         // weight chunk buffers
  static constexpr int kActSlots = (PD + TILES - 1) / TILES + 1;  // activation groups live at once
  static constexpr int kPair = 2;                              // row tiles per reduction round
};

// Workgroup barrier that completes this wave's LDS traffic first but leaves
// global stores in flight (__syncthreads() would also wait for those).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int GMAX, int TILES, int PD, int MSX = 4>
__global__ __launch_bounds__(512) void gemm_rows64_kernel(int m_rows, int64_t n, int64_t k, int64_t rows_per_wg,
                                                          const unsigned char* __restrict__ aq,
                                                          const float* __restrict__ as,
                                                          const unsigned char* __restrict__ wq,
                                                          const float* __restrict__ ws,
                                                          unsigned short* __restrict__ c) {
  using KC = Rows64Kernel<GMAX, TILES, PD, MSX>;
  static_assert(MSX >= 3 && MSX <= 5, "48-, 64- or 80-token tiles");
  constexpr int S = KC::kWaves;
  constexpr int MS = KC::kMS;
  constexpr int CH = KC::kChunks;
  constexpr int RING = KC::kRing;
  constexpr int AS = KC::kActSlots;
  constexpr int PAIR = KC::kPair;
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
  __shared__ v4u astage[S][128];
  __shared__ v4f red[S][PAIR][MS][64];

  // All operands are read through buffer resources with 32-bit offsets: one
  // offset register per stream instead of 64-bit pointers per chunk, and a
  // lane whose row (weight row past the range, token past M) lies outside
  // the resource reads zeros, so absent rows and tokens need no clamping.
  // Groups past the wave's range re-read its last group with a zero scale.
  constexpr uint32_t kOutOfBounds = 0x80000000u;  // past every resource here
  const uint32_t rows_here = static_cast<uint32_t>(r_end - r_begin);
  const uint32_t ku = static_cast<uint32_t>(k);
  const auto wrs = buffer_rsrc(wq + r_begin * k, rows_here * ku);
  const auto ars = buffer_rsrc(aq, static_cast<uint32_t>(m_rows) * ku);
  const auto sars = buffer_rsrc(as, static_cast<uint32_t>(m_rows) * static_cast<uint32_t>(groups) * 4u);
  const int64_t blk0 = r_begin >> 7;
  const auto swrs = buffer_rsrc(ws + blk0 * groups, static_cast<uint32_t>(((r_last >> 7) - blk0 + 1) * groups * 4));

  // Activation of group g: instruction j (0..7) reads tokens 8 j + lane / 8,
  // piece lane % 8: eight whole lines per instruction, like the weights.
  // (Every workgroup reads the same activation lines at about the same
  // time; half-line requests spread over 16 token rows concentrate on a few
  // L2 channels and queue there.) The raw lines are transposed into the
  // MFMA operand when the group starts.
  v4u araw[AS][2 * MS];
  float sa[AS][MS];
  auto load_act = [&](int u) {
    const bool live = u < gcnt;
    const uint32_t g = static_cast<uint32_t>(live ? gbeg + u : glast);
#pragma unroll
    for (int j = 0; j < 2 * MS; ++j) {
      const uint32_t m = static_cast<uint32_t>(8 * j + (lane >> 3));
      araw[u % AS][j] = buffer_load16(ars, m * ku + static_cast<uint32_t>((lane & 7) * 16), g * kGroup);
    }
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      const uint32_t m = static_cast<uint32_t>(16 * s + lrow);
      // a group past the wave's range reads its scale out of bounds (0);
      // selecting on the offset, not on the loaded value, keeps the load
      // from being waited for here
      const uint32_t soff = live ? m * static_cast<uint32_t>(groups) * 4u : kOutOfBounds;
      sa[u % AS][s] = buffer_load_f32(sars, soff, g * 4u);
    }
  };

  // Weight chunk ci = (group u, row tile t) with u = ci / TILES: rows
  // 8 j + lane / 8 of the tile (j = 0, 1), 16-byte piece lane % 8.
  const int lr8 = lane >> 3;
  const int piece = lane & 7;
  v8i wv[RING];
  float sw[RING];
  auto load_chunk = [&](int ci) {
    const int u = ci / TILES;
    const int t = ci - u * TILES;
    if (t == 0) load_act(u);
    const uint32_t g = static_cast<uint32_t>(u < gcnt ? gbeg + u : glast);
    const uint32_t voff = static_cast<uint32_t>(16 * t + lr8) * ku + static_cast<uint32_t>(piece * 16);
    const v4u lo = buffer_load16_nt(wrs, voff, g * kGroup);
    const v4u hi = buffer_load16_nt(wrs, voff + 8u * ku, g * kGroup);
    wv[ci % RING] = join8(lo, hi);
    const uint32_t blk = static_cast<uint32_t>(((r_begin + 16 * t + 4 * quarter) >> 7) - blk0);
    sw[ci % RING] = buffer_load_f32(swrs, blk * static_cast<uint32_t>(groups) * 4u, g * 4u);
  };

  // Pieces this lane loaded (rows lr8 and lr8 + 8, piece `piece`) -> the
  // MFMA operand of row lrow (pieces quarter and quarter + 4), through a
  // private XOR-swizzled LDS slot (conflict-free 8-lane passes both ways).
  auto transpose = [&](const v8i& raw, v4u* slot) -> v8i {
    slot[8 * lr8 + (piece ^ lr8)] = v4u{(unsigned)raw[0], (unsigned)raw[1], (unsigned)raw[2], (unsigned)raw[3]};
    slot[8 * (lr8 + 8) + (piece ^ lr8)] = v4u{(unsigned)raw[4], (unsigned)raw[5], (unsigned)raw[6], (unsigned)raw[7]};
    __builtin_amdgcn_wave_barrier();
    const int x = lrow & 7;
    const v4u lo = slot[8 * lrow + (quarter ^ x)];
    const v4u hi = slot[8 * lrow + ((quarter + 4) ^ x)];
    __builtin_amdgcn_wave_barrier();
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  v8i bcur[MS];  // activation operand of the current group
  v4f acc[TILES][MS];
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int s = 0; s < MS; ++s) acc[t][s] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int ci = 0; ci < PD && ci < CH; ++ci) load_chunk(ci);
#pragma unroll
  for (int ci = 0; ci < CH; ++ci) {
    // the wave that is behind in its chunk sequence gets the SIMD first
    // (1-3% at 48..80 tokens; the same in the <= 32-token kernel cost 4-7%)
    set_prio(3 - (4 * ci) / CH);
    const int u = ci / TILES;
    const int t = ci - u * TILES;
    // keep the scheduler from hoisting later chunks' loads (and their
    // registers) into this one: the chunk sequence is the pipeline
    __builtin_amdgcn_sched_barrier(0);
    if (ci + PD < CH) load_chunk(ci + PD);
    if (t == 0) {
#pragma unroll
      for (int s = 0; s < MS; ++s) bcur[s] = transpose(join8(araw[u % AS][2 * s], araw[u % AS][2 * s + 1]), astage[wave]);
    }
    const v8i wop = transpose(wv[ci % RING], stage[wave][ci & 1]);
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      // lane: rows 16 t + 4 quarter + i (one aligned quad, one weight
      // block), token 16 s + lrow
      const v4f p = mfma_16x16x128_e4m3(wop, bcur[s]);
      const float sc = sa[u % AS][s] * sw[ci % RING];
      acc[t][s][0] = fmaf(sc, p[0], acc[t][s][0]);
      acc[t][s][1] = fmaf(sc, p[1], acc[t][s][1]);
      acc[t][s][2] = fmaf(sc, p[2], acc[t][s][2]);
      acc[t][s][3] = fmaf(sc, p[3], acc[t][s][3]);
      // Pin the update inside this chunk: left free, the compiler defers the
      // FMAs to the accumulator's next use and keeps (or spills) every
      // MFMA result until then.
      asm volatile("" : "+v"(acc[t][s]));
    }
  }

#pragma unroll
  for (int t0 = 0; t0 < TILES; t0 += PAIR) {
#pragma unroll
    for (int p = 0; p < PAIR; ++p)
      if (t0 + p < TILES)
#pragma unroll
        for (int s = 0; s < MS; ++s) red[wave][p][s][lane] = acc[t0 + p][s];
    lds_barrier();
    // items (tile of the pair, sub-tile) = (it / MS, it % MS), it = wave,
    // wave + 8, ...
#pragma unroll
    for (int it0 = 0; it0 < PAIR * MS; it0 += S) {
      const int it = it0 + wave;
      const int rp = it / MS;
      const int rs = it % MS;
      if (it >= PAIR * MS || t0 + rp >= TILES) continue;
      v4f sum = red[0][rp][rs][lane];
#pragma unroll
      for (int w = 1; w < S; ++w) sum += red[w][rp][rs][lane];
      const int m = 16 * rs + lrow;
      const int64_t col = r_begin + 16 * (t0 + rp) + 4 * quarter;  // first of 4 consecutive outputs
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
    if (t0 + PAIR < TILES) lds_barrier();
  }
}

}  // namespace fp8bq

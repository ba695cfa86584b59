// Weight-streaming split-K block-FP8 GEMM with balanced row ranges, gfx950.
//
// At M <= 64 the op reads every weight byte once and is bound by HBM (page 1,
// SmartX blog, section "operator optimisation": the weight-reading matmuls
// take about 89% of a decode step and sit near the bandwidth floor; page 1,
// same section: a library's poor kernel choice at M = 2..7 cost 8.8x, so the
// cost here must not depend on M within a token tile). What decides the
// achieved bandwidth is (a) that every CU streams the same number of bytes,
// (b) that every load instruction reads whole 128-byte lines, and (c) that
// each wave keeps loads in flight without ever draining its queue.
//
// Decomposition. One workgroup per CU (grid = ceil(N / R)). Workgroup w owns
// rows [w R, min(w R + R, N)) of W, R a multiple of 4 that spreads N evenly
// (17408 / 256 = 68 rows), walked as TILES 16-row MFMA tiles. Its S waves
// split the K/128 scale groups into contiguous ranges of at most GMAX groups
// (split-K). A wave's work is TILES x GMAX "chunks" of 16 rows x 128 bytes.
//
// Loads. For a chunk, load instruction j (j = 0, 1) reads rows 8 j .. 8 j + 7
// of the tile and the whole 128-byte group of each (lane l: row 8 j + l / 8,
// 16-byte piece l % 8): 8 full lines per instruction, non-temporal. Rows past
// the range are clamped onto the range's last row and groups past the wave's
// range onto its last group (scale forced to 0), so the code has no branches:
// every wave runs the same straight-line load/compute sequence and the
// compiler can keep the next PD chunks' loads in flight while computing.
//
// Transpose. The MFMA wants lane l to hold 32 bytes of tile row l % 16
// (16 bytes at 16 (l / 16) and 16 bytes at 64 + 16 (l / 16) of the group),
// with the activation operand (token l % 16) in the same byte order. A wave
// writes its chunk to a private LDS slot, piece c of row r at index
// 8 r + (c ^ (r & 7)) (the XOR makes both the 8-lane write passes and the
// 8-lane read passes hit 8 distinct 16-byte bank groups), and reads it back
// in MFMA order. LDS operations of one wave execute in order, so no barrier
// is needed between the write and the read.
//
// Math. One 16x16x128 FP8 MFMA per chunk and 16-token tile gives the 128-long
// dot products of 16 rows x 16 tokens. Lane l's result covers rows
// 4 (l / 16) .. +3: an aligned quad that never straddles a 128-row weight
// block, so acc += (A_scale[m, g] * W_scale[quad / 128, g]) * mfma in fp32.
//
// Reduction. After a tile, each wave parks its fp32 16 x MT partial in LDS;
// at the end the S partials of every tile are summed in wave order 0..S-1
// (deterministic, no atomics), rounded to bf16 (RNE) and stored, 4
// consecutive outputs (8 bytes) per lane.
#pragma once

#include "device_common.h"

namespace fp8bq {

// Activation forms the row-range kernel takes.
enum ActForm : int {
  kActCodes = 0,      // e4m3fn codes + scales, operand loaded directly
  kActCodeLines = 1,  // e4m3fn codes + scales, whole lines + LDS transpose
  kActBf16 = 2,       // bf16 activation, quantised in the kernel
};

// Largest value of v over each aligned group of LPT lanes (a power of two,
// 1..64), returned to every lane of the group; v are bit patterns of
// non-negative floats, whose order as unsigned integers is their order as
// floats. DPP inside 16-lane rows (swap neighbours, swap pairs, mirror
// half-rows, mirror rows), then the four row results read as scalars.
template <int CTRL>
__device__ __forceinline__ unsigned dpp_row(unsigned v) {
  return static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ unsigned umax_u32(unsigned a, unsigned b) { return a > b ? a : b; }

template <int LPT>
__device__ __forceinline__ unsigned lane_group_umax(unsigned v) {
  if constexpr (LPT >= 2) v = umax_u32(v, dpp_row<0xB1>(v));
  if constexpr (LPT >= 4) v = umax_u32(v, dpp_row<0x4E>(v));
  if constexpr (LPT >= 8) v = umax_u32(v, dpp_row<0x141>(v));
  if constexpr (LPT >= 16) v = umax_u32(v, dpp_row<0x140>(v));
  if constexpr (LPT >= 32) {
    const unsigned r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
    const unsigned r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
    if constexpr (LPT == 32)
      v = (threadIdx.x & 32) ? umax_u32(r2, r3) : umax_u32(r0, r1);
    else
      v = umax_u32(umax_u32(r0, r1), umax_u32(r2, r3));
  }
  return v;
}

// Quantise one group for at most TOK (< 16) tokens with the values spread
// over the wave instead of over the MFMA operand (where each lane would
// quantise 32 values, mostly copies of other lanes'): lane l holds bf16
// values V (l % LPT) .. V (l % LPT) + V - 1 of token l / LPT (LPT = 64 / TOK
// lanes per token, V = 2 TOK, raw[] as bf16 pairs). Same rule as
// quant_act_kernel: amax over the 128 values, s = amax / 448 (IEEE; 1 for an
// all-zero group), code = RNE(x / s), with the quotient of
// quotient_e4m3_gemm (device_common.h): equal in code to the IEEE division
// whenever amax >= 2^-96 (a -0 may come out +0, which no GEMM sum can see);
// below, the division. The codes feed only the MFMA, so C is bitwise that of
// fp8bq_quant_act + fp8bq_gemm. The codes go to the wave's LDS slot (row = token,
// 16-byte piece c of a row at 8 row + (c ^ (row & 7))), and the lane gets
// back its MFMA operand, token min(l % 16, m_rows - 1), and that token's
// scale. Requires m_rows <= TOK.
template <int TOK>
__device__ __forceinline__ v8i quant_group_compact(const v4u (&raw)[2], int m_rows, v4u* slot, float* scale) {
  static_assert(TOK == 1 || TOK == 2 || TOK == 4 || TOK == 8, "TOK");
  constexpr int LPT = 64 / TOK;
  constexpr int V = 2 * TOK;
  const int lane = threadIdx.x & 63;
  const int tok = lane / LPT;
  const int off = (lane % LPT) * V;  // first value (= code byte) of the lane in the token's group
  float x[V];
#pragma unroll
  for (int i = 0; i < V / 2; ++i) {
    x[2 * i] = bf16_lo(raw[i / 4][i % 4]);
    x[2 * i + 1] = bf16_hi(raw[i / 4][i % 4]);
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < V; ++j) amax = fmaxf(amax, fabsf(x[j]));
  amax = __builtin_bit_cast(float, lane_group_umax<LPT>(__builtin_bit_cast(unsigned, amax)));
  const float s = group_scale(amax);
  float q[V];
  if (amax >= 0x1p-96f) {
    const RecipPair y = recip_pair(s);
#pragma unroll
    for (int j = 0; j < V; ++j) q[j] = quotient_e4m3_gemm(x[j], y);
  } else {
#pragma unroll
    for (int j = 0; j < V; ++j) q[j] = scaled_clamped(x[j], s);
  }
  unsigned char* base = reinterpret_cast<unsigned char*>(slot);
  unsigned char* dst = base + (8 * tok + ((off >> 4) ^ (tok & 7))) * 16 + (off & 15);
  if constexpr (V == 2) {
    *reinterpret_cast<unsigned short*>(dst) =
        static_cast<unsigned short>(__builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], 0, false));
  } else if constexpr (V == 4) {
    *reinterpret_cast<unsigned*>(dst) = encode4_e4m3(q[0], q[1], q[2], q[3]);
  } else if constexpr (V == 8) {
    *reinterpret_cast<v2u*>(dst) = v2u{encode4_e4m3(q[0], q[1], q[2], q[3]), encode4_e4m3(q[4], q[5], q[6], q[7])};
  } else {
    *reinterpret_cast<v4u*>(dst) = v4u{encode4_e4m3(q[0], q[1], q[2], q[3]), encode4_e4m3(q[4], q[5], q[6], q[7]),
                                       encode4_e4m3(q[8], q[9], q[10], q[11]),
                                       encode4_e4m3(q[12], q[13], q[14], q[15])};
  }
  __builtin_amdgcn_wave_barrier();
  const int lrow = lane & 15;
  const int quarter = lane >> 4;
  const int tm = lrow < m_rows ? lrow : m_rows - 1;
  const v4u lo = slot[8 * tm + (quarter ^ (tm & 7))];
  const v4u hi = slot[8 * tm + ((quarter + 4) ^ (tm & 7))];
  __builtin_amdgcn_wave_barrier();
  *scale = __shfl(s, tm * LPT);
  return join8(lo, hi);
}

template <int MT, int S, int GMAX, int TILES, int PD, int AF, int TOK = 16>
struct RowsKernel {
  static constexpr int kMS = MT / 16;        // 16-token tiles
  static constexpr int kChunks = TILES * GMAX;
  static constexpr int kRing = PD + 1;       // chunk register buffers
  static constexpr int kStageSlots = 2;      // LDS transpose slots per wave
  static constexpr int kLdsBytes =
      S * kStageSlots * 2048 + S * TILES * kMS * 1024 + (AF == kActBf16 ? S * 2048 : 0);
};

template <int MT, int S, int GMAX, int TILES, int PD, int AF, int TOK = 16>
__global__ __launch_bounds__(64 * S) void gemm_rows_kernel(int m_rows, int64_t n, int64_t k, int64_t rows_per_wg,
                                                           const unsigned char* __restrict__ aq,
                                                           const float* __restrict__ as,
                                                           const unsigned char* __restrict__ wq,
                                                           const float* __restrict__ ws,
                                                           unsigned short* __restrict__ c) {
  using KC = RowsKernel<MT, S, GMAX, TILES, PD, AF, TOK>;
  constexpr bool LINES = AF == kActCodeLines;
  constexpr bool BF16 = AF == kActBf16;
  // bf16 activation of at most TOK <= 8 tokens: quantised in the wave-wide
  // layout of quant_group_compact (m_rows <= TOK)
  constexpr bool COMPACT = BF16;
  static_assert(!BF16 || (MT == 16 && TOK <= 8), "in-kernel quantisation serves up to 8 tokens");
  // Chunk order. Tile-major (all groups of tile 0, then tile 1, ...) keeps
  // one accumulator set but holds the activation of all the wave's groups
  // in registers for the whole kernel; group-major (all tiles of group 0,
  // then group 1, ...) holds one accumulator set per tile and only the
  // groups in use, loaded with their group's first weight chunk. Group-major
  // serves in-kernel quantisation (each group's quantisation then falls
  // every TILES chunks rather than all within the first tile), the directly
  // loaded codes of up to 8 tokens (their loads then go out with the weight
  // stream instead of ahead of it: 1-7% faster at M = 1..8 on the five
  // logged shapes) and 32-token tiles with more than 6 groups per wave
  // (whose activation would not fit).
  constexpr bool GROUP_MAJOR = BF16 || AF == kActCodes || (LINES && MT == 32 && GMAX > 6);
  constexpr int MS = KC::kMS;
  constexpr int CH = KC::kChunks;
  constexpr int RING = KC::kRing;
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

  __shared__ v4u stage[S][KC::kStageSlots][128];
  __shared__ v4f red[S][TILES][MS][64];

  // Per-lane load bases: rows 8 j + lane / 8 of each 16-row tile, piece
  // lane % 8 (weights and activation alike: whole lines per instruction).
  const int lr8 = lane >> 3;
  const int piece = lane & 7;

  // Activation operand and scales of this wave's groups, same for all
  // tiles. Load forms (AF):
  //  - kActCodeLines: whole lines (tokens 16 s + 8 j + lane / 8, clamped),
  //    each group transposed into the MFMA operand at its first use, in the
  //    first row tile, while weight chunks are in flight. With many distinct
  //    tokens this matters: every workgroup reads the same activation lines
  //    at about the same time, and half-line requests from 16 token rows
  //    queue in a few L2 channels.
  //  - kActCodes: the operand directly (token 16 s + lane % 16, pieces
  //    quarter and quarter + 4). With few tokens the clamped rows coincide,
  //    an instruction touches few lines, and no transposes are needed.
  //  - kActBf16: the bf16 activation (`aq` then points at bf16 data, `as`
  //    is unused), spread over the wave and quantised into the operand and a
  //    scale at the group's first use (quant_group_compact).
  v8i bv[GMAX][MS];
  float sa[GMAX][MS];
  // (kActBf16: loaded with the group's first weight chunk, PD chunks ahead
  // of its first use, in load_chunk below; group-major order uses a group
  // for TILES consecutive chunks, so only a few groups are ever live.)
  v4u araw[BF16 ? GMAX : 1][2];
  __shared__ v4u astage[COMPACT ? S : 1][128];
  const unsigned short* arow = nullptr;
  if constexpr (COMPACT) {
    constexpr int LPT = 64 / TOK;
    int tok = lane / LPT;
    tok = tok < m_rows ? tok : m_rows - 1;
    arow = reinterpret_cast<const unsigned short*>(aq) + static_cast<int64_t>(tok) * k + (lane % LPT) * (2 * TOK);
  }
  // Activation codes (and scales) of group u for every 16-token tile, as
  // whole lines (LINES) or as the operand directly.
  const unsigned char* ap0[MS];
  const unsigned char* ap1[MS];
  const float* sap[MS];
  bool mval[MS];
  if constexpr (!BF16) {
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      if constexpr (LINES) {
        int m0 = 16 * s + lr8;
        int m1 = m0 + 8;
        m0 = m0 < m_rows ? m0 : m_rows - 1;
        m1 = m1 < m_rows ? m1 : m_rows - 1;
        ap0[s] = aq + static_cast<int64_t>(m0) * k + piece * 16;
        ap1[s] = aq + static_cast<int64_t>(m1) * k + piece * 16;
      } else {
        int m0 = 16 * s + lrow;
        m0 = m0 < m_rows ? m0 : m_rows - 1;
        ap0[s] = aq + static_cast<int64_t>(m0) * k + quarter * 16;
        ap1[s] = ap0[s] + 64;
      }
      const int m = 16 * s + lrow;
      mval[s] = m < m_rows;
      sap[s] = as + static_cast<int64_t>(mval[s] ? m : m_rows - 1) * groups;
    }
  }
  auto load_act_tile = [&](int u, int s) {
    const bool live = u < gcnt;
    const int g = live ? gbeg + u : glast;
    const int64_t off = static_cast<int64_t>(g) * kGroup;
    // Lanes of tokens past M load nothing (their MFMA columns are not
    // stored and their scale is 0): with the clamped address every such lane
    // would read the last token's bytes, and loads whose lanes repeat one
    // address measured up to 10% slower at M = 1..4.
    v4u lo = v4u{0u, 0u, 0u, 0u}, hi = v4u{0u, 0u, 0u, 0u};
    float scale = 0.f;
    if (LINES || mval[s]) {
      lo = *reinterpret_cast<const v4u*>(ap0[s] + off);
      hi = *reinterpret_cast<const v4u*>(ap1[s] + off);
    }
    if (mval[s]) scale = sap[s][g];
    bv[u][s] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    sa[u][s] = live ? scale : 0.f;
  };
  auto load_act = [&](int u) {
#pragma unroll
    for (int s = 0; s < MS; ++s) load_act_tile(u, s);
  };
  if constexpr (!BF16 && !GROUP_MAJOR) {
#pragma unroll
    for (int s = 0; s < MS; ++s)
#pragma unroll
      for (int u = 0; u < GMAX; ++u) load_act_tile(u, s);
  }

  v8i wv[RING];
  float sw[RING];

  auto load_chunk = [&](int ci, int slot) {
    const int t = GROUP_MAJOR ? ci % TILES : ci / GMAX;
    const int u = GROUP_MAJOR ? ci / TILES : ci % GMAX;
    const int g = u < gcnt ? gbeg + u : glast;
    if (GROUP_MAJOR && !BF16 && t == 0) load_act(u);
    if (BF16 && t == 0) {
      const unsigned short* p = arow + static_cast<int64_t>(g) * kGroup;
      // 2 TOK bf16 values of one token
      if constexpr (TOK == 1) {
        araw[u][0][0] = *reinterpret_cast<const unsigned*>(p);
      } else if constexpr (TOK == 2) {
        const v2u d = *reinterpret_cast<const v2u*>(p);
        araw[u][0][0] = d[0];
        araw[u][0][1] = d[1];
      } else {
        araw[u][0] = *reinterpret_cast<const v4u*>(p);
        if constexpr (TOK == 8) araw[u][1] = *reinterpret_cast<const v4u*>(p + 8);
      }
    }
    const int64_t off = static_cast<int64_t>(g) * kGroup + piece * 16;
    int64_t row0 = r_begin + 16 * t + lr8;
    int64_t row1 = row0 + 8;
    row0 = row0 < r_end ? row0 : r_last;
    row1 = row1 < r_end ? row1 : r_last;
    const v4u lo = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wq + row0 * k + off));
    const v4u hi = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wq + row1 * k + off));
    wv[slot] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    int64_t quad = r_begin + 16 * t + 4 * quarter;
    quad = quad < r_end ? quad : r_last;
    sw[slot] = ws[(quad >> 7) * groups + g];
  };

  // Pieces this lane loaded (rows lr8 and lr8 + 8, piece `piece`) -> the
  // MFMA operand of row lrow (pieces quarter and quarter + 4).
  auto transpose = [&](const v8i& raw, int st) -> v8i {
    v4u* slot = stage[wave][st];
    slot[8 * lr8 + (piece ^ lr8)] = v4u{(unsigned)raw[0], (unsigned)raw[1], (unsigned)raw[2], (unsigned)raw[3]};
    slot[8 * (lr8 + 8) + (piece ^ lr8)] = v4u{(unsigned)raw[4], (unsigned)raw[5], (unsigned)raw[6], (unsigned)raw[7]};
    __builtin_amdgcn_wave_barrier();
    const int x = lrow & 7;
    const v4u lo = slot[8 * lrow + (quarter ^ x)];
    const v4u hi = slot[8 * lrow + ((quarter + 4) ^ x)];
    __builtin_amdgcn_wave_barrier();
    return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };

  // Accumulators: one set per tile in group-major order, else one set
  // reused tile after tile. Either way every output sums its groups in the
  // same order 0, 1, ..., so the two orders give bitwise the same result.
  v4f acc[GROUP_MAJOR ? TILES : 1][MS];
#pragma unroll
  for (int t = 0; t < (GROUP_MAJOR ? TILES : 1); ++t)
#pragma unroll
    for (int s = 0; s < MS; ++s) acc[t][s] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ci = 0; ci < PD && ci < CH; ++ci) load_chunk(ci, ci % RING);
#pragma unroll
  for (int ci = 0; ci < CH; ++ci) {
    const int t = GROUP_MAJOR ? ci % TILES : ci / GMAX;
    const int u = GROUP_MAJOR ? ci / TILES : ci % GMAX;
    v4f (&at)[MS] = acc[GROUP_MAJOR ? t : 0];
    // With many groups per wave in group-major order, keep the
    // scheduler from hoisting later chunks' loads (and the activation
    // values they bring) above this one: their registers would outgrow the
    // budget and spill.
    if constexpr (GROUP_MAJOR && GMAX >= 7) __builtin_amdgcn_sched_barrier(0);
    if (ci + PD < CH) load_chunk(ci + PD, (ci + PD) % RING);
    if (!GROUP_MAJOR && u == 0) {
#pragma unroll
      for (int s = 0; s < MS; ++s) at[s] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    if constexpr (BF16) {
      if (t == 0) {  // first use of group u: quantise its activation
        float scale;
        bv[u][0] = quant_group_compact<TOK>(araw[u], m_rows, astage[wave], &scale);
        sa[u][0] = u < gcnt ? scale : 0.f;  // a group past the range adds nothing
      }
    }
    if (LINES && t == 0) {  // first use of group u: its activation lines -> operand
#pragma unroll
      for (int s = 0; s < MS; ++s) bv[u][s] = transpose(bv[u][s], (ci + s + 1) & 1);
    }
    const v8i wop = transpose(wv[ci % RING], ci & 1);
#pragma unroll
    for (int s = 0; s < MS; ++s) {
      const v4f p = mfma_16x16x128_e4m3(wop, bv[u][s]);
      const float sc = sa[u][s] * sw[ci % RING];
      at[s][0] = fmaf(sc, p[0], at[s][0]);
      at[s][1] = fmaf(sc, p[1], at[s][1]);
      at[s][2] = fmaf(sc, p[2], at[s][2]);
      at[s][3] = fmaf(sc, p[3], at[s][3]);
    }
    if (u == GMAX - 1) {
#pragma unroll
      for (int s = 0; s < MS; ++s) red[wave][t][s][lane] = at[s];
    }
  }
  __syncthreads();

  // Sum the S partials of every (tile, token tile) and store.
#pragma unroll
  for (int item0 = 0; item0 < TILES * MS; item0 += S) {
    const int item = item0 + wave;
    if (item < TILES * MS) {
      const int t = item / MS;
      const int s = item - t * MS;
      v4f sum = red[0][t][s][lane];
#pragma unroll
      for (int w = 1; w < S; ++w) sum += red[w][t][s][lane];
      const int m = 16 * s + lrow;
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

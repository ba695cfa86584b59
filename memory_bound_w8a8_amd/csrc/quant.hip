// Activation (per token, 1x128 group) and weight (128x128 block) FP8
// quantisation for gfx950.
//
// Activation side: page 1 (SmartX blog), section "single-stream
// optimisation" -- the W8A8 backend quantises each linear layer's input on
// every call. Weight side: page 2 (ownding.com L20 report), section 8 -- the
// weights are stored as W8A8 block FP8. Rule for one group or block:
// s = amax / 448 (IEEE fp32 division, 1.0 for amax == 0), code =
// e4m3fn_rne(clamp(x / s, -448, 448)); bit-exact with that definition.
#include "device_common.h"
#include "launch.h"

namespace fp8bq {

// One 128-wide group per 16 lanes at a time: each lane holds 8 bf16 (one
// 16-byte load), the 16 lanes of a DPP row reduce the amax with xor
// shuffles, then each lane forms its 8 quotients, encodes them and stores 8
// bytes. Groups are contiguous in memory ([M, K] row-major, K % 128 == 0),
// so the grid walks the flat group index m * (K / 128) + g, each 16-lane row
// taking two groups per trip (both loads issued before either is used) and
// striding by the grid's rows, so that large activations run as a few
// thousand long-lived workgroups with loads in flight rather than one short
// workgroup per 16 groups. The quotient is quotient_e4m3_range (3 VALU
// operations instead of an IEEE division's ~10) above amax = 2^-96, the
// IEEE division below: codes equal to x / s either way.
__device__ __forceinline__ void quant_act_group(const v4u& raw, int64_t g, int sub, bool store,
                                                unsigned char* __restrict__ aq, float* __restrict__ as) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(raw[i]);
    x[2 * i + 1] = bf16_hi(raw[i]);
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
  const float s = group_scale(amax);
  float q[8];
  if (amax >= 0x1p-96f) {
    const float y = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = quotient_e4m3_range(x[i], s, y);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = scaled_clamped(x[i], s);
  }
  v2u out;
  out[0] = encode4_e4m3(q[0], q[1], q[2], q[3]);
  out[1] = encode4_e4m3(q[4], q[5], q[6], q[7]);
  if (store) {
    *reinterpret_cast<v2u*>(aq + g * kGroup + sub * 8) = out;
    if (sub == 0) as[g] = s;
  }
}

// PAIR: two groups per row per trip (activations of more groups than one
// grid trip covers); otherwise one group per row and a single trip, so that
// a decode-sized call pays one load and one quantisation per lane.
template <bool PAIR>
__global__ __launch_bounds__(256) void quant_act_kernel(const unsigned short* __restrict__ a,
                                                        unsigned char* __restrict__ aq,
                                                        float* __restrict__ as, int64_t groups) {
  const int sub = threadIdx.x & 15;
  const int64_t rows = static_cast<int64_t>(gridDim.x) * 16;  // 16-lane rows in the grid
  const int64_t first = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 4;
  if constexpr (!PAIR) {
    const bool valid = first < groups;
    const int64_t g = valid ? first : groups - 1;
    quant_act_group(*reinterpret_cast<const v4u*>(a + g * kGroup + sub * 8), g, sub, valid, aq, as);
  } else {
    for (int64_t g0 = first; g0 < groups; g0 += 2 * rows) {
      const int64_t g1 = g0 + rows < groups ? g0 + rows : g0;  // a row past the end redoes g0, unstored
      const v4u r0 = *reinterpret_cast<const v4u*>(a + g0 * kGroup + sub * 8);
      const v4u r1 = *reinterpret_cast<const v4u*>(a + g1 * kGroup + sub * 8);
      quant_act_group(r0, g0, sub, true, aq, as);
      quant_act_group(r1, g1, sub, g0 + rows < groups, aq, as);
    }
  }
}

// One 128x128 block per 256-thread workgroup. Thread t covers 16-byte
// column chunk t % 32 of rows t / 32 + 8 j (j = 0..15); rows at or beyond N
// (short last row block) are skipped. amax: xor shuffles within each wave,
// then the four wave maxima through LDS.
__global__ __launch_bounds__(256) void quant_weight_kernel(const float* __restrict__ w,
                                                           unsigned char* __restrict__ wq,
                                                           float* __restrict__ ws, int64_t n,
                                                           int64_t k) {
  const int64_t g = blockIdx.x;        // K group
  const int64_t b = blockIdx.y;        // row block
  const int64_t groups = k / kGroup;
  const int t = threadIdx.x;
  const int col4 = t & 31;             // which 4-float chunk of the 128 columns
  const int64_t row0 = b * kGroup;
  const int64_t rows = (n - row0) < kGroup ? (n - row0) : kGroup;

  v4f v[16];
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = (t >> 5) + 8 * j;
    v[j] = v4f{0.f, 0.f, 0.f, 0.f};
    if (r < rows) {
      v[j] = *reinterpret_cast<const v4f*>(w + (row0 + r) * k + g * kGroup + col4 * 4);
      amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[j][0]), fabsf(v[j][1])), fmaxf(fabsf(v[j][2]), fabsf(v[j][3]))));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  __shared__ float wave_max[4];
  if ((t & 63) == 0) wave_max[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));

  const float s = group_scale(amax);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = (t >> 5) + 8 * j;
    if (r < rows) {
      const unsigned codes = encode4_e4m3(scaled_clamped(v[j][0], s), scaled_clamped(v[j][1], s),
                                          scaled_clamped(v[j][2], s), scaled_clamped(v[j][3], s));
      *reinterpret_cast<unsigned*>(wq + (row0 + r) * k + g * kGroup + col4 * 4) = codes;
    }
  }
  if (t == 0) ws[b * groups + g] = s;
}

hipError_t launch_quant_act(int64_t m, int64_t k, const void* a, void* aq, float* as, hipStream_t stream) {
  const int64_t groups = m * (k / kGroup);
  // 16 groups per 256-thread block and trip; at most 2048 blocks (8 per
  // CU), which then loop over pairs of groups
  constexpr int64_t kMaxBlocks = 2048;
  const int64_t blocks = (groups + 15) / 16;
  if (blocks <= kMaxBlocks) {
    hipLaunchKernelGGL(quant_act_kernel<false>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       static_cast<const unsigned short*>(a), static_cast<unsigned char*>(aq), as, groups);
  } else {
    hipLaunchKernelGGL(quant_act_kernel<true>, dim3(static_cast<unsigned>(kMaxBlocks)), dim3(256), 0, stream,
                       static_cast<const unsigned short*>(a), static_cast<unsigned char*>(aq), as, groups);
  }
  return hipGetLastError();
}

hipError_t launch_quant_weight(int64_t n, int64_t k, const float* w, void* wq, float* ws,
                               hipStream_t stream) {
  const int64_t nb = (n + kGroup - 1) / kGroup;
  hipLaunchKernelGGL(quant_weight_kernel, dim3(static_cast<unsigned>(k / kGroup), static_cast<unsigned>(nb)),
                     dim3(256), 0, stream, w, static_cast<unsigned char*>(wq), ws, n, k);
  return hipGetLastError();
}

}  // namespace fp8bq

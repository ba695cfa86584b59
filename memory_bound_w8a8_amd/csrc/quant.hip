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

// One 128-wide group per 16 lanes: each lane holds 8 bf16 (one 16-byte
// load), the 16 lanes of a DPP row reduce the amax with xor shuffles, then
// each lane divides, encodes and stores its 8 codes (8 bytes). Groups are
// contiguous in memory ([M, K] row-major, K % 128 == 0), so the kernel walks
// the flat group index m * (K / 128) + g.
__global__ __launch_bounds__(256) void quant_act_kernel(const unsigned short* __restrict__ a,
                                                        unsigned char* __restrict__ aq,
                                                        float* __restrict__ as, int64_t groups) {
  const int64_t gid = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  const bool valid = gid < groups;
  const int64_t g = valid ? gid : groups - 1;

  v4u raw = {0u, 0u, 0u, 0u};
  if (valid) raw = *reinterpret_cast<const v4u*>(a + g * kGroup + sub * 8);
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
  v2u out;
  out[0] = encode4_e4m3(scaled_clamped(x[0], s), scaled_clamped(x[1], s), scaled_clamped(x[2], s),
                        scaled_clamped(x[3], s));
  out[1] = encode4_e4m3(scaled_clamped(x[4], s), scaled_clamped(x[5], s), scaled_clamped(x[6], s),
                        scaled_clamped(x[7], s));
  if (valid) {
    *reinterpret_cast<v2u*>(aq + g * kGroup + sub * 8) = out;
    if (sub == 0) as[g] = s;
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
  const int64_t blocks = (groups + 15) / 16;  // 16 groups per 256-thread block
  hipLaunchKernelGGL(quant_act_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     static_cast<const unsigned short*>(a), static_cast<unsigned char*>(aq), as, groups);
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

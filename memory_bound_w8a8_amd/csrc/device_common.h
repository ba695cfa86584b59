// Device helpers shared by the fp8bq kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fp8bq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int kGroup = 128;       // K entries per scale group
constexpr float kE4m3Max = 448.f;  // largest finite e4m3fn magnitude

// 16x16 output tile, K = 128, both operands OCP e4m3fn, fresh fp32 result.
// Operand layout (gfx950 V_MFMA_F32_16X16X128_F8F6F4): lane l supplies row
// l % 16 of the first operand and column l % 16 of the second; the 32 bytes
// a lane holds are 32 K-slots determined by (l / 16, byte). The two operands
// use the same K-slot map, so any consistent placement of a row's 128 bytes
// gives the exact dot product. Result: lane l, element i holds row
// 4 * (l / 16) + i, column l % 16. Format code 0 selects e4m3 for both
// operands; zero scale operands select the unscaled instruction.
__device__ __forceinline__ v4f mfma_16x16x128_e4m3(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Same instruction accumulating into c.
__device__ __forceinline__ v4f mfma_16x16x128_e4m3_acc(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Two fp32 values to two bf16 (round to nearest even, V_CVT_PK_BF16_F32),
// packed low = lo, high = hi.
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  const v2f f = {lo, hi};
  const v2bf r = __builtin_convertvector(f, v2bf);
  return __builtin_bit_cast(unsigned, r);
}

// Four fp32 values to four e4m3fn codes, round to nearest even, byte i =
// code of the i-th argument (V_CVT_PK_FP8_F32). Magnitudes up to 464 round
// to the nearest code (those in (448, 464] to 448); above 464 the hardware
// gives the NaN code, so callers keep |x| <= 464.
__device__ __forceinline__ unsigned encode4_e4m3(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return static_cast<unsigned>(w);
}

// Raw buffer resource over [base, base + bytes) (bytes < 2^32). A buffer
// load whose per-lane byte offset (the VGPR part plus the instruction's
// immediate) is at or past `bytes` returns zeros without touching memory,
// which the kernels use to mask absent rows and tokens. The uniform SGPR
// offset of a load is kept in range by the caller and not relied on for that
// check. Word 3 is the gfx9-family raw-buffer format (32-bit data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}

// 16-byte and 4-byte buffer loads; the non-temporal form marks streamed data
// that is read once.
__device__ __forceinline__ v4u buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 0);
}
__device__ __forceinline__ v4u buffer_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(voff), static_cast<int>(soff), 2);
}
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(voff), static_cast<int>(soff), 0));
}

__device__ __forceinline__ v8i join8(const v4u& lo, const v4u& hi) {
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Scale of a group from its amax: IEEE fp32 division by 448, 1.0 for zero.
__device__ __forceinline__ float group_scale(float amax) { return amax > 0.f ? amax / kE4m3Max : 1.f; }

// Quotient clamped into the e4m3fn range; -0 stays -0.
__device__ __forceinline__ float scaled_clamped(float x, float s) {
  return fminf(fmaxf(x / s, -kE4m3Max), kE4m3Max);
}

// Exact-in-code quotient for e4m3 quantisation: Markstein's fma-based
// correction of a reciprocal-based quotient. The correctly rounded
// reciprocal y = 1 / s is formed once per group and, per value, q0 = x y,
// r = fma(-q0, s, x) (the exact residual), q = fma(r, y, q0). q is not
// always the correctly rounded x / s, but its e4m3 code (after the clamp) is
// that of the IEEE division for every bf16 x with |x| <= amax and every
// bf16 amax >= 2^-96: tests/quotient_check.c checks all 5.2e8 such pairs on
// the host, and the GPU tests compare the kernels' codes with the oracle for
// every bf16 x within 19 binades below every bf16 amax mantissa at 29
// exponents (subnormal maxima and the 2^-104 .. 2^-96 neighbourhood
// included). Callers take the IEEE division below amax = 2^-96.
// fma(r, y, q0) equals q0 when r == 0 and x != 0 (adding a zero to a
// non-zero value is exact) and has the sign of x otherwise; copysign(., x)
// only fixes x = -0, whose quotient must stay -0.
__device__ __forceinline__ float quotient_e4m3_range(float x, float s, float y) {
  const float q0 = x * y;
  const float r = fmaf(-q0, s, x);
  return fminf(fmaxf(copysignf(fmaf(r, y, q0), x), -kE4m3Max), kE4m3Max);
}

// Quotient for the quantisation inside the fused GEMM, where only the codes'
// values matter (a zero code adds nothing to a GEMM sum, whatever its sign).
// The reciprocal of s is kept as two floats, y_hi = 1 / s (correctly
// rounded) and y_lo = (1 - s y_hi) y_hi (the residual, one fma and one
// multiply), once per group; per value q = fma(x, y_hi, x y_lo): 2 VALU
// operations. For every bf16 x with |x| <= amax and every bf16 amax >= 2^-96
// the e4m3 code of q equals that of the IEEE division x / s except that
// x = -0 may give +0 (tests/quotient_check.c checks the same 5.2e8 pairs on
// the host). No clamp is needed: |q| <= 448 (1 + 2^-23), and the hardware
// conversion rounds magnitudes up to 464 to 448 (it returns the NaN code only
// above 464).
struct RecipPair {
  float hi, lo;
};
__device__ __forceinline__ RecipPair recip_pair(float s) {
  const float hi = 1.0f / s;
  return RecipPair{hi, fmaf(-s, hi, 1.0f) * hi};
}
__device__ __forceinline__ float quotient_e4m3_gemm(float x, const RecipPair& y) { return fmaf(x, y.hi, x * y.lo); }

}  // namespace fp8bq

// Measurement kernels: the denominators the GEMM's roofline fractions are
// read against on this machine, besides the published peaks.
//
// Page 1 (SmartX blog, "single-stream optimisation") reports a decode step
// as bytes moved per step over time against a calibrated bandwidth, and its
// "test background" section calibrates the tools before measuring. The same
// is done here with four kernels:
//  - a plain streaming read of a buffer (the most a weight-streaming GEMM of
//    that many bytes could reach per call, launch and ramp included);
//  - an empty kernel (the fixed cost of one launch in a stream);
//  - a loop of independent FP8 16x16x128 MFMAs (the matrix-core rate the
//    clock actually sustains), on one repeated code or on operands read from
//    memory (realistic data: the rate the power budget allows a GEMM), and
//    the same with the block-scaled GEMM's 4 scale FMAs per MFMA.
#include "device_common.h"
#include "launch.h"

namespace fp8bq {

namespace {

__device__ __forceinline__ unsigned xor4(const v4u& v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

// Streaming read of n16 16-byte units: consecutive lanes read consecutive
// units (1 KB per wave instruction), a grid-wide stride between a lane's
// units, twelve non-temporal loads in flight per lane per trip (lanes past
// the end skip theirs, so a transfer smaller than twelve grid-strides still
// has all of its loads in flight at once).
// Every lane XORs what it read; each workgroup writes the XOR over its lanes
// to sink[blockIdx.x], which keeps the loads live and lets a test check that
// every word was read exactly once.
constexpr int kReadBatch = 12;

__global__ __launch_bounds__(512) void mb_read_kernel(const v4u* __restrict__ src, int64_t n16,
                                                      unsigned* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 512;
  unsigned x = 0;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 512 + threadIdx.x; i < n16; i += kReadBatch * stride) {
    v4u v[kReadBatch];
#pragma unroll
    for (int u = 0; u < kReadBatch; ++u) {
      const int64_t j = i + u * stride;
      v[u] = v4u{0u, 0u, 0u, 0u};
      if (j < n16) v[u] = __builtin_nontemporal_load(src + j);
    }
#pragma unroll
    for (int u = 0; u < kReadBatch; ++u) x ^= xor4(v[u]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= static_cast<unsigned>(__shfl_xor(static_cast<int>(x), o));
  __shared__ unsigned part[8];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned y = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) y ^= part[w];
    sink[blockIdx.x] = y;
  }
}

__global__ void mb_empty_kernel() {}

// Eight independent accumulation chains of V_MFMA_F32_16X16X128_F8F6F4 per
// wave (the matrix core's issue rate, not its latency, bounds the loop).
// Both operands hold the e4m3 code `code` in every byte (a kernel argument,
// so nothing folds): every output of one MFMA is 128 * dec(code)^2, and
// thread t writes the sum of its 32 accumulator values,
// 8 * 4 * 128 * iters * dec(code)^2, to sink[t].
__global__ __launch_bounds__(256) void mb_mfma_kernel(int iters, unsigned code, float* __restrict__ sink) {
  const int word = static_cast<int>(code * 0x01010101u);
  const v8i a = {word, word, word, word, word, word, word, word};
  const v8i b = a;
  v4f acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = mfma_16x16x128_e4m3_acc(a, b, acc[u]);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) s += (acc[u][0] + acc[u][1]) + (acc[u][2] + acc[u][3]);
  sink[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;
}

// The same loop with operands read from memory: chain u's first and second
// operand in lane l are the 32 bytes at codes + 32 ((2 u + o) 64 + l),
// o = 0, 1 (32 KB, shared by every wave). With realistic codes (quantised
// Gaussian values rather than one repeated byte) the matrix core's switching
// activity, and with it the clock the chip can hold, is that of a real GEMM.
// Thread t writes the sum of its 32 accumulator values to sink[t].
//
// SCALED: the block-scaled GEMM's inner loop instead. Every MFMA starts from
// zero (one 128-wide scale group per instruction) and its result is folded
// into the chain's running sum by 4 fp32 FMAs with `scale`, one MFMA later
// (acc += scale * previous product), so the matrix core and the VALU work
// side by side as in the GEMM: thread t writes scale times the same sum.
template <bool SCALED>
__global__ __launch_bounds__(256) void mb_mfma_data_kernel(int iters, const v4u* __restrict__ codes, float scale,
                                                           float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  v8i a[8], b[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const v4u* pa = codes + 2 * ((2 * u) * 64 + lane);
    const v4u* pb = codes + 2 * ((2 * u + 1) * 64 + lane);
    a[u] = join8(pa[0], pa[1]);
    b[u] = join8(pb[0], pb[1]);
  }
  v4f acc[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = v4f{0.f, 0.f, 0.f, 0.f};
  if constexpr (SCALED) {
    v4f prev[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) prev[u] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const v4f p = mfma_16x16x128_e4m3(a[u], b[u]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[u][e] = fmaf(scale, prev[u][e], acc[u][e]);
        asm volatile("" : "+v"(acc[u]));
        prev[u] = p;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[u][e] = fmaf(scale, prev[u][e], acc[u][e]);
  } else {
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = mfma_16x16x128_e4m3_acc(a[u], b[u], acc[u]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) s += (acc[u][0] + acc[u][1]) + (acc[u][2] + acc[u][3]);
  sink[static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_mb_read(const void* buf, int64_t bytes, int grid, unsigned* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mb_read_kernel, dim3(grid), dim3(512), 0, stream, static_cast<const v4u*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_mb_empty(int grid, int block, hipStream_t stream) {
  hipLaunchKernelGGL(mb_empty_kernel, dim3(grid), dim3(block), 0, stream);
  return hipGetLastError();
}

hipError_t launch_mb_mfma(int grid, int iters, unsigned code, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mb_mfma_kernel, dim3(grid), dim3(256), 0, stream, iters, code, sink);
  return hipGetLastError();
}

hipError_t launch_mb_mfma_data(int grid, int iters, const void* codes, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mb_mfma_data_kernel<false>, dim3(grid), dim3(256), 0, stream, iters,
                     static_cast<const v4u*>(codes), 1.f, sink);
  return hipGetLastError();
}

hipError_t launch_mb_mfma_scaled(int grid, int iters, const void* codes, float scale, float* sink,
                                 hipStream_t stream) {
  hipLaunchKernelGGL(mb_mfma_data_kernel<true>, dim3(grid), dim3(256), 0, stream, iters,
                     static_cast<const v4u*>(codes), scale, sink);
  return hipGetLastError();
}

}  // namespace fp8bq

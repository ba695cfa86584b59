// Two-stage vocabulary scoring on gfx950: exact top-k of the coarse bf16
// logits, then exact bf16 rescoring of the survivors.
//
// Page 1 (SmartX blog, "Qwen3.8-27B performance optimisation"), section
// "single-stream optimisation": the draft head reads the whole vocabulary
// projection every step; screening all candidates with FP8 scores and scoring
// only the survivors exactly in BF16 cuts that traffic. The coarse logits
// come from the block-FP8 GEMM (fp8bq_gemm / fp8bq_gemm_fused); this file
// holds the selection and the rescoring.
//
// Order: a bf16 value's 16-bit key is its bit pattern mapped to a monotone
// unsigned order (negative patterns inverted, positive ones with the top bit
// set, so -0 sits just below +0); entries compare by key, equal keys by the
// lower index.
//
// Top-k, exact, with no atomics and no sort network: a wave holds up to 1024
// candidates (16 per lane, position 64 r + lane in register r) and selects
// its k best directly. It bisects the 16-bit key space for the k-th largest
// key t, counting candidates with a ballot and a popcount per register (16
// steps, no barriers); takes every candidate above t, and of those equal to t
// the lowest positions, ranked by ballot prefix counts; and writes the k
// chosen in position order. Candidate lists are kept in index order at every
// level, so position order is index order and ties go to the lower index.
//   launch 1: a workgroup of G waves per G chunks of 1024 logits; each wave
//             selects its chunk's k best into LDS, then wave 0 selects the
//             workgroup's k best from those G k candidates (G = min(4,
//             1024 / k));
//   launch 2+: a workgroup of up to min(16, 1024 / k) waves; each wave
//             selects the k best of 1024 / k lists, then wave 0 the k best
//             of the waves' results; repeated until a row has one list
//             (one merge launch for up to 256 first-level lists at k = 64).
// The last selection orders its k by (key descending, index ascending), each
// entry counting the entries ranked above it, and writes indices and values.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace fp8bq {

namespace {

constexpr int kPer = 16;                  // candidates per lane
constexpr int kWaveCand = 64 * kPer;      // candidates per wave
constexpr int kMaxGroup = 16;             // waves per workgroup (at most)
constexpr int kChunkGroup = 4;            // chunk waves per first-level workgroup

__device__ __forceinline__ unsigned key16(unsigned b) { return (b & 0x8000u) ? (~b & 0xffffu) : (b | 0x8000u); }
__device__ __forceinline__ unsigned unkey16(unsigned key) { return (key & 0x8000u) ? (key & 0x7fffu) : (~key & 0xffffu); }

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return static_cast<int>(
      __builtin_amdgcn_mbcnt_hi(static_cast<unsigned>(mask >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(mask), 0u)));
}

// Largest and smallest value over the wave: DPP within each row of 16 lanes
// (swap neighbours, swap pairs, mirror halves, mirror the row), then the four
// row results read as scalars.
template <int CTRL>
__device__ __forceinline__ unsigned dpp(unsigned v) {
  return static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ unsigned umax(unsigned a, unsigned b) { return a > b ? a : b; }
__device__ __forceinline__ unsigned umin(unsigned a, unsigned b) { return a < b ? a : b; }

__device__ __forceinline__ void wave_max_min(unsigned v, unsigned* vmax, unsigned* vmin) {
  unsigned hi = v, lo = v;
  hi = umax(hi, dpp<0xB1>(hi));  // quad_perm [1, 0, 3, 2]
  lo = umin(lo, dpp<0xB1>(lo));
  hi = umax(hi, dpp<0x4E>(hi));  // quad_perm [2, 3, 0, 1]
  lo = umin(lo, dpp<0x4E>(lo));
  hi = umax(hi, dpp<0x141>(hi));  // row_half_mirror
  lo = umin(lo, dpp<0x141>(lo));
  hi = umax(hi, dpp<0x140>(hi));  // row_mirror
  lo = umin(lo, dpp<0x140>(lo));
  *vmax = umax(umax(__builtin_amdgcn_readlane(hi, 0), __builtin_amdgcn_readlane(hi, 16)),
               umax(__builtin_amdgcn_readlane(hi, 32), __builtin_amdgcn_readlane(hi, 48)));
  *vmin = umin(umin(__builtin_amdgcn_readlane(lo, 0), __builtin_amdgcn_readlane(lo, 16)),
               umin(__builtin_amdgcn_readlane(lo, 32), __builtin_amdgcn_readlane(lo, 48)));
}

// Candidates: key[r] = 1 + the 16-bit key (0 = empty, never chosen), idx[r]
// its vocabulary index, at position 64 r + lane. Writes the k best -- by key,
// equal keys by lower position -- to dst[0 .. k) in position order, padded
// with empty entries when fewer than k are not empty. One whole wave calls it.
template <int PER>
__device__ __forceinline__ void wave_select(const unsigned (&key)[PER], const unsigned (&idx)[PER], int k, v2u* dst) {
  const int lane = threadIdx.x & 63;
  // t: the largest key with at least k candidates at or above it (1 when
  // fewer than k candidates are not empty). It lies in [lo, hi): hi is one
  // past the largest key; for k <= 64 every lane holds a key at or above the
  // smallest lane maximum, so that is a valid lo.
  unsigned lane_max = key[0];
#pragma unroll
  for (int r = 1; r < PER; ++r) lane_max = umax(lane_max, key[r]);
  unsigned wmax, wmin;
  wave_max_min(lane_max, &wmax, &wmin);
  unsigned hi = wmax + 1u;
  unsigned lo = (k <= 64 && wmin > 1u && wmin < hi) ? wmin : 1u;
  for (int step = 0; step < 17 && hi - lo > 1u; ++step) {
    const unsigned mid = (lo + hi) >> 1;
    int count = 0;
#pragma unroll
    for (int r = 0; r < PER; ++r) count += __popcll(__ballot(key[r] >= mid));
    if (count >= k) {
      lo = mid;
    } else {
      hi = mid;
    }
  }
  const unsigned t = lo;
  int above = 0;
#pragma unroll
  for (int r = 0; r < PER; ++r) above += __popcll(__ballot(key[r] > t));
  const int need = k - above;  // candidates equal to t to take, lowest positions first
  int ties_before = 0;
  int out = 0;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const unsigned long long tie = __ballot(key[r] == t);
    const bool take = key[r] > t || (key[r] == t && ties_before + lanes_below(tie) < need);
    ties_before += __popcll(tie);
    const unsigned long long taken = __ballot(take);
    if (take) dst[out + lanes_below(taken)] = v2u{key[r], idx[r]};
    out += __popcll(taken);
  }
  for (int j = out + lane; j < k; j += 64) dst[j] = v2u{0u, 0u};
}

// The k best of the n (<= 1024) candidates src[0 .. n) (position order),
// written to dst as wave_select does. One whole wave calls it.
template <int PER>
__device__ __forceinline__ void select_from(const v2u* src, int n, int k, v2u* dst) {
  const int lane = threadIdx.x & 63;
  unsigned key[PER], idx[PER];
  // every load in bounds (index clamped to n - 1) and unconditional, so the
  // PER loads are in flight together; positions past n become empty
  const int last = n > 0 ? n - 1 : 0;
  v2u e[PER];
  if (n > 0) {
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int p = 64 * r + lane;
      e[r] = src[p < n ? p : last];
    }
#pragma unroll
    for (int r = 0; r < PER; ++r) asm volatile("" : "+v"(e[r]));
  } else {
#pragma unroll
    for (int r = 0; r < PER; ++r) e[r] = v2u{0u, 0u};
  }
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    const int p = 64 * r + lane;
    key[r] = p < n ? e[r][0] : 0u;
    idx[r] = e[r][1];
  }
  wave_select<PER>(key, idx, k, dst);
}

__device__ __forceinline__ void select_list(const v2u* src, int n, int k, v2u* dst) {
  if (n <= 256) {
    select_from<4>(src, n, k, dst);
  } else {
    select_from<16>(src, n, k, dst);
  }
}

// sel[0 .. k): a row's k best in position order (all non-empty). Writes them
// ordered by (key descending, position ascending): each entry's slot is the
// number of entries ranked above it. One whole wave calls it.
__device__ __forceinline__ void wave_place(const v2u* sel, int k, int* __restrict__ out_idx, unsigned short* __restrict__ out_val) {
  const int lane = threadIdx.x & 63;
  for (int i = lane; i < k; i += 64) {
    const v2u e = sel[i];
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < k; ++j) {
      const v2u f = sel[j];
      rank += (f[0] > e[0]) | ((f[0] == e[0]) & (j < i));
    }
    out_idx[rank] = static_cast<int>(e[1]);
    out_val[rank] = static_cast<unsigned short>(unkey16(e[0] - 1u));
  }
}

__global__ __launch_bounds__(64 * kMaxGroup) void topk_chunk_kernel(int64_t v, int k, int group, int parts,
                                                                    const unsigned short* __restrict__ logits,
                                                                    v2u* __restrict__ lists,
                                                                    int* __restrict__ out_idx,
                                                                    unsigned short* __restrict__ out_val) {
  __shared__ v2u wave_lists[kWaveCand];  // group * k <= 1024
  __shared__ v2u best[256];
  const int64_t row = blockIdx.x / parts;
  const int part = static_cast<int>(blockIdx.x - row * parts);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t base = (static_cast<int64_t>(part) * group + wave) * kWaveCand;
  const unsigned short* x = logits + row * v;
  unsigned key[kPer], idx[kPer];
  // loads from clamped (in-bounds) positions, all issued before any is
  // used (the empty asm keeps the compiler from moving each load into a
  // branch on pos < v, which would wait for the loads one at a time);
  // positions past the row become empty
  unsigned raw[kPer];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int64_t pos = base + 64 * r + lane;
    raw[r] = x[pos < v ? pos : v - 1];
  }
#pragma unroll
  for (int r = 0; r < kPer; ++r) asm volatile("" : "+v"(raw[r]));
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int64_t pos = base + 64 * r + lane;
    key[r] = pos < v ? key16(raw[r]) + 1u : 0u;
    idx[r] = static_cast<unsigned>(pos);
  }
  wave_select<kPer>(key, idx, k, wave_lists + wave * k);
  __syncthreads();
  if (wave != 0) return;
  if (parts > 1) {
    select_list(wave_lists, group * k, k, lists + (row * parts + part) * k);
  } else {
    select_list(wave_lists, group * k, k, best);
    __builtin_amdgcn_wave_barrier();
    wave_place(best, k, out_idx + row * k, out_val + row * k);
  }
}

// Merges `lists` lists of k per row: wave w of a workgroup selects the k
// best of `fan` consecutive lists, then wave 0 selects the k best of the
// waves' results, so a workgroup turns `fan` * (its waves) lists into one
// list of `next`, or, on the last level, into the row's ordered output.
__global__ __launch_bounds__(64 * kMaxGroup) void topk_merge_kernel(int k, int lists, int fan,
                                                                    const v2u* __restrict__ src,
                                                                    v2u* __restrict__ next, int* __restrict__ out_idx,
                                                                    unsigned short* __restrict__ out_val) {
  __shared__ v2u wave_lists[kWaveCand];  // waves * k <= 1024
  __shared__ v2u best[256];
  const int waves = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6;
  const int span = fan * waves;
  const int lists_out = (lists + span - 1) / span;
  const int64_t row = blockIdx.x / lists_out;
  const int part = static_cast<int>(blockIdx.x - row * lists_out);
  const int first = part * span + wave * fan;
  const int count = lists - first < fan ? lists - first : fan;  // may be <= 0: no candidates
  select_list(src + (row * lists + first) * k, count > 0 ? count * k : 0, k, wave_lists + wave * k);
  __syncthreads();
  if (wave != 0) return;
  if (lists_out > 1) {
    select_list(wave_lists, waves * k, k, next + (row * lists_out + part) * k);
  } else {
    select_list(wave_lists, waves * k, k, best);
    __builtin_amdgcn_wave_barrier();
    wave_place(best, k, out_idx + row * k, out_val + row * k);
  }
}

// Exact rescoring: wave w of workgroup (row, b) scores survivor 16 b + w.
// Lane l multiplies the bf16 pairs of the 16-byte pieces l, l + 64, ... of
// the two K rows (products exact in fp32), accumulating in fp32 in that
// order, element by element; the 64 lane sums are then added by xor
// butterflies (distance 32, 16, ..., 1). A survivor index outside [0, V)
// reads nothing and scores NaN.
constexpr int kRescoreWaves = 16;

__device__ __forceinline__ float bf16_lo_f(unsigned w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi_f(unsigned w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

__device__ __forceinline__ float dot8(v4u a, v4u b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = fmaf(bf16_lo_f(a[i]), bf16_lo_f(b[i]), acc);
    acc = fmaf(bf16_hi_f(a[i]), bf16_hi_f(b[i]), acc);
  }
  return acc;
}

__global__ __launch_bounds__(64 * kRescoreWaves) void rescore_kernel(int64_t kdim, int64_t v, int k, int blocks_per_row,
                                                                     const unsigned short* __restrict__ h,
                                                                     const unsigned short* __restrict__ w,
                                                                     const int* __restrict__ idx,
                                                                     float* __restrict__ scores) {
  const int64_t row = blockIdx.x / blocks_per_row;
  const int b = static_cast<int>(blockIdx.x - row * blocks_per_row);
  const int lane = threadIdx.x & 63;
  const int j = b * kRescoreWaves + (threadIdx.x >> 6);
  if (j >= k) return;
  const int r = idx[row * k + j];
  if (r < 0 || r >= v) {
    if (lane == 0) scores[row * k + j] = __builtin_nanf("");
    return;
  }
  const v4u* hrow = reinterpret_cast<const v4u*>(h + row * kdim);
  const v4u* wrow = reinterpret_cast<const v4u*>(w + static_cast<int64_t>(r) * kdim);
  const int64_t pieces = kdim >> 3;
  float acc = 0.f;
  // Batches of kBatch pieces per lane: every load of a batch is issued
  // before the first product waits (K up to 6144 is one memory round trip),
  // then the products are accumulated in piece order as before.
  constexpr int kBatch = 12;
  for (int64_t base = lane; base < pieces; base += 64 * kBatch) {
    v4u hv[kBatch], wv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int64_t i = base + 64 * u;
      if (i < pieces) {
        hv[u] = hrow[i];
        wv[u] = __builtin_nontemporal_load(wrow + i);
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (base + 64 * u < pieces) acc = dot8(hv[u], wv[u], acc);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (lane == 0) scores[row * k + j] = acc;
}

// Best survivor of each row by (score descending, index ascending); NaN
// scores never win; -1 when every score is NaN. One wave per row.
__global__ __launch_bounds__(64) void pick_kernel(int k, const int* __restrict__ idx, const float* __restrict__ scores,
                                                  int* __restrict__ pick) {
  const int64_t row = blockIdx.x;
  float best = 0.f;
  int bi = -1;
  for (int j = threadIdx.x; j < k; j += 64) {
    const float s = scores[row * k + j];
    const int r = idx[row * k + j];
    if (s == s && (bi < 0 || s > best || (s == best && r < bi))) {
      best = s;
      bi = r;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float s = __shfl_xor(best, off);
    const int r = __shfl_xor(bi, off);
    if (r >= 0 && (bi < 0 || s > best || (s == best && r < bi))) {
      best = s;
      bi = r;
    }
  }
  if (threadIdx.x == 0) pick[row] = bi;
}

int topk_group(int64_t k) { return static_cast<int>(kChunkGroup < kWaveCand / k ? kChunkGroup : kWaveCand / k); }

// Waves of a merge workgroup: each takes kWaveCand / k lists; the workgroup
// holds no more waves than its lists need, nor more than wave 0 can merge.
int merge_waves(int lists, int k) {
  const int fan = kWaveCand / k;
  const int cap = kMaxGroup < kWaveCand / k ? kMaxGroup : kWaveCand / k;
  const int need = (lists + fan - 1) / fan;
  return need < cap ? need : cap;
}

int64_t topk_parts(int64_t v, int64_t k) {
  const int64_t chunks = (v + kWaveCand - 1) / kWaveCand;
  return (chunks + topk_group(k) - 1) / topk_group(k);
}

}  // namespace

int64_t topk_workspace_bytes(int64_t m, int64_t v, int64_t k) {
  const int64_t l1 = topk_parts(v, k);
  const int64_t fan = kWaveCand / k;
  const int64_t l2 = (l1 + fan - 1) / fan;
  return (l1 + l2) * m * k * static_cast<int64_t>(sizeof(v2u));
}

int64_t topk_grid_blocks(int64_t m, int64_t v, int64_t k) { return m * topk_parts(v, k); }

hipError_t launch_topk(int64_t m, int64_t v, int k, const void* logits, void* workspace, int* idx, void* val,
                       hipStream_t stream) {
  const int group = topk_group(k);
  const int fan = kWaveCand / k;
  int lists = static_cast<int>(topk_parts(v, k));
  auto* a = static_cast<v2u*>(workspace);
  auto* b = a + static_cast<int64_t>(lists) * m * k;  // the next level's lists
  auto* out_val = static_cast<unsigned short*>(val);
  hipLaunchKernelGGL(topk_chunk_kernel, dim3(static_cast<unsigned>(m * lists)), dim3(64 * group), 0, stream, v, k,
                     group, lists, static_cast<const unsigned short*>(logits), a, idx, out_val);
  hipError_t e = hipGetLastError();
  while (e == hipSuccess && lists > 1) {
    const int waves = merge_waves(lists, k);
    const int lists_out = (lists + fan * waves - 1) / (fan * waves);
    hipLaunchKernelGGL(topk_merge_kernel, dim3(static_cast<unsigned>(m * lists_out)), dim3(64 * waves), 0, stream, k,
                       lists, fan, a, b, idx, out_val);
    e = hipGetLastError();
    lists = lists_out;
    auto* t = a;
    a = b;
    b = t;
  }
  return e;
}

// Workspace of fp8bq_topk_bf16_noalloc: a static device array, one copy per
// GPU for the life of the process. In host code `scratch` names a host-side
// stand-in, not the device memory: the device address comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept per device; only that pointer is ever passed to a kernel. The top-k
// kernels ignore the workspace's contents on entry, so nothing is cleared.
// Every no-allocation call on one GPU shares the array: calls that overlap
// on one GPU (different streams, or threads without ordering) race.
static __device__ __align__(256) unsigned char scratch[kTopkScratchBytes];

namespace {

constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchMaxDevices];

}  // namespace

hipError_t topk_scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_topk_noalloc(int64_t m, int64_t v, int k, const void* logits, int* idx, void* val,
                               hipStream_t stream) {
  if (topk_workspace_bytes(m, v, k) > kTopkScratchBytes) return hipErrorInvalidValue;
  void* ws = nullptr;
  const hipError_t e = topk_scratch_address(&ws);
  if (e != hipSuccess) return e;
  return launch_topk(m, v, k, logits, ws, idx, val, stream);
}

int64_t rescore_grid_blocks(int64_t m, int64_t k) { return m * ((k + kRescoreWaves - 1) / kRescoreWaves); }

hipError_t launch_rescore(int64_t m, int64_t kdim, int64_t v, int64_t k, const void* h, const void* w,
                          const int* idx, float* scores, int* pick, hipStream_t stream) {
  const int blocks_per_row = static_cast<int>((k + kRescoreWaves - 1) / kRescoreWaves);
  hipLaunchKernelGGL(rescore_kernel, dim3(static_cast<unsigned>(m * blocks_per_row)), dim3(64 * kRescoreWaves), 0,
                     stream, kdim, v, static_cast<int>(k), blocks_per_row, static_cast<const unsigned short*>(h),
                     static_cast<const unsigned short*>(w), idx, scores);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pick_kernel, dim3(static_cast<unsigned>(m)), dim3(64), 0, stream, static_cast<int>(k), idx, scores,
                     pick);
  return hipGetLastError();
}

}  // namespace fp8bq

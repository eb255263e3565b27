// Scored-window statistics ("Qwen3.8-27B Quantization Challenge": "Golden
// distributions" -- the first score_from positions of a document are not
// scored -- and "The score" -- the mean over all positions and over a subset
// such as the long traces; "Qwen3.8-27B fidelity suite v5": exact exceedance
// counts and the score_from 0 / 256 / 1024 window control).
//
// One block per segment sums its scored values in a fixed order (f64) and
// counts them and their exceedances; one block then adds the segments'
// sums and counts in a fixed order.  No atomics: results are bitwise
// reproducible.
#include "kld.h"
#include "kld_device.hpp"
#include "kld_launch.hpp"

namespace kld {

namespace {

constexpr int WT = 256;
constexpr int WU = 4;   // loads in flight per thread

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long x) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// One block per segment.  Each thread keeps WU loads in flight, a running
// f64 sum and one exceedance counter per threshold; waves reduce with a fixed
// butterfly, then thread 0 adds the four wave results in order.
__global__ __launch_bounds__(WT) void window_seg_kernel(
    const float *__restrict__ kl, int64_t n, const int64_t *__restrict__ offsets,
    int64_t score_from, WindowThresholds thr, double *__restrict__ seg_sum,
    int64_t *__restrict__ seg_count, int64_t *__restrict__ seg_exceed) {
  __shared__ double wsum[WT / 64];
  __shared__ unsigned int wcnt[WT / 64][KLD_MAX_THRESHOLDS];
  const int64_t seg = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t a = offsets[seg], b = offsets[seg + 1];
  const bool bad = a < 0 || b < a || b > n;
  const int64_t s = !bad && b - a > score_from ? a + score_from : b;
  double acc = 0.0;
  unsigned int c[KLD_MAX_THRESHOLDS];
#pragma unroll
  for (int t = 0; t < KLD_MAX_THRESHOLDS; ++t) c[t] = 0u;
  // Loads go through a buffer resource over [s, b): offsets past it read 0
  // and touch no memory, so the loop has no branch around a load (a branch
  // would make every load wait for the one before).  Segments are read in
  // pieces of at most 2^28 positions so that byte offsets fit 31 bits.
  for (int64_t p0 = s; p0 < b; p0 += (int64_t)1 << 28) {
  const int64_t pn = b - p0 < ((int64_t)1 << 28) ? b - p0 : ((int64_t)1 << 28);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float *>(kl + p0), (short)0, (int)(pn * 4), 0x00020000);
  for (int j0 = threadIdx.x; j0 < pn; j0 += WT * WU) {
    float x[WU];
#pragma unroll
    for (int u = 0; u < WU; ++u)
      x[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                 rs, (j0 + u * WT) * 4, 0, 2 /* streaming */));
#pragma unroll
    for (int u = 0; u < WU; ++u) {
      const bool in = j0 + u * WT < pn;
      acc += (double)x[u];
#pragma unroll
      for (int t = 0; t < KLD_MAX_THRESHOLDS; ++t)
        c[t] += (t < thr.count && in && x[u] > thr.value[t]) ? 1u : 0u;
    }
  }
  }
  acc = wave_sum_f64(acc);
  if (lane == 0) wsum[wave] = acc;
  for (int t = 0; t < thr.count; ++t) {
    const unsigned long long w = wave_sum_u64(c[t]);
    if (lane == 0) wcnt[wave][t] = (unsigned int)w;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
#pragma unroll
    for (int w = 0; w < WT / 64; ++w) sum += wsum[w];
    seg_sum[seg] = bad ? __builtin_nan("") : sum;
    seg_count[seg] = bad ? 0 : b - s;
  }
  if ((int)threadIdx.x < thr.count) {
    unsigned long long e = 0;
#pragma unroll
    for (int w = 0; w < WT / 64; ++w) e += wcnt[w][threadIdx.x];
    seg_exceed[seg * thr.count + threadIdx.x] = (int64_t)e;
  }
}

// One block: the totals over every segment in a fixed order.  A malformed
// segment's NaN sum makes the mean NaN.
constexpr int TT = 1024;

__global__ __launch_bounds__(TT) void window_total_kernel(
    const double *__restrict__ seg_sum, const int64_t *__restrict__ seg_count,
    const int64_t *__restrict__ seg_exceed, int64_t nseg, int nthr, double *__restrict__ totals) {
  __shared__ double wsum[TT / 64];
  __shared__ unsigned long long wcnt[TT / 64][KLD_MAX_THRESHOLDS + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double acc = 0.0;
  unsigned long long c[KLD_MAX_THRESHOLDS + 1];
#pragma unroll
  for (int t = 0; t <= KLD_MAX_THRESHOLDS; ++t) c[t] = 0ull;
  // every load unconditional (a clamped, valid index) so that an
  // iteration's loads are all in flight at once
  for (int64_t i = threadIdx.x; i < nseg; i += TT) {
    acc += seg_sum[i];
    c[KLD_MAX_THRESHOLDS] += (unsigned long long)seg_count[i];
    if (nthr > 0) {
      const int64_t *row = seg_exceed + i * nthr;
      int64_t e[KLD_MAX_THRESHOLDS];
#pragma unroll
      for (int t = 0; t < KLD_MAX_THRESHOLDS; ++t) e[t] = row[t < nthr ? t : 0];
#pragma unroll
      for (int t = 0; t < KLD_MAX_THRESHOLDS; ++t) c[t] += t < nthr ? (unsigned long long)e[t] : 0ull;
    }
  }
  acc = wave_sum_f64(acc);
  if (lane == 0) wsum[wave] = acc;
#pragma unroll
  for (int t = 0; t <= KLD_MAX_THRESHOLDS; ++t) {
    const unsigned long long w = wave_sum_u64(c[t]);
    if (lane == 0) wcnt[wave][t] = w;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
    unsigned long long cnt = 0;
#pragma unroll
    for (int w = 0; w < TT / 64; ++w) {
      sum += wsum[w];
      cnt += wcnt[w][KLD_MAX_THRESHOLDS];
    }
    totals[0] = cnt == 0ull ? __builtin_nan("") : sum / (double)cnt;
    totals[1] = (double)cnt;
  }
  if ((int)threadIdx.x < nthr) {
    unsigned long long e = 0;
#pragma unroll
    for (int w = 0; w < TT / 64; ++w) e += wcnt[w][threadIdx.x];
    totals[2 + threadIdx.x] = (double)e;
  }
}

}  // namespace

hipError_t launch_window_summary(const float *kl, int64_t n, const int64_t *offsets, int64_t nseg,
                                 int64_t score_from, const WindowThresholds &thr, double *seg_sum,
                                 int64_t *seg_count, int64_t *seg_exceed, double *totals,
                                 hipStream_t stream) {
  if (nseg > 0) {
    hipLaunchKernelGGL(window_seg_kernel, dim3((unsigned)nseg), dim3(WT), 0, stream, kl, n,
                       offsets, score_from, thr, seg_sum, seg_count, seg_exceed);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(window_total_kernel, dim3(1), dim3(TT), 0, stream, seg_sum, seg_count,
                     seg_exceed, nseg, thr.count, totals);
  return hipGetLastError();
}

}  // namespace kld

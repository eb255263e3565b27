// Scored-window statistics ("Qwen3.8-27B Quantization Challenge": "Golden
// distributions" -- the first score_from positions of a document are not
// scored -- and "The score" -- the mean over all positions and over a subset
// such as the long traces; "Qwen3.8-27B fidelity suite v5": exact exceedance
// counts and the score_from 0 / 256 / 1024 window control).
//
// One block per segment sums its scored values in a fixed order (f64) and
// counts them and their exceedances; the exceedance counts of all segments
// go to integer counters (exact in any order); one block then adds the
// segment sums in segment order.  Results are bitwise reproducible.
#include "kld.h"
#include "kld_device.hpp"
#include "kld_launch.hpp"

namespace kld {

namespace {

constexpr int WT = 256;

__global__ __launch_bounds__(WT) void window_zero_kernel(unsigned long long *counters, int m) {
  if ((int)threadIdx.x < m) counters[threadIdx.x] = 0ull;
}

__global__ __launch_bounds__(WT) void window_seg_kernel(
    const float *__restrict__ kl, int64_t n, const int64_t *__restrict__ offsets,
    int64_t score_from, WindowThresholds thr, double *__restrict__ seg_sum,
    int64_t *__restrict__ seg_count, unsigned long long *__restrict__ counters) {
  __shared__ double red[WT];
  __shared__ unsigned int cnt[KLD_MAX_THRESHOLDS];
  const int64_t seg = blockIdx.x;
  const int64_t a = offsets[seg], b = offsets[seg + 1];
  const bool bad = a < 0 || b < a || b > n;
  const int64_t s = !bad && b - a > score_from ? a + score_from : b;
  if ((int)threadIdx.x < KLD_MAX_THRESHOLDS) cnt[threadIdx.x] = 0u;
  __syncthreads();
  double acc = 0.0;
  unsigned int c[KLD_MAX_THRESHOLDS];
#pragma unroll
  for (int t = 0; t < KLD_MAX_THRESHOLDS; ++t) c[t] = 0u;
  if (!bad) {
    for (int64_t j = s + threadIdx.x; j < b; j += WT) {
      const float x = kl[j];
      acc += (double)x;
#pragma unroll
      for (int t = 0; t < KLD_MAX_THRESHOLDS; ++t)
        if (t < thr.count && x > thr.value[t]) ++c[t];
    }
  }
#pragma unroll
  for (int t = 0; t < KLD_MAX_THRESHOLDS; ++t)
    if (t < thr.count && c[t]) atomicAdd(&cnt[t], c[t]);
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int h = WT / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    seg_sum[seg] = bad ? __builtin_nan("") : red[0];
    seg_count[seg] = bad ? 0 : b - s;
    if (bad) atomicAdd(&counters[KLD_MAX_THRESHOLDS], 1ull);
  }
  if ((int)threadIdx.x < thr.count && cnt[threadIdx.x])
    atomicAdd(&counters[threadIdx.x], (unsigned long long)cnt[threadIdx.x]);
}

__global__ __launch_bounds__(WT) void window_total_kernel(
    const double *__restrict__ seg_sum, const int64_t *__restrict__ seg_count, int64_t nseg,
    const unsigned long long *__restrict__ counters, int nthr, double *__restrict__ totals) {
  __shared__ double red[WT];
  __shared__ unsigned long long rc[WT];
  double acc = 0.0;
  unsigned long long c = 0ull;
  for (int64_t i = threadIdx.x; i < nseg; i += WT) {
    acc += seg_sum[i];
    c += (unsigned long long)seg_count[i];
  }
  red[threadIdx.x] = acc;
  rc[threadIdx.x] = c;
  __syncthreads();
  for (int h = WT / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) {
      red[threadIdx.x] += red[threadIdx.x + h];
      rc[threadIdx.x] += rc[threadIdx.x + h];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const bool bad = counters[KLD_MAX_THRESHOLDS] != 0ull;
    const double cnt = (double)rc[0];
    totals[0] = bad || rc[0] == 0ull ? __builtin_nan("") : red[0] / cnt;
    totals[1] = cnt;
  }
  if ((int)threadIdx.x < nthr) totals[2 + threadIdx.x] = (double)counters[threadIdx.x];
}

}  // namespace

hipError_t launch_window_summary(const float *kl, int64_t n, const int64_t *offsets, int64_t nseg,
                                 int64_t score_from, const WindowThresholds &thr, double *seg_sum,
                                 int64_t *seg_count, double *totals, void *ws, hipStream_t stream) {
  unsigned long long *counters = static_cast<unsigned long long *>(ws);
  hipLaunchKernelGGL(window_zero_kernel, dim3(1), dim3(WT), 0, stream, counters,
                     KLD_MAX_THRESHOLDS + 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nseg > 0) {
    hipLaunchKernelGGL(window_seg_kernel, dim3((unsigned)nseg), dim3(WT), 0, stream, kl, n,
                       offsets, score_from, thr, seg_sum, seg_count, counters);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(window_total_kernel, dim3(1), dim3(WT), 0, stream, seg_sum, seg_count, nseg,
                     counters, thr.count, totals);
  return hipGetLastError();
}

}  // namespace kld

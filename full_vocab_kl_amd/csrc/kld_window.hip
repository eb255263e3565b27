// Scored-window statistics ("Qwen3.8-27B Quantization Challenge": "Golden
// distributions" -- the first score_from positions of a document are not
// scored -- and "The score" -- the mean over all positions and over a subset
// such as the long traces; "Qwen3.8-27B fidelity suite v5": exact exceedance
// counts and the score_from 0 / 256 / 1024 window control).
//
// One block per segment (one wave when segments are short) sums its scored
// values in a fixed order (f64) and counts them and their exceedances; one
// block then adds the segments' sums and counts in a fixed order.  No atomics: results are bitwise
// reproducible.
#include "kld.h"
#include "kld_device.hpp"
#include "kld_launch.hpp"

namespace kld {

namespace {

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

// Exceedance counting.  The host pads the threshold list with +inf up to NT
// (0, 4, 8 or 16), so every position meets exactly NT compares and no
// per-threshold predicate; a position past the segment is replaced by -inf
// once, which exceeds nothing.  NaN scores exceed nothing either.
template <int NT>
__device__ __forceinline__ void count_exceed(float x, unsigned int (&c)[NT > 0 ? NT : 1],
                                             const WindowThresholds &thr) {
#pragma unroll
  for (int t = 0; t < NT; ++t) c[t] += x > thr.value[t] ? 1u : 0u;
}

// Sums NT per-lane counters over a wave: afterwards lane l holds the sum of
// counter l / (64 / NT).  Each step hands half of the counters still held to
// the partner lane (reduce-scatter), then a butterfly finishes, so the wave
// needs 6 exchange rounds in all instead of 6 per counter.
template <int NT>
__device__ __forceinline__ unsigned long long wave_scatter_sum(unsigned long long (&c)[NT],
                                                               int lane) {
#pragma unroll
  for (int k = NT, m = 32; k > 1; k >>= 1, m >>= 1) {
    const bool hi = (lane & m) != 0;
#pragma unroll
    for (int i = 0; i < k / 2; ++i) {
      const unsigned long long send = hi ? c[i] : c[i + k / 2];
      const unsigned long long keep = hi ? c[i + k / 2] : c[i];
      c[i] = keep + __shfl_xor(send, m);
    }
  }
  unsigned long long x = c[0];
#pragma unroll
  for (int m = 64 / NT / 2; m > 0; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// The scored range [s, b) of segment seg, read through a buffer resource:
// offsets past it read 0 and touch no memory, so the loop has no branch
// around a load (a branch would make every load wait for the one before).
// Segments are read in pieces of at most 2^28 positions so that byte
// offsets fit 31 bits.  Lane i of the T cooperating threads takes positions
// i, i + T, ... in a fixed order.
template <int T, int WU, int NT>
__device__ __forceinline__ void scan_segment(const float *kl, int64_t s, int64_t b, int i,
                                             const WindowThresholds &thr, double &acc,
                                             unsigned int (&c)[NT > 0 ? NT : 1]) {
  for (int64_t p0 = s; p0 < b; p0 += (int64_t)1 << 28) {
    const int64_t pn = b - p0 < ((int64_t)1 << 28) ? b - p0 : ((int64_t)1 << 28);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(kl + p0), (short)0, (int)(pn * 4), 0x00020000);
    for (int j0 = i; j0 < pn; j0 += T * WU) {
      float x[WU];
#pragma unroll
      for (int u = 0; u < WU; ++u)
        x[u] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                   rs, (j0 + u * T) * 4, 0, 2 /* streaming */));
#pragma unroll
      for (int u = 0; u < WU; ++u) {
        acc += (double)x[u];   // 0 past the end
        count_exceed<NT>(j0 + u * T < (int)pn ? x[u] : -__builtin_inff(), c, thr);
      }
    }
  }
}

// Long segments: one segment per block of WT threads.  Waves reduce with the
// fixed butterflies above, then the wave results are added in order.
template <int WT, int WU, int NT>
__global__ __launch_bounds__(WT) void window_seg_kernel(
    const float *__restrict__ kl, int64_t n, const int64_t *__restrict__ offsets,
    int64_t score_from, WindowThresholds thr, double *__restrict__ seg_sum,
    int64_t *__restrict__ seg_count, int64_t *__restrict__ seg_exceed) {
  __shared__ double wsum[WT / 64];
  __shared__ unsigned long long wcnt[WT / 64][NT > 0 ? NT : 1];
  const int64_t seg = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t a = offsets[seg], b = offsets[seg + 1];
  const bool bad = a < 0 || b < a || b > n;
  const int64_t s = !bad && b - a > score_from ? a + score_from : b;
  double acc = 0.0;
  unsigned int c[NT > 0 ? NT : 1];
#pragma unroll
  for (int t = 0; t < (NT > 0 ? NT : 1); ++t) c[t] = 0u;
  scan_segment<WT, WU, NT>(kl, s, b, threadIdx.x, thr, acc, c);
  acc = wave_sum_f64(acc);
  if (lane == 0) wsum[wave] = acc;
  if constexpr (NT > 0) {
    unsigned long long cw[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) cw[t] = c[t];
    const unsigned long long e = wave_scatter_sum<NT>(cw, lane);
    if (lane % (64 / NT) == 0) wcnt[wave][lane / (64 / NT)] = e;
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

// Short segments: one wave per segment, SW segments per block, so that a
// whole batch of segments is resident at once and the launch costs about
// one round of load latency.
template <int SW, int WU, int NT>
__global__ __launch_bounds__(64 * SW) void window_seg_wave_kernel(
    const float *__restrict__ kl, int64_t n, const int64_t *__restrict__ offsets, int64_t nseg,
    int64_t score_from, WindowThresholds thr, double *__restrict__ seg_sum,
    int64_t *__restrict__ seg_count, int64_t *__restrict__ seg_exceed) {
  const int lane = threadIdx.x & 63;
  // the wave index made visibly uniform, so that the segment bounds and the
  // buffer resource live in scalar registers
  const int64_t seg = (int64_t)blockIdx.x * SW + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (seg >= nseg) return;   // whole waves; no barrier below
  const int64_t a = offsets[seg], b = offsets[seg + 1];
  const bool bad = a < 0 || b < a || b > n;
  const int64_t s = !bad && b - a > score_from ? a + score_from : b;
  double acc = 0.0;
  unsigned int c[NT > 0 ? NT : 1];
#pragma unroll
  for (int t = 0; t < (NT > 0 ? NT : 1); ++t) c[t] = 0u;
  scan_segment<64, WU, NT>(kl, s, b, lane, thr, acc, c);
  acc = wave_sum_f64(acc);
  if constexpr (NT > 0) {
    unsigned long long cw[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) cw[t] = c[t];
    const unsigned long long e = wave_scatter_sum<NT>(cw, lane);
    const int t = lane / (64 / NT);
    if (lane % (64 / NT) == 0 && t < thr.count) seg_exceed[seg * thr.count + t] = (int64_t)e;
  }
  if (lane == 0) {
    seg_sum[seg] = bad ? __builtin_nan("") : acc;
    seg_count[seg] = bad ? 0 : b - s;
  }
}

// One block: the totals over every segment in a fixed order.  A malformed
// segment's NaN sum makes the mean NaN.  Every array is read with coalesced,
// unconditional (clamped) loads, TR per thread in flight: the sums and counts
// by segment index, the exceedance counts as one flat [nseg * nthr] array
// with a stride that is a multiple of nthr, so that each thread only ever
// meets one threshold's column.
constexpr int TT = 1024;
constexpr int TR = 8;

__global__ __launch_bounds__(TT) void window_total_kernel(
    const double *__restrict__ seg_sum, const int64_t *__restrict__ seg_count,
    const int64_t *__restrict__ seg_exceed, int64_t nseg, int nthr, double *__restrict__ totals) {
  __shared__ double wsum[TT / 64];
  __shared__ unsigned long long wcnt[TT / 64];
  __shared__ unsigned long long part[TT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t last = nseg > 0 ? nseg - 1 : 0;
  double acc = 0.0;
  unsigned long long cnt = 0;
  if (nseg > 0) {
    for (int64_t i0 = threadIdx.x; i0 < nseg; i0 += (int64_t)TT * TR) {
      double v[TR];
      int64_t k[TR];
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        const int64_t i = i0 + (int64_t)r * TT;
        v[r] = seg_sum[i < nseg ? i : last];
        k[r] = seg_count[i < nseg ? i : last];
      }
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        const bool in = i0 + (int64_t)r * TT < nseg;
        acc += in ? v[r] : 0.0;
        cnt += in ? (unsigned long long)k[r] : 0ull;
      }
    }
  }
  // exceedance counts: thread j < stride sums the flat entries j, j + stride,
  // ... (all in column j % nthr)
  const int stride = nthr > 0 ? TT - TT % nthr : 0;
  const int64_t flat = nseg * (int64_t)nthr;
  unsigned long long e = 0;
  if ((int)threadIdx.x < stride) {
    const int64_t flast = flat > 0 ? flat - 1 : 0;
    for (int64_t i0 = threadIdx.x; i0 < flat; i0 += (int64_t)stride * TR) {
      int64_t x[TR];
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        const int64_t i = i0 + (int64_t)r * stride;
        x[r] = seg_exceed[i < flat ? i : flast];
      }
#pragma unroll
      for (int r = 0; r < TR; ++r)
        e += i0 + (int64_t)r * stride < flat ? (unsigned long long)x[r] : 0ull;
    }
  }
  part[threadIdx.x] = e;
  acc = wave_sum_f64(acc);
  cnt = wave_sum_u64(cnt);
  if (lane == 0) {
    wsum[wave] = acc;
    wcnt[wave] = cnt;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
    unsigned long long c = 0;
#pragma unroll
    for (int w = 0; w < TT / 64; ++w) {
      sum += wsum[w];
      c += wcnt[w];
    }
    totals[0] = c == 0ull ? __builtin_nan("") : sum / (double)c;
    totals[1] = (double)c;
  }
  // wave t (< nthr) adds column t's stride / nthr partials: lane l takes
  // partials t + nthr * (l + 64 m)
  if (wave < nthr) {
    const int per = stride / nthr;
    unsigned long long s = 0;
    for (int q = lane; q < per; q += 64) s += part[wave + nthr * q];
    s = wave_sum_u64(s);
    if (lane == 0) totals[2 + wave] = (double)s;
  }
}

template <int NT>
void launch_seg(const float *kl, int64_t n, const int64_t *offsets, int64_t nseg,
                int64_t score_from, const WindowThresholds &thr, double *seg_sum,
                int64_t *seg_count, int64_t *seg_exceed, hipStream_t stream) {
  // one wave per segment when the segments average at most 16 Ki positions
  // and there are enough of them to fill the chip, else one 256-thread block
  constexpr int SW = 1;
  if (nseg >= 1024 && n <= nseg * 16384)
    hipLaunchKernelGGL((window_seg_wave_kernel<SW, 32, NT>), dim3((unsigned)((nseg + SW - 1) / SW)),
                       dim3(64 * SW), 0, stream, kl, n, offsets, nseg, score_from, thr, seg_sum,
                       seg_count, seg_exceed);
  else
    hipLaunchKernelGGL((window_seg_kernel<256, 8, NT>), dim3((unsigned)nseg), dim3(256), 0,
                       stream, kl, n, offsets, score_from, thr, seg_sum, seg_count, seg_exceed);
}

}  // namespace

hipError_t launch_window_summary(const float *kl, int64_t n, const int64_t *offsets, int64_t nseg,
                                 int64_t score_from, const WindowThresholds &thr, double *seg_sum,
                                 int64_t *seg_count, int64_t *seg_exceed, double *totals,
                                 hipStream_t stream) {
  if (nseg > 0) {
    WindowThresholds padded = thr;   // +inf past the list: exceeded by nothing
    for (int t = thr.count; t < KLD_MAX_THRESHOLDS; ++t) padded.value[t] = __builtin_inff();
    if (thr.count == 0)
      launch_seg<0>(kl, n, offsets, nseg, score_from, padded, seg_sum, seg_count, seg_exceed, stream);
    else if (thr.count <= 4)
      launch_seg<4>(kl, n, offsets, nseg, score_from, padded, seg_sum, seg_count, seg_exceed, stream);
    else if (thr.count <= 8)
      launch_seg<8>(kl, n, offsets, nseg, score_from, padded, seg_sum, seg_count, seg_exceed, stream);
    else
      launch_seg<16>(kl, n, offsets, nseg, score_from, padded, seg_sum, seg_count, seg_exceed,
                     stream);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(window_total_kernel, dim3(1), dim3(TT), 0, stream, seg_sum, seg_count,
                     seg_exceed, nseg, thr.count, totals);
  return hipGetLastError();
}

}  // namespace kld

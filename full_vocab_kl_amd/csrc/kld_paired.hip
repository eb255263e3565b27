// Paired per-context comparison of two candidates with a source-cluster
// bootstrap interval ("Qwen3.8-27B fidelity suite v5": "Replay: score your
// own checkpoint against the published BF16 reference" -- the difference of
// two reports' means paired per context, a 95 % bootstrap interval over
// source clusters and the contexts each side wins or ties; "What these inputs
// measured" -- bootstrap intervals over clusters).
//
// The difference is position-weighted: sum_c (sum_a - sum_b) / sum_c count.
// A bootstrap replicate draws as many clusters as there are, with
// replacement (the draws are an input), and recomputes that difference over
// the drawn clusters' contexts; the interval is the type-7 percentile of the
// replicates (linear interpolation, h = q (n - 1)).
//
//   paired_cluster_kernel   one block per cluster: its summed difference and
//                           scored positions; one extra block: the overall
//                           difference, wins, ties and a check of the labels
//                           and counts, whose failure turns every replicate
//                           and percentile into NaN (a flag in the workspace)
//   paired_replicate_kernel one wave per replicate: gather-sum over its draws
//   paired_runsort_kernel   one block per run of 1,024 replicates: bitonic
//                           sort of the run in LDS
//   paired_rank_kernel      every replicate's rank among all of them (its
//                           place in its own run plus a binary search in
//                           each other run; ties ordered by run), scattered
//                           into the sorted array
//   paired_quantile_kernel  one block: NaN check and the interpolated
//                           percentiles
// Every sum runs in a fixed order, so results are bitwise reproducible.
#include "kld.h"
#include "kld_device.hpp"
#include "kld_launch.hpp"

namespace kld {

namespace {

constexpr int PT = 256;

// Sum over the block in a fixed order: a butterfly within each wave, then the
// wave results in order.  red holds PT / 64 entries.
template <typename T>
__device__ __forceinline__ T block_sum(T x, T *red) {
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) x += __shfl_xor(x, m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  T r = red[0];
#pragma unroll
  for (int w = 1; w < PT / 64; ++w) r += red[w];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(PT) void paired_cluster_kernel(
    const double *__restrict__ sum_a, const double *__restrict__ sum_b,
    const int64_t *__restrict__ count, int64_t nctx, const int32_t *__restrict__ cluster,
    int64_t nclust, longlong2 *__restrict__ clus, long long *__restrict__ flag,
    double *__restrict__ out) {
  __shared__ double rd[PT / 64];
  __shared__ long long ri[PT / 64];
  constexpr int U = 8;   // contexts per thread and round, loads issued together
  const int64_t k = blockIdx.x;
  const int64_t last = nctx > 0 ? nctx - 1 : 0;
  if (k < nclust) {
    // every block reads all labels (unconditional, clamped loads); a
    // context's values are loaded only where its label matches, a branch
    // almost never taken
    double d = 0.0;
    long long c = 0;
    for (int64_t i0 = threadIdx.x; i0 < nctx; i0 += (int64_t)PT * U) {
      int32_t lab[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + (int64_t)u * PT;
        lab[u] = cluster[i < nctx ? i : last];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = i0 + (int64_t)u * PT;
        if (i < nctx && lab[u] == k) {
          d += sum_a[i] - sum_b[i];
          c += count[i];
        }
      }
    }
    d = block_sum(d, rd);
    c = block_sum(c, ri);
    if (threadIdx.x == 0) {
      clus[k] = make_longlong2(__double_as_longlong(d), c);   // one 16-byte gather later
    }
    return;
  }
  // the overall difference, wins and ties, and a check of the labels
  double d = 0.0;
  long long c = 0, wa = 0, wb = 0, ti = 0, bad = 0;
  for (int64_t i0 = threadIdx.x; i0 < nctx; i0 += (int64_t)PT * U) {
    double va[U], vb[U];
    int64_t vn[U];
    int32_t vl[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i0u = i0 + (int64_t)u * PT, i = i0u < nctx ? i0u : last;
      va[u] = sum_a[i];
      vb[u] = sum_b[i];
      vn[u] = count[i];
      vl[u] = cluster[i];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i0 + (int64_t)u * PT >= nctx) continue;
      const double a = va[u], b = vb[u];
      const int64_t n = vn[u];
      d += a - b;
      c += n;
      bad += (vl[u] < 0 || vl[u] >= nclust || n < 0) ? 1 : 0;
      if (n > 0) {
        const double ma = a / (double)n, mb = b / (double)n;
        wa += ma < mb;
        wb += mb < ma;
        ti += ma == mb;
      }
    }
  }
  d = block_sum(d, rd);
  c = block_sum(c, ri);
  wa = block_sum(wa, ri);
  wb = block_sum(wb, ri);
  ti = block_sum(ti, ri);
  bad = block_sum(bad, ri);
  if (threadIdx.x == 0) {
    flag[0] = bad;   // read by the replicate and quantile kernels (later in stream order)
    out[0] = (bad || c == 0) ? __builtin_nan("") : d / (double)c;
    out[1] = (double)wa;
    out[2] = (double)wb;
    out[3] = (double)ti;
  }
}

constexpr int RW = 4;   // waves (replicates) per block

__global__ __launch_bounds__(RW * 64) void paired_replicate_kernel(
    const longlong2 *__restrict__ clus, const long long *__restrict__ flag, int64_t nclust,
    const int32_t *__restrict__ draws, int64_t nrep, double *__restrict__ reps) {
  const int lane = threadIdx.x & 63;
  // the wave index made visibly uniform, so that the buffer resource lives
  // in scalar registers (else every load would loop over the lanes)
  const int64_t r = (int64_t)blockIdx.x * RW + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (r >= nrep) return;
  const int32_t *dr = draws + r * nclust;
  double num = 0.0;
  long long den = 0;
  int bad = 0;
  // draws through a buffer resource (past the row: 0, no memory touched) and
  // gathers at clamped indices, contributions masked: no branch around a load
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int32_t *>(dr), (short)0, (int)(nclust * 4), 0x00020000);
  constexpr int RU = 16;   // draws per lane and round: 1,024 per wave
  for (int i0 = lane; i0 < nclust; i0 += 64 * RU) {
    int32_t k[RU];
#pragma unroll
    for (int u = 0; u < RU; ++u)
      k[u] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, (i0 + 64 * u) * 4, 0, 0);
#pragma unroll
    for (int u = 0; u < RU; ++u) {
      const bool in = i0 + 64 * u < nclust;
      const bool ok = k[u] >= 0 && k[u] < nclust;
      const int32_t kk = ok ? k[u] : 0;
      const longlong2 cv = clus[kk];   // the cluster's summed difference and count
      const double x = __longlong_as_double(cv.x);
      const long long n = cv.y;
      bad |= (in && !ok) ? 1 : 0;
      num += (in && ok) ? x : 0.0;
      den += (in && ok) ? n : 0;
    }
  }
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) {
    num += __shfl_xor(num, m);
    den += __shfl_xor(den, m);
    bad |= __shfl_xor(bad, m);
  }
  // a context label outside [0, nclust) or a negative count invalidates every
  // cluster sum: all replicates are NaN then
  if (lane == 0) reps[r] = (bad || den == 0 || flag[0]) ? __builtin_nan("") : num / (double)den;
}

// Sorting the replicates: runs of RUN values are sorted one block each,
// then every value's rank among all of them is its place in its own run plus,
// for each other run, how many of that run's values precede it (values of
// earlier runs that are <= it, of later runs that are < it), found by binary
// search.  The ranks are a permutation, so each value lands in its own slot.
// NaN replicates sort as +inf here; the quantile kernel reports NaN for them.
constexpr int RUN = 1024;
constexpr int MAXRUNS = KLD_MAX_REPLICATES / RUN;
static_assert(MAXRUNS * RUN == KLD_MAX_REPLICATES, "replicate capacity");

__device__ __forceinline__ double sort_key(double v) { return v != v ? __builtin_inf() : v; }

__global__ __launch_bounds__(RUN) void paired_runsort_kernel(const double *__restrict__ reps,
                                                             int64_t nrep,
                                                             double *__restrict__ runs) {
  __shared__ double x[RUN];
  const int t = threadIdx.x;
  const int64_t g = (int64_t)blockIdx.x * RUN + t;
  x[t] = g < nrep ? sort_key(reps[g]) : __builtin_inf();
  __syncthreads();
  for (int size = 2; size <= RUN; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (t < RUN / 2) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const double a = x[i], b = x[j];
        if ((b < a) == up) {
          x[i] = b;
          x[j] = a;
        }
      }
      __syncthreads();
    }
  }
  runs[(int64_t)blockIdx.x * RUN + t] = x[t];
}

constexpr int RT = 256;
static_assert((RUN / 2) % RT == 0, "runs are copied in whole 16-byte rows of the block");

__global__ __launch_bounds__(RT) void paired_rank_kernel(const double *__restrict__ runs,
                                                         int64_t nrep, int nruns,
                                                         double *__restrict__ sorted) {
  __shared__ double r[KLD_MAX_REPLICATES];
  // copy every run into LDS as 16-byte pieces, eight loads in flight per
  // thread (clamped, unconditional), then the stores that are in range
  {
    const double2 *src = reinterpret_cast<const double2 *>(runs);
    double2 *dst = reinterpret_cast<double2 *>(r);
    const int per = nruns * (RUN / 2 / RT);   // pieces per thread (RUN / 2 a multiple of RT)
    for (int j0 = 0; j0 < per; j0 += 8) {
      double2 x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u < per ? j0 + u : per - 1;
        x[u] = src[j * RT + threadIdx.x];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (j0 + u < per) dst[(j0 + u) * RT + threadIdx.x] = x[u];
    }
  }
  __syncthreads();
  const int64_t e = (int64_t)blockIdx.x * RT + threadIdx.x;
  if (e >= nrep) return;
  const int own = (int)(e / RUN);
  const double v = r[e];
  int64_t rank = e - (int64_t)own * RUN;
  for (int q = 0; q < nruns; ++q) {
    if (q == own) continue;
    const double *run = r + q * RUN;
    // lo = number of leading values of run q that precede v
    int lo = 0, hi = RUN;
    if (q < own) {
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (run[mid] <= v) lo = mid + 1; else hi = mid;
      }
    } else {
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (run[mid] < v) lo = mid + 1; else hi = mid;
      }
    }
    rank += lo;
  }
  sorted[rank] = v;
}

constexpr int QT = 1024;

__global__ __launch_bounds__(QT) void paired_quantile_kernel(const double *__restrict__ reps,
                                                             const double *__restrict__ sorted,
                                                             const long long *__restrict__ flag,
                                                             int64_t nrep, PairedQuantiles qs,
                                                             double *__restrict__ out) {
  __shared__ int any_nan;
  if (threadIdx.x == 0) any_nan = flag[0] != 0;
  __syncthreads();
  int nan_here = 0;
  for (int64_t i = threadIdx.x; i < nrep; i += QT) nan_here |= reps[i] != reps[i];
  if (nan_here) any_nan = 1;
  __syncthreads();
  if ((int)threadIdx.x < qs.count) {
    double v = __builtin_nan("");
    if (nrep > 0 && !any_nan) {
      const double h = qs.q[threadIdx.x] * (double)(nrep - 1);
      const int64_t lo = (int64_t)floor(h);
      const int64_t hi = lo + 1 < nrep ? lo + 1 : nrep - 1;
      v = sorted[lo] + (h - (double)lo) * (sorted[hi] - sorted[lo]);
    }
    out[4 + threadIdx.x] = v;
  }
}

}  // namespace

// Workspace: the input-check flag (16 bytes, keeping what follows 16-byte
// aligned), per cluster its difference and count (16 bytes), the sorted runs
// and the sorted replicates.
constexpr size_t kFlagBytes = 16;

size_t paired_workspace_bytes(int64_t nclust, int64_t nrep) {
  const int64_t c = nclust > 0 ? nclust : 0;
  const int64_t runs = nrep > 0 ? (nrep + RUN - 1) / RUN : 0;
  return kFlagBytes + (size_t)c * (sizeof(double) + sizeof(int64_t)) +
         (size_t)(runs * RUN + (nrep > 0 ? nrep : 0)) * sizeof(double);
}

hipError_t launch_paired_bootstrap(const double *sum_a, const double *sum_b, const int64_t *count,
                                   int64_t nctx, const int32_t *cluster, int64_t nclust,
                                   const int32_t *draws, int64_t nrep, const PairedQuantiles &qs,
                                   double *reps, double *out, void *ws, hipStream_t stream) {
  long long *flag = static_cast<long long *>(ws);
  longlong2 *clus = reinterpret_cast<longlong2 *>(static_cast<char *>(ws) + kFlagBytes);
  // per cluster: difference (f64 bits), count
  double *runs = reinterpret_cast<double *>(clus + nclust);
  const int nruns = (int)((nrep + RUN - 1) / RUN);
  double *sorted = runs + (int64_t)nruns * RUN;
  hipLaunchKernelGGL(paired_cluster_kernel, dim3((unsigned)(nclust + 1)), dim3(PT), 0, stream,
                     sum_a, sum_b, count, nctx, cluster, nclust, clus, flag, out);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (nrep > 0) {
    hipLaunchKernelGGL(paired_replicate_kernel, dim3((unsigned)((nrep + RW - 1) / RW)),
                       dim3(RW * 64), 0, stream, clus, flag, nclust, draws, nrep, reps);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(paired_runsort_kernel, dim3((unsigned)nruns), dim3(RUN), 0, stream, reps,
                       nrep, runs);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(paired_rank_kernel, dim3((unsigned)((nrep + RT - 1) / RT)), dim3(RT), 0,
                       stream, runs, nrep, nruns, sorted);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(paired_quantile_kernel, dim3(1), dim3(QT), 0, stream, reps, sorted, flag, nrep,
                     qs, out);
  return hipGetLastError();
}

}  // namespace kld

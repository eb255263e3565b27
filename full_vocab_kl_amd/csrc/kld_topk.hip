// Top-64 merge and the top-64 + tail-bucket KLD ("Qwopus3.8-27B-Coder-Flash:
// quality-eval reference": "Files" -- top-64 ids int32 and fp16 log-probs per
// position, sorted most likely first; "Method" -- KL over the reference's 64
// listed ids plus one cell for all other ids, where a reference id that the
// candidate list lacks is given an equal share of the candidate's unlisted
// mass).
#include "kld_device.hpp"
#include "kld_launch.hpp"

namespace kld {

namespace {

constexpr int MT = 256;   // threads per merge block

// One block per row: merge the per-split candidate lists of each side (each
// sorted, padded with key 0), keep the best 64, write ids and fp16 log-probs
// lp = z - lse (lse in f64 from the row's merged state).
__global__ __launch_bounds__(MT) void topk_merge_kernel(
    const uint64_t *__restrict__ keys /*[n][splits][2][64]*/, int splits, int nsides, int64_t n,
    const double *__restrict__ lse_d /*[2][n]*/, TopkOut out) {
  __shared__ uint64_t buf[kTopkMergeMax];
  const int64_t row = blockIdx.x;
  for (int side = 0; side < nsides; ++side) {
    int32_t *ids = side ? out.ids_cand : out.ids_ref;
    uint16_t *lp = side ? out.lp_cand : out.lp_ref;
    if (!ids && !lp) continue;
    const int total = splits * 64;
    int m = 64;
    while (m < total) m <<= 1;
    for (int i = threadIdx.x; i < m; i += MT) {
      uint64_t k = 0ull;
      if (i < total) {
        const int sp = i / 64, e = i % 64;
        k = keys[((row * splits + sp) * 2 + side) * 64 + e];
      }
      buf[i] = k;
    }
    __syncthreads();
    if (splits > 1) bitonic_desc<MT>(buf, m);
    if (threadIdx.x < 64) {
      const uint64_t k = buf[threadIdx.x];
      const double l = lse_d[side * n + row];
      if (ids) ids[row * 64 + threadIdx.x] = key_id(k);
      if (lp) lp[row * 64 + threadIdx.x] = f32_to_f16_bits((float)((double)key_value(k) - l));
    }
    __syncthreads();
  }
}

// One wave per position: the 65-cell KL of the reference list P against the
// candidate list Q, in f64 from the fp16 log-probs.
__global__ __launch_bounds__(256) void topk_tail_kernel(
    const int32_t *__restrict__ ids_p, const uint16_t *__restrict__ lp_p,
    const int32_t *__restrict__ ids_q, const uint16_t *__restrict__ lp_q, int64_t n, int64_t v,
    float *__restrict__ kl_tail) {
  __shared__ int32_t qid[4][64];
  __shared__ double qv[4][64];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pos = (int64_t)blockIdx.x * 4 + w;
  const bool live = pos < n;
  const int64_t base = (live ? pos : 0) * 64 + lane;
  const double p = exp((double)__builtin_bit_cast(_Float16, lp_p[base]));
  const int32_t pid = ids_p[base];
  const double q = exp((double)__builtin_bit_cast(_Float16, lp_q[base]));
  qid[w][lane] = ids_q[base];
  qv[w][lane] = q;
  __syncthreads();
  // this lane's reference id: candidate probability if listed, else the share u
  double mine = -1.0;
  for (int j = 0; j < 64; ++j)
    if (qid[w][j] == pid) mine = qv[w][j];
  double sp = p, sq = q;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const double op = __shfl_xor(sp, m), oq = __shfl_xor(sq, m);
    const bool lower = (lane & m) == 0;
    sp = lower ? sp + op : op + sp;
    sq = lower ? sq + oq : oq + sq;
  }
  const double p_tail = fmax(0.0, 1.0 - sp);
  const double r = fmax(0.0, 1.0 - sq);
  const double u = v > 64 ? r / (double)(v - 64) : 0.0;
  const double qh = mine >= 0.0 ? mine : u;
  double sqh = qh;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const double o = __shfl_xor(sqh, m);
    sqh = (lane & m) == 0 ? sqh + o : o + sqh;
  }
  const double q_tail = fmax(0.0, 1.0 - sqh);
  const double inf = __builtin_inf();
  double term = p == 0.0 ? 0.0 : (qh == 0.0 ? inf : p * log(p / qh));
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const double o = __shfl_xor(term, m);
    term = (lane & m) == 0 ? term + o : o + term;
  }
  if (lane == 0 && live) {
    const double tail = p_tail == 0.0 ? 0.0 : (q_tail == 0.0 ? inf : p_tail * log(p_tail / q_tail));
    kl_tail[pos] = (float)(term + tail);
  }
}

}  // namespace

hipError_t launch_topk_merge(const uint64_t *keys, int splits, int nsides, int64_t n,
                             const double *lse_d, const TopkOut &out, hipStream_t stream) {
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)n), dim3(MT), 0, stream, keys, splits, nsides,
                     n, lse_d, out);
  return hipGetLastError();
}

hipError_t launch_topk_tail(const int32_t *ids_p, const uint16_t *lp_p, const int32_t *ids_q,
                            const uint16_t *lp_q, int64_t n, int64_t v, float *kl_tail,
                            hipStream_t stream) {
  hipLaunchKernelGGL(topk_tail_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream, ids_p,
                     lp_p, ids_q, lp_q, n, v, kl_tail);
  return hipGetLastError();
}

}  // namespace kld

// Logits path: one streaming pass over the reference and candidate logit rows.
//
// Each block owns one (row, vocabulary split) pair and streams both rows'
// slices once, coalesced, 16 bytes per lane per load.  Every lane folds its
// elements into an online RowState (kld_device.hpp), batch by batch: one
// max per batch, one rebase when the max moves, then one exp2 per element
// per side.  Lanes merge by butterfly, waves through LDS, and the block
// writes one partial state; finalize_rows_kernel merges the splits (in f64) in a
// fixed order and writes the per-position outputs.  HBM-bound: 2 v sizeof(T)
// bytes per position are read once.
//
// Top-64 export ("Qwopus3.8-27B-Coder-Flash: quality-eval reference",
// "Files": top-64 ids and fp16 log-probs, sorted) rides the same pass.  Each
// element is ranked by a 64-bit key (order-preserving f32 bits, then the
// complemented id, so equal values rank the lower id first).  The block keeps
// a candidate buffer per side in LDS and a threshold key: an element enters
// the buffer only if its key beats the threshold.  The first batch seeds the
// threshold just below the 64th largest of the 256 per-thread batch maxima (a
// valid bound: they are 256 distinct elements); whenever the buffer passes a
// high-water mark it is sorted (bitonic, in LDS), cut to its 64 best keys and
// the threshold becomes the 64th.  An append that finds the buffer full is
// remembered by its thread and retried after the compaction, so no candidate
// is lost.  The block writes its sorted 64 best keys per side;
// topk_merge_kernel (kld_topk.hip) merges the splits of a row and converts
// them to ids and fp16 log-probs.
#include "kld_device.hpp"
#include "kld_launch.hpp"

namespace kld {

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Vec;
template <> struct Vec<float> { static constexpr int N = 4; };
template <> struct Vec<uint16_t> { static constexpr int N = 8; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return bf16_to_f32(x); }

// Load VEC consecutive elements starting at element `pos` (< hi) of a row,
// as f32; elements at or beyond `hi` read as -inf.  Fast path: one 16-byte
// load when the whole vector is in range and the row is 16-byte aligned.
template <typename T, int VEC, bool ALIGNED>
__device__ __forceinline__ void load_vec(const T *__restrict__ row, int64_t pos, int64_t hi,
                                         float (&x)[VEC]) {
  if (ALIGNED && pos + VEC <= hi) {
    if constexpr (sizeof(T) == 4) {
      f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + pos));
      x[0] = q[0]; x[1] = q[1]; x[2] = q[2]; x[3] = q[3];
    } else {
      u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(row + pos));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(q[i] << 16);
        x[2 * i + 1] = __uint_as_float(q[i] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < VEC; ++j) x[j] = (pos + j < hi) ? to_f32(row[pos + j]) : kNegInf;
  }
}

constexpr int kThreads = 256;
constexpr int kCap = 2048;            // candidate buffer entries per side
constexpr int kHigh = kCap - 512;     // compact once the buffer holds more than this

struct TopkShared {
  uint64_t buf[2][kCap];
  uint64_t seed[kThreads];
  uint64_t thr[2];
  int count[2];
};

// Sort the filled part of one side's buffer, keep its 64 best keys and set
// the threshold to the 64th (0 while fewer than 64 are known).  Block-wide.
__device__ void compact(TopkShared &sh, int side) {
  const int cnt = min(sh.count[side], kCap);
  int n = 64;
  while (n < cnt) n <<= 1;
  for (int i = cnt + (int)threadIdx.x; i < n; i += kThreads) sh.buf[side][i] = 0ull;
  __syncthreads();
  bitonic_desc<kThreads>(sh.buf[side], n);
  if (threadIdx.x == 0) {
    sh.count[side] = min(cnt, 64);
    sh.thr[side] = cnt >= 64 ? sh.buf[side][63] : 0ull;
  }
  __syncthreads();
}

template <typename T, int VEC, int U, bool ALIGNED, bool TWO, bool TOPK>
__global__ __launch_bounds__(kThreads) void logits_partial_kernel(
    const T *__restrict__ ref, const T *__restrict__ cand, int64_t ld_ref, int64_t ld_cand,
    int64_t v, int64_t chunk, int splits, RowState *__restrict__ part,
    uint64_t *__restrict__ topk_keys /*[n][splits][2][64]*/) {
  const int64_t row = blockIdx.x / splits;
  const int split = (int)(blockIdx.x % splits);
  const int64_t lo = (int64_t)split * chunk;
  const int64_t hi = lo + chunk < v ? lo + chunk : v;
  const T *ra = ref + row * ld_ref;
  const T *rb = TWO ? cand + row * ld_cand : ra;
  constexpr int NS = TWO ? 2 : 1;

  __shared__ TopkShared sh_storage[1];
  TopkShared &sh = sh_storage[0];
  if constexpr (TOPK) {
    if (threadIdx.x < NS) { sh.count[threadIdx.x] = 0; sh.thr[threadIdx.x] = 0ull; }
  }

  float ma = kNegInf, sa = 0.f, t = 0.f, mb = kNegInf, sb = 0.f;
  int ia = kNoId, ib = kNoId;

  constexpr int64_t kStride = (int64_t)kThreads * VEC;
  // every thread runs the same number of rounds so the block can synchronise
  const int64_t rounds = (hi - lo + kStride * U - 1) / (kStride * U);
  for (int64_t rd = 0; rd < rounds; ++rd) {
    const int64_t base = lo + rd * kStride * U + (int64_t)threadIdx.x * VEC;
    float xa[U][VEC], xb[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t pos = base + u * kStride;
      if (pos < hi) {
        load_vec<T, VEC, ALIGNED>(ra, pos, hi, xa[u]);
        if (TWO) load_vec<T, VEC, ALIGNED>(rb, pos, hi, xb[u]);
      } else {
#pragma unroll
        for (int j = 0; j < VEC; ++j) { xa[u][j] = kNegInf; xb[u][j] = kNegInf; }
      }
    }
    float bma = kNegInf, bmb = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        bma = fmaxf(bma, xa[u][j]);
        if (TWO) bmb = fmaxf(bmb, xb[u][j]);
      }
    if (bma > ma) {   // new maximum: locate its lowest id in this batch, rebase the sums
      int id = kNoId;
#pragma unroll
      for (int u = U - 1; u >= 0; --u)
#pragma unroll
        for (int j = VEC - 1; j >= 0; --j)
          if (xa[u][j] == bma) id = (int)(base + u * kStride + j);
      const float f = rescale(ma, bma);
      if (TWO && sa != 0.f) t = fmaf(-sa, bma - ref_of(ma), t);
      t *= f; sa *= f; ma = bma; ia = id;
    }
    if (TWO && bmb > mb) {
      int id = kNoId;
#pragma unroll
      for (int u = U - 1; u >= 0; --u)
#pragma unroll
        for (int j = VEC - 1; j >= 0; --j)
          if (xb[u][j] == bmb) id = (int)(base + u * kStride + j);
      if (sa != 0.f) t = fmaf(sa, bmb - ref_of(mb), t);
      sb *= rescale(mb, bmb); mb = bmb; ib = id;
    }
    const float rfa = ref_of(ma), rfb = ref_of(mb);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float x = xa[u][j] - rfa;
        const float w = exp2_fast(x * kL2E);
        sa += w;
        if (TWO) {
          const float y = xb[u][j] - rfb;
          // x - y is clamped below so that a -inf reference id (w = 0) adds
          // exactly 0 even when the candidate id is -inf too.
          t = fmaf(w, fmaxf(x - y, -kFltMax), t);
          sb += exp2_fast(y * kL2E);
        }
      }

    if constexpr (TOPK) {
      if (rd == 0) {
        // seed each side's threshold just below the 64th best per-thread maximum
        for (int side = 0; side < NS; ++side) {
          uint64_t best = 0ull;
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
              const int64_t id = base + u * kStride + j;
              if (id < hi) {
                const uint64_t k = topk_key(side ? xb[u][j] : xa[u][j], (int)id);
                best = k > best ? k : best;
              }
            }
          sh.seed[threadIdx.x] = best;
          __syncthreads();
          bitonic_desc<kThreads>(sh.seed, kThreads);
          if (threadIdx.x == 0) sh.thr[side] = sh.seed[63] == 0ull ? 0ull : sh.seed[63] - 1ull;
          __syncthreads();
        }
      }
      // append every element whose key beats the threshold; remember what did
      // not fit and retry after compacting
      uint32_t pending[2] = {0u, 0u};
      for (int side = 0; side < NS; ++side) {
        const uint64_t th = sh.thr[side];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int j = 0; j < VEC; ++j) {
            const int64_t id = base + u * kStride + j;
            const float x = side ? xb[u][j] : xa[u][j];
            if (id < hi) {
              const uint64_t k = topk_key(x, (int)id);
              if (k > th) {
                const int slot = atomicAdd(&sh.count[side], 1);
                if (slot < kCap) sh.buf[side][slot] = k;
                else pending[side] |= 1u << (u * VEC + j);
              }
            }
          }
      }
      for (;;) {
        __syncthreads();
        bool any = false;
        for (int side = 0; side < NS; ++side) any = any || sh.count[side] > kHigh;
        if (!any) break;
        for (int side = 0; side < NS; ++side)
          if (sh.count[side] > kHigh) compact(sh, side);
        // retry the elements that found the buffer full
        for (int side = 0; side < NS; ++side) {
          const uint64_t th = sh.thr[side];
          uint32_t still = 0u;
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < VEC; ++j) {
              if (pending[side] & (1u << (u * VEC + j))) {
                const uint64_t k =
                    topk_key(side ? xb[u][j] : xa[u][j], (int)(base + u * kStride + j));
                if (k > th) {
                  const int slot = atomicAdd(&sh.count[side], 1);
                  if (slot < kCap) sh.buf[side][slot] = k;
                  else still |= 1u << (u * VEC + j);
                }
              }
            }
          pending[side] = still;
        }
      }
    }
  }

  if constexpr (TOPK) {
    for (int side = 0; side < NS; ++side) {
      compact(sh, side);
      uint64_t *dst = topk_keys + ((row * splits + split) * 2 + side) * 64;
      if (threadIdx.x < 64)
        dst[threadIdx.x] = (int)threadIdx.x < sh.count[side] ? sh.buf[side][threadIdx.x] : 0ull;
    }
  }

  RowState s;
  s.ma = ma; s.sa = sa; s.t = t; s.mb = mb; s.sb = sb; s.ia = ia; s.ib = ib;
  s = wave_merge(s);
  __shared__ RowState waves[kThreads / 64];
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) waves[wave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    RowState r = waves[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = merge(r, waves[w]);
    part[row * splits + split] = r;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void finalize_rows_kernel(
    const RowState *__restrict__ part, int splits, int64_t n, const T *__restrict__ ref,
    const T *__restrict__ cand, int64_t ld_ref, int64_t ld_cand, int64_t v,
    const int32_t *__restrict__ target, RowsOut out, double *__restrict__ lse_d /*[2][n]*/,
    float *__restrict__ target_lp) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= n) return;
  RowStateD s = to_d(part[row * splits]);
  for (int i = 1; i < splits; ++i) s = merge_d(s, to_d(part[row * splits + i]));
  double la, lb;
  const RowResult r = finish_d(s, &la, &lb);
  if (lse_d) { lse_d[row] = la; lse_d[n + row] = lb; }
  if (out.kl) out.kl[row] = r.kl;
  if (out.lse_ref) out.lse_ref[row] = r.lse_a;
  if (out.lse_cand) out.lse_cand[row] = r.lse_b;
  if (out.argmax_ref) out.argmax_ref[row] = r.ia;
  if (out.argmax_cand) out.argmax_cand[row] = r.ib;
  if (target) {
    const int32_t tg = target[row];
    const bool ok = tg >= 0 && (int64_t)tg < v;
    const float nan = __builtin_nanf("");
    if (out.nll_ref) out.nll_ref[row] = ok ? (float)(la - (double)to_f32(ref[row * ld_ref + tg])) : nan;
    if (out.nll_cand)
      out.nll_cand[row] = ok ? (float)(lb - (double)to_f32(cand[row * ld_cand + tg])) : nan;
    if (target_lp) target_lp[row] = ok ? (float)((double)to_f32(ref[row * ld_ref + tg]) - la) : nan;
  }
}

template <typename T, int VEC, int U, bool ALIGNED, bool TWO, bool TOPK>
hipError_t launch_partial_t(const LogitsArgs &a, RowState *part, uint64_t *keys) {
  dim3 grid((unsigned)(a.n * a.splits));
  hipError_t e = record(a.ev.start, a.stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((logits_partial_kernel<T, VEC, U, ALIGNED, TWO, TOPK>), grid, dim3(kThreads), 0,
                     a.stream, (const T *)a.ref, (const T *)a.cand, a.ld_ref, a.ld_cand, a.v, a.chunk,
                     a.splits, part, keys);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return record(a.ev.stop, a.stream);
}

template <typename T, int VEC, int U>
hipError_t launch_partial(const LogitsArgs &a, RowState *part, uint64_t *keys) {
  const bool tk = keys != nullptr;
  if (a.two) {
    if (a.aligned) return tk ? launch_partial_t<T, VEC, U, true, true, true>(a, part, keys)
                             : launch_partial_t<T, VEC, U, true, true, false>(a, part, keys);
    return tk ? launch_partial_t<T, VEC, U, false, true, true>(a, part, keys)
              : launch_partial_t<T, VEC, U, false, true, false>(a, part, keys);
  }
  // one side is only used for the top-k export
  if (a.aligned) return launch_partial_t<T, VEC, U, true, false, true>(a, part, keys);
  return launch_partial_t<T, VEC, U, false, false, true>(a, part, keys);
}

template <typename T>
hipError_t launch_finalize(const LogitsArgs &a, const RowState *part, double *lse_d,
                           float *target_lp) {
  const unsigned blocks = (unsigned)((a.n + 255) / 256);
  hipLaunchKernelGGL((finalize_rows_kernel<T>), dim3(blocks), dim3(256), 0, a.stream, part,
                     a.splits, a.n, (const T *)a.ref, (const T *)a.cand, a.ld_ref, a.ld_cand, a.v,
                     a.target, a.out, lse_d, target_lp);
  return hipGetLastError();
}

}  // namespace

int logits_vec_elems(int dtype) { return dtype == 0 ? Vec<float>::N : Vec<uint16_t>::N; }

hipError_t launch_logits_state(const LogitsArgs &a, RowState *part, uint64_t *topk_keys) {
  if (a.dtype == 0) return launch_partial<float, 4, 4>(a, part, topk_keys);
  return launch_partial<uint16_t, 8, 2>(a, part, topk_keys);
}

hipError_t launch_logits_finalize(const LogitsArgs &a, const RowState *part, double *lse_d,
                                  float *target_lp) {
  if (a.dtype == 0) return launch_finalize<float>(a, part, lse_d, target_lp);
  return launch_finalize<uint16_t>(a, part, lse_d, target_lp);
}

}  // namespace kld

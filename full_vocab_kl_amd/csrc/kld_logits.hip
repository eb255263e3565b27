// Logits path: one streaming pass over the reference and candidate logit rows.
//
// Each block owns one (row, vocabulary split) pair and streams both rows'
// slices once, coalesced, 16 bytes per lane per load.  Every lane folds its
// elements into an online RowState (kld_device.hpp), batch by batch: one
// max per batch, one rescale when the max moves, then one exp2 per element
// per side.  Lanes merge by butterfly, waves through LDS, and the block
// writes one partial state; kld_finalize_rows merges the splits in a fixed
// order and writes the per-position outputs.  HBM-bound: 2 * v * sizeof(T)
// bytes per position are read once.
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
      const uint32_t w[4] = {q[0], q[1], q[2], q[3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[2 * i] = __uint_as_float(w[i] << 16);
        x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < VEC; ++j) x[j] = (pos + j < hi) ? to_f32(row[pos + j]) : kNegInf;
  }
}

constexpr int kThreads = 256;

template <typename T, int VEC, int U, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void logits_partial_kernel(
    const T *__restrict__ ref, const T *__restrict__ cand, int64_t ld_ref, int64_t ld_cand,
    int64_t v, int64_t chunk, int splits, RowState *__restrict__ part) {
  const int64_t row = blockIdx.x / splits;
  const int split = (int)(blockIdx.x % splits);
  const int64_t lo = (int64_t)split * chunk;
  const int64_t hi = lo + chunk < v ? lo + chunk : v;
  const T *ra = ref + row * ld_ref;
  const T *rb = cand + row * ld_cand;

  float ma = kNegInf, sa = 0.f, t = 0.f, mb = kNegInf, sb = 0.f;
  int ia = kNoId, ib = kNoId;

  constexpr int64_t kStride = (int64_t)kThreads * VEC;
  for (int64_t base = lo + (int64_t)threadIdx.x * VEC; base < hi; base += kStride * U) {
    float xa[U][VEC], xb[U][VEC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t pos = base + u * kStride;
      if (pos < hi) {
        load_vec<T, VEC, ALIGNED>(ra, pos, hi, xa[u]);
        load_vec<T, VEC, ALIGNED>(rb, pos, hi, xb[u]);
      } else {
#pragma unroll
        for (int j = 0; j < VEC; ++j) { xa[u][j] = kNegInf; xb[u][j] = kNegInf; }
      }
    }
    float bma = kNegInf, bmb = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < VEC; ++j) { bma = fmaxf(bma, xa[u][j]); bmb = fmaxf(bmb, xb[u][j]); }
    if (bma > ma) {   // new maximum: locate its lowest id in this batch, rebase the sums
      int id = kNoId;
#pragma unroll
      for (int u = U - 1; u >= 0; --u)
#pragma unroll
        for (int j = VEC - 1; j >= 0; --j)
          if (xa[u][j] == bma) id = (int)(base + u * kStride + j);
      const float f = rescale(ma, bma);
      if (sa != 0.f) t = fmaf(-sa, bma - ref_of(ma), t);
      t *= f; sa *= f; ma = bma; ia = id;
    }
    if (bmb > mb) {
      int id = kNoId;
#pragma unroll
      for (int u = U - 1; u >= 0; --u)
#pragma unroll
        for (int j = VEC - 1; j >= 0; --j)
          if (xb[u][j] == bmb) id = (int)(base + u * kStride + j);
      if (sa != 0.f) t = fmaf(sa, bmb - ref_of(mb), t);
      sb *= rescale(mb, bmb); mb = bmb; ib = id;
    }
    const float ra = ref_of(ma), rb = ref_of(mb);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float x = xa[u][j] - ra, y = xb[u][j] - rb;
        const float w = exp2_fast(x * kL2E);
        sa += w;
        // x - y is clamped below so that a -inf reference id (w = 0) adds
        // exactly 0 even when the candidate id is -inf too.
        t = fmaf(w, fmaxf(x - y, -kFltMax), t);
        sb += exp2_fast(y * kL2E);
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
    const int32_t *__restrict__ target, RowsOut out) {
  const int64_t row = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (row >= n) return;
  RowState s = part[row * splits];
  for (int i = 1; i < splits; ++i) s = merge(s, part[row * splits + i]);
  const RowResult r = finish(s);
  out.kl[row] = r.kl;
  if (out.lse_ref) out.lse_ref[row] = r.lse_a;
  if (out.lse_cand) out.lse_cand[row] = r.lse_b;
  if (out.argmax_ref) out.argmax_ref[row] = r.ia;
  if (out.argmax_cand) out.argmax_cand[row] = r.ib;
  if (target) {
    const int32_t tg = target[row];
    const bool ok = tg >= 0 && (int64_t)tg < v;
    const float nan = __builtin_nanf("");
    if (out.nll_ref)
      out.nll_ref[row] = ok ? (float)((double)r.lse_a - (double)to_f32(ref[row * ld_ref + tg])) : nan;
    if (out.nll_cand)
      out.nll_cand[row] = ok ? (float)((double)r.lse_b - (double)to_f32(cand[row * ld_cand + tg])) : nan;
  }
}

template <typename T, int VEC, int U, bool ALIGNED>
hipError_t launch_partial(const LogitsArgs &a, RowState *part) {
  dim3 grid((unsigned)(a.n * a.splits));
  if (record(a.ev.start, a.stream) != hipSuccess) return hipErrorInvalidValue;
  hipLaunchKernelGGL((logits_partial_kernel<T, VEC, U, ALIGNED>), grid, dim3(kThreads), 0, a.stream,
                     (const T *)a.ref, (const T *)a.cand, a.ld_ref, a.ld_cand, a.v, a.chunk, a.splits,
                     part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return record(a.ev.stop, a.stream);
}

template <typename T>
hipError_t launch_finalize(const LogitsArgs &a, const RowState *part) {
  const unsigned blocks = (unsigned)((a.n + 255) / 256);
  hipLaunchKernelGGL((finalize_rows_kernel<T>), dim3(blocks), dim3(256), 0, a.stream, part,
                     a.splits, a.n, (const T *)a.ref, (const T *)a.cand, a.ld_ref, a.ld_cand, a.v,
                     a.target, a.out);
  return hipGetLastError();
}

}  // namespace

int logits_vec_elems(int dtype) { return dtype == 0 ? Vec<float>::N : Vec<uint16_t>::N; }

hipError_t launch_logits_state(const LogitsArgs &a, RowState *part) {
  if (a.dtype == 0) {
    if (a.aligned) return launch_partial<float, 4, 4, true>(a, part);
    return launch_partial<float, 4, 4, false>(a, part);
  }
  if (a.aligned) return launch_partial<uint16_t, 8, 2, true>(a, part);
  return launch_partial<uint16_t, 8, 2, false>(a, part);
}

hipError_t launch_logits_finalize(const LogitsArgs &a, const RowState *part) {
  if (a.dtype == 0) return launch_finalize<float>(a, part);
  return launch_finalize<uint16_t>(a, part);
}

}  // namespace kld

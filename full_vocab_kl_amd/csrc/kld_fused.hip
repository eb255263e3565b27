// Fused head path: logits z = W h for the reference and the candidate hidden
// states through one shared bf16 head, reduced on the fly -- the logits never
// reach memory ("Qwen3.8-27B fidelity suite v5", opening paragraphs: one
// shared BF16 head for both sides; "What is in here": hidden states
// [2047, 5120] bf16).
//
// Kernel fused_head_kernel computes, per block, the transposed tile
// Z^T[BV vocab x BP positions] for both sides with bf16 MFMA
// (v_mfma_f32_32x32x16_bf16): the head tile is the A operand (rows = vocab
// ids, K = hidden), the hidden tile the B operand (columns = positions), so
// every lane's accumulators hold one position and 16 vocabulary ids, and the
// per-position reduction over the vocabulary is mostly lane-local.  Reference
// and candidate columns of the same position sit in the same lane and
// register slot.  Operands are staged through LDS (double-buffered, 16-byte
// chunks with an XOR swizzle so fragment reads spread over the banks).
//
// Epilogue: the block's 256 x 128 tile of (a, b) pairs is folded into one
// RowState per position (kld_device.hpp) and written as a partial state for
// (vocab tile, position).  fused_finalize_kernel merges the partial states
// of each position over all vocabulary tiles in a fixed order.
//
// Grid: one block per (vocab tile, position tile).  Consecutive hardware
// block ids are dealt round-robin over the 8 XCDs; the block id is remapped
// so that each XCD receives a contiguous range of tiles, position tiles
// fastest, so all position tiles of one head tile run together on one XCD
// and the head tile is fetched from HBM about once into that XCD's L2.
#include "kld_device.hpp"
#include "kld_launch.hpp"

namespace kld {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BV = 256;            // vocabulary ids per block
constexpr int BP = 128;            // positions per block (x2 sides = 256 B columns)
constexpr int BK = 64;             // hidden elements per pipeline stage
constexpr int NT = 256;            // threads per block (4 waves: 2 vocab x 2 position)
constexpr int CH = BK / 8;         // 16-byte chunks per staged row
constexpr int ROWS = BV + 2 * BP;  // staged rows per stage (head rows, then ref, then cand)
constexpr int STAGE_CHUNKS = ROWS * CH;
constexpr int LOADS = ROWS * CH / NT;   // 16-byte global loads per thread per stage
constexpr int kXcds = 8;

static_assert(LOADS == 16, "tile shape");

// Swizzled position of chunk c of staged row r.  Rows are 128 bytes; the
// chunk index is XORed with (r ^ r >> 3) & 7 so that 8 consecutive rows (and
// the even or odd rows among 16) read at one logical chunk hit distinct banks.
__device__ __forceinline__ int swz(int r, int c) { return r * CH + (c ^ ((r ^ (r >> 3)) & 7)); }

// Map the hardware block id to a logical tile id so that each XCD gets a
// contiguous range of logical ids.
__device__ __forceinline__ int logical_block(int b, int nb) {
  const int xcd = b % kXcds, slot = b / kXcds;
  const int q = nb / kXcds, r = nb % kXcds;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
}

__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fused_head_kernel(const uint16_t *__restrict__ W, const uint16_t *__restrict__ Hr,
                       const uint16_t *__restrict__ Hc, int64_t v, int64_t d, int64_t n, int npt,
                       int64_t npad, int64_t nvt, float *__restrict__ part) {
  extern __shared__ u32x4 smem[];   // [2][STAGE_CHUNKS]

  const int L = logical_block((int)blockIdx.x, (int)gridDim.x);
  const int vt = L / npt, pt = L % npt;
  const int64_t v0 = (int64_t)vt * BV, p0 = (int64_t)pt * BP;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = wave >> 1, wp = wave & 1;

  // ---- global -> register staging: thread loads chunk (tid % 8) of staged
  // rows tid / 8 + 32 j, j = 0..15 (rows 0..255 head, 256..383 ref, 384..511 cand).
  const int lc = tid & 7, lr = tid >> 3;
  const uint16_t *src[LOADS];
#pragma unroll
  for (int j = 0; j < LOADS; ++j) {
    const int r = lr + 32 * j;
    if (r < BV) {
      const int64_t vr = v0 + r;
      src[j] = W + (vr < v ? vr : v - 1) * d + lc * 8;
    } else {
      const int hr = r - BV;
      const int64_t pos = p0 + (hr & (BP - 1));
      src[j] = (hr < BP ? Hr : Hc) + (pos < n ? pos : n - 1) * d + lc * 8;
    }
  }
  u32x4 stage[LOADS];
  const int KT = (int)((d + BK - 1) / BK);

  // Rows beyond v or n read a valid clamped row: their results are masked or
  // discarded.  Only hidden elements beyond d must read as zero, which can
  // happen in the last stage alone.
  auto load_stage = [&](int kt) {
    const int64_t k = (int64_t)kt * BK + lc * 8;
    if (k < d) {
#pragma unroll
      for (int j = 0; j < LOADS; ++j)
        stage[j] = *reinterpret_cast<const u32x4 *>(src[j] + (int64_t)kt * BK);
    } else {
#pragma unroll
      for (int j = 0; j < LOADS; ++j) stage[j] = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_stage = [&](int buf) {
    u32x4 *s = smem + buf * STAGE_CHUNKS;
#pragma unroll
    for (int j = 0; j < LOADS; ++j) s[swz(lr + 32 * j, lc)] = stage[j];
  };

  f32x16 acc[4][2][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][c][i] = 0.f;

  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int fr = lane & 31, fh = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) load_stage(kt + 1);
    const u32x4 *s = smem + cur * STAGE_CHUNKS;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = 2 * ks + fh;
      bf16x8 fa[4], fb[2][2];
#pragma unroll
      for (int vs = 0; vs < 4; ++vs)
        fa[vs] = __builtin_bit_cast(bf16x8, s[swz(wv * 128 + vs * 32 + fr, c)]);
#pragma unroll
      for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int sd = 0; sd < 2; ++sd)
          fb[pg][sd] = __builtin_bit_cast(bf16x8, s[swz(BV + sd * BP + wp * 64 + pg * 32 + fr, c)]);
#pragma unroll
      for (int vs = 0; vs < 4; ++vs)
#pragma unroll
        for (int pg = 0; pg < 2; ++pg)
#pragma unroll
          for (int sd = 0; sd < 2; ++sd)
            acc[vs][pg][sd] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[vs], fb[pg][sd], acc[vs][pg][sd], 0, 0, 0);
    }
    if (kt + 1 < KT) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds position p0 + wp*64 + pg*32 + (lane & 31) and
  // vocabulary ids vb + 32 vs + 8 (i / 4) + (i % 4), vb = v0 + 128 wv + 4 (lane >> 5).
  const int64_t vb = v0 + wv * 128 + 4 * fh;
  const bool vtail = v0 + BV > v;
  RowState *xch = reinterpret_cast<RowState *>(smem);   // [2 pos waves][2 pg][32] states
#pragma unroll
  for (int pg = 0; pg < 2; ++pg) {
    if (vtail) {
#pragma unroll
      for (int vs = 0; vs < 4; ++vs)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (vb + 32 * vs + 8 * (i >> 2) + (i & 3) >= v) {
            acc[vs][pg][0][i] = kNegInf;
            acc[vs][pg][1][i] = kNegInf;
          }
    }
    float ma = kNegInf, mb = kNegInf;
#pragma unroll
    for (int vs = 0; vs < 4; ++vs)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        ma = fmaxf(ma, acc[vs][pg][0][i]);
        mb = fmaxf(mb, acc[vs][pg][1][i]);
      }
    int ia = kNoId, ib = kNoId;
#pragma unroll
    for (int vs = 3; vs >= 0; --vs)
#pragma unroll
      for (int i = 15; i >= 0; --i) {
        const int off = 32 * vs + 8 * (i >> 2) + (i & 3);
        if (acc[vs][pg][0][i] == ma) ia = off;
        if (acc[vs][pg][1][i] == mb) ib = off;
      }
    const float ra = ref_of(ma), rb = ref_of(mb);
    float sa = 0.f, sb = 0.f, t = 0.f;
#pragma unroll
    for (int vs = 0; vs < 4; ++vs)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = acc[vs][pg][0][i] - ra, y = acc[vs][pg][1][i] - rb;
        const float w = exp2_fast(x * kL2E);
        sa += w;
        t = fmaf(w, fmaxf(x - y, -kFltMax), t);
        sb += exp2_fast(y * kL2E);
      }
    RowState st;
    st.ma = ma; st.sa = sa; st.t = t; st.mb = mb; st.sb = sb;
    st.ia = ia == kNoId ? kNoId : (int)(vb + ia);
    st.ib = ib == kNoId ? kNoId : (int)(vb + ib);
    // lanes l and l ^ 32 hold the same position (interleaved ids)
    const RowState o = shfl_xor_state(st, 32);
    st = fh == 0 ? merge(st, o) : merge(o, st);
    if (wv == 1 && fh == 0) xch[(wp * 2 + pg) * 32 + fr] = st;
    __syncthreads();
    if (wv == 0 && fh == 0) {
      st = merge(st, xch[(wp * 2 + pg) * 32 + fr]);
      const int64_t pos = p0 + wp * 64 + pg * 32 + fr;
      if (pos < n) {
        const int64_t plane = nvt * npad;
        float *q = part + (int64_t)vt * npad + pos;
        q[0] = st.ma; q[plane] = st.sa; q[2 * plane] = st.t; q[3 * plane] = st.mb;
        q[4 * plane] = st.sb;
        q[5 * plane] = __int_as_float(st.ia);
        q[6 * plane] = __int_as_float(st.ib);
      }
    }
    __syncthreads();
  }
}

// Target logits z_t = W[target] . h for both sides, f32 accumulation of exact
// bf16 products in a fixed order: one wave per position.
__global__ __launch_bounds__(256) void target_logit_kernel(
    const uint16_t *__restrict__ W, const uint16_t *__restrict__ Hr,
    const uint16_t *__restrict__ Hc, int64_t v, int64_t d, int64_t n,
    const int32_t *__restrict__ target, float *__restrict__ zt /*[2][n]*/) {
  const int64_t pos = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (pos >= n) return;
  const int32_t tg = target[pos];
  if (tg < 0 || (int64_t)tg >= v) {
    if (lane == 0) { zt[pos] = __builtin_nanf(""); zt[n + pos] = __builtin_nanf(""); }
    return;
  }
  const uint16_t *w = W + (int64_t)tg * d;
  const uint16_t *hr = Hr + pos * d, *hc = Hc + pos * d;
  float sr = 0.f, sc = 0.f;
  for (int64_t k = (int64_t)lane * 8; k < d; k += 64 * 8) {
    const u32x4 qw = *reinterpret_cast<const u32x4 *>(w + k);
    const u32x4 qr = *reinterpret_cast<const u32x4 *>(hr + k);
    const u32x4 qc = *reinterpret_cast<const u32x4 *>(hc + k);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float w0 = __uint_as_float(qw[e] << 16), w1 = __uint_as_float(qw[e] & 0xffff0000u);
      sr = fmaf(w0, __uint_as_float(qr[e] << 16), sr);
      sr = fmaf(w1, __uint_as_float(qr[e] & 0xffff0000u), sr);
      sc = fmaf(w0, __uint_as_float(qc[e] << 16), sc);
      sc = fmaf(w1, __uint_as_float(qc[e] & 0xffff0000u), sc);
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float orr = __shfl_xor(sr, m), oc = __shfl_xor(sc, m);
    const bool lower = (lane & m) == 0;
    sr = lower ? sr + orr : orr + sr;
    sc = lower ? sc + oc : oc + sc;
  }
  if (lane == 0) { zt[pos] = sr; zt[n + pos] = sc; }
}

// Merge the partial states of each position over the vocabulary tiles: block
// = 32 positions x 8 groups; group g merges tiles g, g + 8, ... in order, then
// the 8 group states merge in order through LDS.
constexpr int FP = 32, FG = 8;
__global__ __launch_bounds__(FP * FG) void fused_finalize_kernel(
    const float *__restrict__ part, int64_t nvt, int64_t npad, int64_t n,
    const float *__restrict__ zt, const int32_t *__restrict__ target, RowsOut out) {
  __shared__ RowState red[FG][FP];
  const int pl = threadIdx.x % FP, g = threadIdx.x / FP;
  const int64_t pos = (int64_t)blockIdx.x * FP + pl;
  const int64_t plane = nvt * npad;
  RowState s = empty_state();
  if (pos < n) {
    for (int64_t vt = g; vt < nvt; vt += FG) {
      const float *q = part + vt * npad + pos;
      RowState x;
      x.ma = q[0]; x.sa = q[plane]; x.t = q[2 * plane]; x.mb = q[3 * plane]; x.sb = q[4 * plane];
      x.ia = __float_as_int(q[5 * plane]); x.ib = __float_as_int(q[6 * plane]);
      s = merge(s, x);
    }
  }
  red[g][pl] = s;
  __syncthreads();
  if (g == 0 && pos < n) {
    for (int i = 1; i < FG; ++i) s = merge(s, red[i][pl]);
    const RowResult r = finish(s);
    out.kl[pos] = r.kl;
    if (out.lse_ref) out.lse_ref[pos] = r.lse_a;
    if (out.lse_cand) out.lse_cand[pos] = r.lse_b;
    if (out.argmax_ref) out.argmax_ref[pos] = r.ia;
    if (out.argmax_cand) out.argmax_cand[pos] = r.ib;
    if (target) {
      if (out.nll_ref) out.nll_ref[pos] = (float)((double)r.lse_a - (double)zt[pos]);
      if (out.nll_cand) out.nll_cand[pos] = (float)((double)r.lse_b - (double)zt[n + pos]);
    }
  }
}

}  // namespace

FusedGeom fused_geom(int64_t n, int64_t v) {
  FusedGeom g;
  g.nvt = (v + BV - 1) / BV;
  g.npt = (n + BP - 1) / BP;
  g.npad = g.npt * BP;
  return g;
}

hipError_t launch_fused(const FusedArgs &a, float *part, float *zt) {
  const FusedGeom g = fused_geom(a.n, a.v);
  // 128 KB of LDS per block (above the 64 KB default): set on every call so
  // that no library state is kept; the call is host-side and cheap.
  hipError_t e = hipFuncSetAttribute((const void *)fused_head_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     2 * STAGE_CHUNKS * (int)sizeof(u32x4));
  if (e != hipSuccess) return e;
  const int64_t nblocks = g.nvt * g.npt;
  e = record(a.ev.start, a.stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fused_head_kernel, dim3((unsigned)nblocks), dim3(NT),
                     2 * STAGE_CHUNKS * sizeof(u32x4), a.stream, a.W, a.h_ref, a.h_cand, a.v, a.d,
                     a.n, (int)g.npt, g.npad, g.nvt, part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = record(a.ev.stop, a.stream);
  if (e != hipSuccess) return e;
  if (a.target) {
    hipLaunchKernelGGL(target_logit_kernel, dim3((unsigned)((a.n + 3) / 4)), dim3(256), 0,
                       a.stream, a.W, a.h_ref, a.h_cand, a.v, a.d, a.n, a.target, zt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fused_finalize_kernel, dim3((unsigned)((a.n + FP - 1) / FP)), dim3(FP * FG), 0,
                     a.stream, part, g.nvt, g.npad, a.n, zt, a.target, a.out);
  return hipGetLastError();
}

}  // namespace kld

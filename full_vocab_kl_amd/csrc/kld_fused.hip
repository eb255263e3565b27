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
// register slot.  Operands stream straight from global memory into a
// 5-unit LDS ring (buffer loads into LDS, 16 bytes per lane): a stage of 64
// hidden elements is a head unit and a hidden unit of 256 rows x 128 bytes
// each, and three units are in flight while a stage is consumed.  Whole
// 128-byte row segments per load matter on gfx950: measured, L2-resident
// loads of 64-byte row pieces move about two thirds of the bytes per cycle
// that 128-byte segments do.  Rows carry an XOR swizzle so fragment reads
// spread over the LDS banks.
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
constexpr int CH = BK / 8;         // 16-byte chunks per staged row (128-byte rows)
constexpr int NT = 256;            // threads per block (4 waves: 2 vocab x 2 position)
constexpr int UROWS = 256;         // staged rows per unit: a stage is a head unit + a hidden unit
constexpr int UCHUNKS = UROWS * CH;                 // 2048 chunks = 32 KB
constexpr int NSLOT = 5;                            // units in the LDS ring
constexpr int ULOADS = UCHUNKS / 64 / (NT / 64);    // wave-wide loads per wave per unit
constexpr int kXcds = 8;
constexpr size_t kFusedLds = (size_t)NSLOT * UCHUNKS * 16;   // 160 KB

static_assert(ULOADS == 8 && BV == UROWS && 2 * BP == UROWS, "tile shape");

// Swizzled position of chunk c of staged row r.  Rows are 128 bytes (8
// chunks); the chunk index is XORed with (r ^ r >> 3) & 7.  Measured on gfx950
// (SQ_LDS_BANK_CONFLICT), the fragment reads -- lanes 0..31 on 32 consecutive
// rows at chunk c, lanes 32..63 on the same rows at chunk c + 1 -- are then
// free of bank conflicts.
__device__ __forceinline__ int swz_key(int r) { return (r ^ (r >> 3)) & 7; }
__device__ __forceinline__ int swz(int r, int c) { return r * CH + (c ^ swz_key(r)); }

// Workgroup execution barrier without the memory fence of __syncthreads();
// the memory clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt immediate that waits until at most `vm` vector-memory operations
// of this wave are outstanding (expcnt and lgkmcnt left unconstrained).
template <int vm>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(vm >= 0 && vm < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until every LDS access of this wave has completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// Map the hardware block id to a logical tile id so that each XCD gets a
// contiguous range of logical ids.
__device__ __forceinline__ int logical_block(int b, int nb) {
  const int xcd = b % kXcds, slot = b / kXcds;
  const int q = nb / kXcds, r = nb % kXcds;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + slot;
}

// Buffer resource over `bytes` bytes at p (raw addressing, no stride): loads
// at offsets past the range return zero and touch no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
  const int num = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, num, 0x00020000);
}

template <bool TOPK>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fused_head_kernel(const uint16_t *__restrict__ W, const uint16_t *__restrict__ Hr,
                       const uint16_t *__restrict__ Hc, int64_t v, int64_t d, int64_t n, int npt,
                       int64_t npad, int64_t nvt, float *__restrict__ part,
                       uint64_t *__restrict__ ckeys, float *__restrict__ resid) {
  extern __shared__ u32x4 smem[];   // [NSLOT][UCHUNKS]

  const int L = logical_block((int)blockIdx.x, (int)gridDim.x);
  const int vt = L / npt, pt = L % npt;
  const int64_t v0 = (int64_t)vt * BV, p0 = (int64_t)pt * BP;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = wave >> 1, wp = wave & 1;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // ---- global -> LDS staging.  A stage (BK hidden elements) is two units of
  // 256 staged rows x 128 bytes: the head unit (rows = vocabulary ids v0 ..
  // v0 + 255) and the hidden unit (rows 0..127 reference positions p0 .., rows
  // 128..255 candidate positions).  Unit u = 2 s + (0 head | 1 hidden) of
  // stage s lives in ring slot u % 5.  Wave w fills rows 64 w .. 64 w + 63 of
  // a unit with 8 wave-wide 16-byte buffer loads straight into LDS: load j
  // covers rows 64 w + 8 j .. + 7, lane i lands at physical chunk i % 8 of row
  // 64 w + 8 j + i / 8 and fetches the logical chunk (i % 8) ^ swizzle(row),
  // so every load reads eight whole 128-byte row segments.  Rows past v or n
  // read a clamped valid row (their results are masked or discarded); hidden
  // elements past d are zeroed in the fragments of the last stage.
  uint32_t vo_w[ULOADS], vo_h[ULOADS];   // byte offsets of this lane's chunk in row block
#pragma unroll
  for (int j = 0; j < ULOADS; ++j) {
    const int r = 64 * wave + 8 * j + (lane >> 3);
    const int cl = (lane & 7) ^ swz_key(r);
    const int64_t rw = v0 + r < v ? r : v - 1 - v0;
    const int q = r & (BP - 1);
    const int64_t rh = p0 + q < n ? q : n - 1 - p0;
    vo_w[j] = (uint32_t)(rw * d * 2 + cl * 16);
    vo_h[j] = (uint32_t)(rh * d * 2 + cl * 16);
  }
  const uint16_t *wbase = W + v0 * d;
  const uint16_t *hbase = (wave_u < 2 ? Hr : Hc) + p0 * d;
  const int64_t wbytes = (v - v0) * d * 2, hbytes = (n - p0) * d * 2;
  const int KT = (int)((d + BK - 1) / BK);
  const bool ktail = (d % BK) != 0;

  // Issue loads j0 .. j0 + cnt - 1 of the head (H = false) or hidden unit of
  // stage st.  The resource starts at the stage's first element, so offsets
  // past the end of the operand -- the K tail of its last row, and stages past
  // the last one -- fetch nothing.
  auto issue = [&](int st, bool H, int j0, int cnt) {
    const int64_t kb = (int64_t)st * BK * 2;
    const __amdgpu_buffer_rsrc_t rs =
        H ? make_rsrc(hbase + (int64_t)st * BK, hbytes - kb) : make_rsrc(wbase + (int64_t)st * BK, wbytes - kb);
    u32x4 *dst = smem + ((2 * st + (H ? 1 : 0)) % NSLOT) * UCHUNKS + wave_u * (UCHUNKS / 4);
#pragma unroll
    for (int j = j0; j < j0 + cnt; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void *)(dst + j * 64), 16, H ? vo_h[j] : vo_w[j],
          0, 0, 0);
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

  const int fr = lane & 31, fh = lane >> 5;
  // fragments of one 16-wide K step: 4 head (A) and 2 x 2 hidden (B) operands.
  // K step ks of a stage uses chunks 2 ks (lanes 0..31) and 2 ks + 1 (lanes
  // 32..63) of the same rows for both operands.
  struct Frags {
    bf16x8 a[4], b[2][2];
  };
  auto load_frags = [&](int st, int ks, Frags &f) {
    const u32x4 *sw = smem + ((2 * st) % NSLOT) * UCHUNKS;
    const u32x4 *sh = smem + ((2 * st + 1) % NSLOT) * UCHUNKS;
    const int c = 2 * ks + fh;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int sd = 0; sd < 2; ++sd)
        f.b[pg][sd] = __builtin_bit_cast(bf16x8, sh[swz(sd * BP + wp * 64 + pg * 32 + fr, c)]);
#pragma unroll
    for (int vs = 0; vs < 4; ++vs)
      f.a[vs] = __builtin_bit_cast(bf16x8, sw[swz(wv * 128 + vs * 32 + fr, c)]);
  };
  auto mfma = [&](const Frags &f) {
#pragma unroll
    for (int vs = 0; vs < 4; ++vs)
#pragma unroll
      for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int sd = 0; sd < 2; ++sd)
          acc[vs][pg][sd] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[vs], f.b[pg][sd], acc[vs][pg][sd], 0, 0, 0);
  };
  // Hidden elements past d (the last stage of a width that is not a multiple
  // of BK) hold zeros or data of the next row; zero both operands there.
  auto mask_tail = [&](Frags &f, int st, int ks) {
    if ((int64_t)st * BK + (2 * ks + fh) * 8 >= d) {
      const bf16x8 z = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
      for (int vs = 0; vs < 4; ++vs) f.a[vs] = z;
#pragma unroll
      for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int sd = 0; sd < 2; ++sd) f.b[pg][sd] = z;
    }
  };
  // 16 MFMAs interleaved with 8 LDS fragment reads and 4 global loads.
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one global load
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };

  // Software pipeline (per wave).  Stage s runs four K steps of 16 MFMAs on
  // four fragment buffers; each K step reads the fragments of the step two
  // ahead and issues 4 of the 16 loads that go out between two barriers.
  // Barrier s sits between K steps 1 and 2 of stage s.  Between barrier s - 1
  // and barrier s (K steps 2, 3 of stage s - 1 and 0, 1 of stage s) a wave
  // issues the hidden unit of stage s + 1 (unit 2 s + 3) and then the head
  // unit of stage s + 2 (unit 2 s + 4), into the slots of stage s - 1, which
  // every wave released at barrier s - 1.  Before barrier s a wave waits for
  // its loads of stage s + 1 (all but the last 8 loads) and for its own LDS
  // reads, the last of which belong to stage s, so after the barrier stage
  // s + 1 is in LDS and the slots of stage s are free.  Units of stages past
  // the last one read in-bounds data, or nothing, into free slots, which
  // keeps the loop free of branches.
  static_assert(NSLOT == 5, "the schedule below keeps three units ahead");
  Frags f0, f1, f2, f3;
  issue(0, false, 0, ULOADS);
  issue(0, true, 0, ULOADS);
  issue(1, false, 0, ULOADS);
  issue(1, true, 0, ULOADS);
  wait_vmcnt<2 * ULOADS>();   // stage 0 has landed
  block_barrier();
  load_frags(0, 0, f0);
  load_frags(0, 1, f1);
  for (int s = 0; s + 1 < KT; ++s) {
    load_frags(s, 2, f2);
    issue(s + 2, false, 0, ULOADS / 2);
    mfma(f0);
    interleave();
    load_frags(s, 3, f3);
    issue(s + 2, false, ULOADS / 2, ULOADS / 2);
    mfma(f1);
    interleave();
    wait_vmcnt<ULOADS>();
    wait_lgkm0();
    block_barrier();
    load_frags(s + 1, 0, f0);
    issue(s + 2, true, 0, ULOADS / 2);
    mfma(f2);
    interleave();
    load_frags(s + 1, 1, f1);
    issue(s + 2, true, ULOADS / 2, ULOADS / 2);
    mfma(f3);
    interleave();
  }
  {   // last stage
    const int s = KT - 1;
    load_frags(s, 2, f2);
    load_frags(s, 3, f3);
    if (ktail) {
      mask_tail(f0, s, 0);
      mask_tail(f1, s, 1);
      mask_tail(f2, s, 2);
      mask_tail(f3, s, 3);
    }
    mfma(f0);
    mfma(f1);
    mfma(f2);
    mfma(f3);
  }
  wait_vmcnt<0>();   // no load may still write LDS when the epilogue reuses it
  __syncthreads();   // all fragment reads done before the epilogue reuses LDS

  // ---- epilogue: lane holds position p0 + wp*64 + pg*32 + (lane & 31) and
  // vocabulary ids vb + 32 vs + 8 (i / 4) + (i % 4), vb = v0 + 128 wv + 4 (lane >> 5).
  // Each (lane, vs) holds a group of 16 ids of one position.  Per side and
  // group: the maximum m1 with its lowest id and the second largest value m2.
  // The row maximum and argmax come from the group maxima.  With top-k, every
  // group maximum is written as a candidate key and the tile's residual --
  // the largest m2 over its 16 groups -- bounds every id that is not a
  // candidate.
  const int64_t vb = v0 + wv * 128 + 4 * fh;
  const bool vtail = v0 + BV > v;
  RowState *xch = reinterpret_cast<RowState *>(smem);          // [2 pos waves][2 pg][32]
  float *rx = reinterpret_cast<float *>(xch + 2 * 2 * 32);       // [2 sides][2][2][32]
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
    float gm1[2][4], gm2[2][4];
    int gid[2][4];
#pragma unroll
    for (int sd = 0; sd < 2; ++sd)
#pragma unroll
      for (int vs = 0; vs < 4; ++vs) {
        float m1 = kNegInf, m2 = kNegInf;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float x = acc[vs][pg][sd][i];
          if (TOPK) m2 = fmaxf(m2, fminf(m1, x));
          m1 = fmaxf(m1, x);
        }
        int id = kNoId;
#pragma unroll
        for (int i = 15; i >= 0; --i)
          if (acc[vs][pg][sd][i] == m1) id = 32 * vs + 8 * (i >> 2) + (i & 3);
        gm1[sd][vs] = m1; gm2[sd][vs] = m2; gid[sd][vs] = id;
      }
    float ma = gm1[0][0], mb = gm1[1][0];
    int ia = gid[0][0], ib = gid[1][0];
#pragma unroll
    for (int vs = 1; vs < 4; ++vs) {   // groups ascend in id: strict > keeps the lowest id
      if (gm1[0][vs] > ma) { ma = gm1[0][vs]; ia = gid[0][vs]; }
      if (gm1[1][vs] > mb) { mb = gm1[1][vs]; ib = gid[1][vs]; }
    }
    if (ma == kNegInf) ia = kNoId;
    if (mb == kNegInf) ib = kNoId;
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
    const int64_t pos = p0 + wp * 64 + pg * 32 + fr;
    float r2[2] = {kNegInf, kNegInf};
    if constexpr (TOPK) {
#pragma unroll
      for (int sd = 0; sd < 2; ++sd) {
        float r = fmaxf(fmaxf(gm2[sd][0], gm2[sd][1]), fmaxf(gm2[sd][2], gm2[sd][3]));
        r2[sd] = fmaxf(r, __shfl_xor(r, 32));
        if (pos < n) {
          uint64_t *dst = ckeys + (((int64_t)sd * nvt + vt) * npad + pos) * 16 + (wv * 2 + fh) * 4;
#pragma unroll
          for (int vs = 0; vs < 4; ++vs)
            dst[vs] = gm1[sd][vs] == kNegInf ? 0ull : topk_key(gm1[sd][vs], (int)(vb + gid[sd][vs]));
        }
      }
    }
    if (wv == 1 && fh == 0) {
      xch[(wp * 2 + pg) * 32 + fr] = st;
      if (TOPK) {
        rx[((0 * 2 + wp) * 2 + pg) * 32 + fr] = r2[0];
        rx[((1 * 2 + wp) * 2 + pg) * 32 + fr] = r2[1];
      }
    }
    __syncthreads();
    if (wv == 0 && fh == 0 && pos < n) {
      st = merge(st, xch[(wp * 2 + pg) * 32 + fr]);
      const int64_t plane = nvt * npad;
      float *q = part + (int64_t)vt * npad + pos;
      q[0] = st.ma; q[plane] = st.sa; q[2 * plane] = st.t; q[3 * plane] = st.mb;
      q[4 * plane] = st.sb;
      q[5 * plane] = __int_as_float(st.ia);
      q[6 * plane] = __int_as_float(st.ib);
      if (TOPK) {
        resid[((int64_t)0 * nvt + vt) * npad + pos] =
            fmaxf(r2[0], rx[((0 * 2 + wp) * 2 + pg) * 32 + fr]);
        resid[((int64_t)1 * nvt + vt) * npad + pos] =
            fmaxf(r2[1], rx[((1 * 2 + wp) * 2 + pg) * 32 + fr]);
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
    const float *__restrict__ zt, const int32_t *__restrict__ target, RowsOut out,
    double *__restrict__ lse_d) {
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
    if (lse_d) {
      lse_d[pos] = (double)ref_of(s.ma) + log((double)s.sa);
      lse_d[n + pos] = (double)ref_of(s.mb) + log((double)s.sb);
    }
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

// Exact top-64 of one (position, side) from the fused kernel's candidates.
//
// Candidates: for every vocabulary tile, the maximum of each of its 16
// groups (key = value bits, then complemented id).  Every id that is not a
// candidate is <= its tile's residual (the largest second-largest value of
// the tile's groups).
//  A. Radix-narrow (8 bits per pass, MSB first) the bucket that holds the
//     64th largest candidate key until it fits the LDS buffer; gather every
//     key at or above that bucket, sort, keep 64.  T = the 64th key.
//  B. Any tile whose residual reaches T's value may hide an id that belongs
//     in the top 64 (or fewer than 64 candidates exist): its 256 logits are
//     recomputed here from W and h (f32 dot products), its old candidates
//     are dropped, and the running top 64 is re-cut.  On generic inputs no
//     tile is flagged; degenerate inputs (exact ties across many ids) only
//     cost time.
//  C. Write ids and fp16 log-probs lp = z - lse.
constexpr int TK = 256;
constexpr int kSelBuf = 4096;
__global__ __launch_bounds__(TK) void fused_topk_kernel(
    const uint64_t *__restrict__ ckeys, const float *__restrict__ resid, int64_t nvt, int64_t npad,
    int64_t n, const uint16_t *__restrict__ W, const uint16_t *__restrict__ Hr,
    const uint16_t *__restrict__ Hc, int64_t v, int64_t d, const double *__restrict__ lse_d,
    TopkOut out) {
  const int64_t pos = blockIdx.x >> 1;
  const int side = blockIdx.x & 1;
  int32_t *ids = side ? out.ids_cand : out.ids_ref;
  uint16_t *lp = side ? out.lp_cand : out.lp_ref;
  if ((!ids && !lp) || pos >= n) return;

  __shared__ uint32_t hist[256];
  __shared__ uint64_t buf[kSelBuf];
  __shared__ uint64_t sh_prefix;
  __shared__ int sh_pbits, sh_need, sh_cnt, sh_fill, sh_nflag;
  __shared__ int flagged[TK];

  const uint64_t *base = ckeys + ((int64_t)side * nvt * npad + pos) * 16;
  const int64_t total = nvt * 16;
  const int64_t tstride = npad * 16;
  const int tid = threadIdx.x;

  // ---- A: narrow the bucket of the 64th largest candidate key
  uint64_t prefix = 0;
  int pbits = 0, need = 64;
  for (;;) {
    hist[tid] = 0;
    __syncthreads();
    for (int64_t i = tid; i < total; i += TK) {
      const uint64_t k = base[(i >> 4) * tstride + (i & 15)];
      if (pbits == 0 || (k >> (64 - pbits)) == prefix) atomicAdd(&hist[(k >> (56 - pbits)) & 255], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, dd = 0;
      for (dd = 255; dd > 0; --dd) {
        if (cum + (int)hist[dd] >= need) break;
        cum += (int)hist[dd];
      }
      sh_need = need - cum;
      sh_prefix = (prefix << 8) | (uint64_t)dd;
      sh_pbits = pbits + 8;
      sh_cnt = (int)hist[dd];
    }
    __syncthreads();
    prefix = sh_prefix; pbits = sh_pbits; need = sh_need;
    const int cnt = sh_cnt;
    __syncthreads();
    if (pbits == 64 || cnt <= kSelBuf - 64) break;
  }
  // gather every key whose top pbits reach the bucket
  if (tid == 0) sh_fill = 0;
  __syncthreads();
  for (int64_t i = tid; i < total; i += TK) {
    const uint64_t k = base[(i >> 4) * tstride + (i & 15)];
    if ((pbits == 64 ? k : (k >> (64 - pbits))) >= prefix && k != 0ull) {
      const int slot = atomicAdd(&sh_fill, 1);
      buf[slot] = k;
    }
  }
  __syncthreads();
  {
    const int fill = sh_fill;
    int m = 64;
    while (m < fill) m <<= 1;
    for (int i = fill + tid; i < m; i += TK) buf[i] = 0ull;
    __syncthreads();
    bitonic_desc<TK>(buf, m);
  }
  const uint64_t T = buf[63];
  const float tval = key_value(T);

  // ---- B: recompute tiles whose residual reaches T (all tiles if T is unset)
  const uint16_t *h = (side ? Hc : Hr) + pos * d;
  for (int64_t r0 = 0; r0 < nvt; r0 += TK) {
    if (tid == 0) sh_nflag = 0;
    __syncthreads();
    const int64_t vt = r0 + tid;
    if (vt < nvt && (T == 0ull || resid[((int64_t)side * nvt + vt) * npad + pos] >= tval))
      flagged[atomicAdd(&sh_nflag, 1)] = (int)vt;
    __syncthreads();
    const int nf = sh_nflag;
    for (int f = 0; f < nf; ++f) {
      const int64_t t0 = (int64_t)flagged[f] * BV;   // the tile's first id
      // drop the tile's old candidates from the running top 64
      if (tid < 64) {
        const int id = key_id(buf[tid]);
        if (buf[tid] != 0ull && id >= t0 && id < t0 + BV) buf[tid] = 0ull;
      }
      // its 256 logits, one per thread
      const int64_t j = t0 + tid;
      uint64_t k = 0ull;
      if (j < v) {
        const uint16_t *w = W + j * d;
        float z = 0.f;
        for (int64_t e = 0; e < d; e += 8) {
          const u32x4 qw = *reinterpret_cast<const u32x4 *>(w + e);
          const u32x4 qh = *reinterpret_cast<const u32x4 *>(h + e);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            z = fmaf(__uint_as_float(qw[q] << 16), __uint_as_float(qh[q] << 16), z);
            z = fmaf(__uint_as_float(qw[q] & 0xffff0000u), __uint_as_float(qh[q] & 0xffff0000u), z);
          }
        }
        k = topk_key(z, (int)j);
      }
      buf[64 + tid] = k;
      for (int i = 64 + TK + tid; i < 512; i += TK) buf[i] = 0ull;
      __syncthreads();
      bitonic_desc<TK>(buf, 512);
    }
    __syncthreads();
  }

  // ---- C: ids and log-probs
  if (tid < 64) {
    const uint64_t k = buf[tid];
    const double l = lse_d[(int64_t)side * n + pos];
    if (ids) ids[pos * 64 + tid] = key_id(k);
    if (lp) lp[pos * 64 + tid] = f32_to_f16_bits((float)((double)key_value(k) - l));
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

hipError_t launch_fused(const FusedArgs &a, const FusedWs &w) {
  const FusedGeom g = fused_geom(a.n, a.v);
  const bool tk = a.topk.ids_ref || a.topk.lp_ref || a.topk.ids_cand || a.topk.lp_cand;
  const void *kern = tk ? (const void *)fused_head_kernel<true> : (const void *)fused_head_kernel<false>;
  // 128 KB of LDS per block (above the 64 KB default): set on every call so
  // that no library state is kept; the call is host-side and cheap.
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)kFusedLds);
  if (e != hipSuccess) return e;
  const int64_t nblocks = g.nvt * g.npt;
  e = record(a.ev.start, a.stream);
  if (e != hipSuccess) return e;
  if (tk)
    hipLaunchKernelGGL(fused_head_kernel<true>, dim3((unsigned)nblocks), dim3(NT),
                       kFusedLds, a.stream, a.W, a.h_ref, a.h_cand, a.v, a.d,
                       a.n, (int)g.npt, g.npad, g.nvt, w.part, w.ckeys, w.resid);
  else
    hipLaunchKernelGGL(fused_head_kernel<false>, dim3((unsigned)nblocks), dim3(NT),
                       kFusedLds, a.stream, a.W, a.h_ref, a.h_cand, a.v, a.d,
                       a.n, (int)g.npt, g.npad, g.nvt, w.part, nullptr, nullptr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = record(a.ev.stop, a.stream);
  if (e != hipSuccess) return e;
  if (a.target) {
    hipLaunchKernelGGL(target_logit_kernel, dim3((unsigned)((a.n + 3) / 4)), dim3(256), 0,
                       a.stream, a.W, a.h_ref, a.h_cand, a.v, a.d, a.n, a.target, w.zt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(fused_finalize_kernel, dim3((unsigned)((a.n + FP - 1) / FP)), dim3(FP * FG), 0,
                     a.stream, w.part, g.nvt, g.npad, a.n, w.zt, a.target, a.out, w.lse);
  e = hipGetLastError();
  if (e != hipSuccess || !tk) return e;
  hipLaunchKernelGGL(fused_topk_kernel, dim3((unsigned)(2 * a.n)), dim3(TK), 0, a.stream, w.ckeys,
                     w.resid, g.nvt, g.npad, a.n, a.W, a.h_ref, a.h_cand, a.v, a.d, w.lse, a.topk);
  return hipGetLastError();
}

}  // namespace kld

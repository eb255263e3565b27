// Logits path: one streaming pass over the reference and candidate logit rows.
//
// Each block owns one (row, vocabulary split) pair and streams both rows'
// slices once, coalesced, 16 bytes per lane per load.  Every lane folds its
// elements into an online RowState (kld_device.hpp), batch by batch: one max
// per batch, a rebase when the maximum moves, then one fma and one exp2 per
// element per side.  The plain kernels take the wave's maximum as the offset,
// so the rebase and the argmax search run only when the wave's maximum rises;
// the top-k kernels keep each lane's own maximum, which their threshold
// needs, and locate the argmax id after the loop.  Lanes merge by butterfly,
// waves through LDS, and the block writes one partial state;
// finalize_rows_kernel merges the splits (in f64) in a fixed order and writes
// the per-position outputs.  HBM-bound: 2 v sizeof(T) bytes per position are
// read once.
//
// Top-64 export ("Qwopus3.8-27B-Coder-Flash: quality-eval reference",
// "Files": top-64 ids and fp16 log-probs, sorted) rides the same pass.  Each
// element is ranked by a 64-bit key (order-preserving f32 bits, then the
// complemented id, so equal values rank the lower id first).  Per side, an
// element becomes a candidate only if its value reaches a threshold that at
// least 64 elements of the block's range are known to reach: at rounds 0, 1,
// 2, 3, 5, 7, 11, 15, ... every wave finds the 16th largest of its 64 lanes'
// running maxima (distinct elements) and publishes it; the smallest of the
// four waves' values is reached by 64 distinct elements.  Candidates are
// appended to a per-wave LDS buffer (ballot + mbcnt offsets, no atomics, no
// block barrier in the streaming loop); a wave whose buffer fills sorts it
// in registers, keeps its 64 best keys and from then on also requires keys
// above the 64th.  At the end each wave drops the entries below the final
// threshold; after a block barrier one wave per side gathers the four waves'
// survivors and cuts them to the 64 best (the two sides in parallel, beside
// a third wave that merges the row states); topk_merge_kernel (kld_topk.hip)
// merges the splits of a row and converts them to ids and fp16 log-probs.  On
// these inputs only a few hundred elements per row and side pass the
// threshold, so the export costs little beyond the streaming pass.
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

// 16 bytes of a row as loaded: 4 f32 or 8 bf16 elements.
constexpr int kNonTemporal = 2;   // buffer-load cache policy: streaming (nt)

template <typename T> struct RawOf;
template <> struct RawOf<float> { using type = f32x4; };
template <> struct RawOf<uint16_t> { using type = u32x4; };

// Load the VEC elements starting at element `pos` of a row; elements at or
// beyond `hi` read as -inf.  Fast path: one 16-byte load when the whole
// vector is in range and the row is 16-byte aligned.
template <typename T, int VEC, bool ALIGNED>
__device__ __forceinline__ typename RawOf<T>::type load_raw(const T *__restrict__ row, int64_t pos,
                                                           int64_t hi) {
  using R = typename RawOf<T>::type;
  if (ALIGNED && pos + VEC <= hi) return __builtin_nontemporal_load(reinterpret_cast<const R *>(row + pos));
  R r;
  if constexpr (sizeof(T) == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = pos + j < hi ? row[pos + j] : kNegInf;
  } else {
    constexpr uint32_t kNegInfBf16 = 0xff80u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t a = pos + 2 * i < hi ? row[pos + 2 * i] : kNegInfBf16;
      const uint32_t b = pos + 2 * i + 1 < hi ? row[pos + 2 * i + 1] : kNegInfBf16;
      r[i] = a | (b << 16);
    }
  }
  return r;
}

// Element j of a loaded vector, as f32.
__device__ __forceinline__ float elem(const f32x4 &q, int j) { return q[j]; }
__device__ __forceinline__ float elem(const u32x4 &q, int j) {
  return __uint_as_float((j & 1) ? (q[j >> 1] & 0xffff0000u) : (q[j >> 1] << 16));
}
// Element j of a loaded vector set to -inf.
__device__ __forceinline__ void set_neg_inf(f32x4 &q, int j) { q[j] = kNegInf; }
__device__ __forceinline__ void set_neg_inf(u32x4 &q, int j) {
  q[j >> 1] = (j & 1) ? ((q[j >> 1] & 0x0000ffffu) | 0xff800000u) : ((q[j >> 1] & 0xffff0000u) | 0xff80u);
}
__device__ __forceinline__ void set_elem(f32x4 &q, int j, float x) { q[j] = x; }
__device__ __forceinline__ void set_elem(u32x4 &q, int j, uint16_t x) {
  q[j >> 1] = (j & 1) ? ((q[j >> 1] & 0x0000ffffu) | ((uint32_t)x << 16))
                      : ((q[j >> 1] & 0xffff0000u) | x);
}

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kWCap = 256;            // candidate keys per wave and side (64 kept + room for batches)

// SCAP staged vectors per wave and side.
template <int SCAP>
struct TopkShared {
  uint64_t buf[2][kWaves][kWCap];     // per side and wave: appended candidates (make_entry)
  u32x4 stage[2][kWaves][SCAP];       // per side and wave: staged vectors (as loaded)
  int sid[2][kWaves][SCAP];           // id of each staged vector's first element
  float bound[2][kWaves];             // per side and wave: threshold bound (nondecreasing)
  int lcount[2][kWaves];              // per side and wave: entries in its final list
};

// Values that are equal in every lane, moved to scalar registers so that the
// compiler treats them (and branches on them) as wave-uniform.
__device__ __forceinline__ float uniform_f(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
// Maximum over the wave's 64 lanes (no NaN among them), in a scalar register.
__device__ __forceinline__ float wave_max_uniform(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return uniform_f(x);
}
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(x >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Candidate buffer entries hold (value bits, id) as they were appended; the
// 64-bit ranking key is formed only when the entries are ranked.
__device__ __forceinline__ uint64_t make_entry(float x, int id) {
  return ((uint64_t)(uint32_t)id << 32) | __float_as_uint(x);
}
__device__ __forceinline__ uint64_t entry_key(uint64_t e) {
  return topk_key(__uint_as_float((uint32_t)e), (int)(e >> 32));
}

// Two key lists of 64, one key per lane, each sorted descending: a from
// lane order, b given reversed (lane l holds b[63 - l]).  Returns the 64
// largest keys of both, sorted descending: the lane-wise maximum of a and
// reversed b holds them as a bitonic sequence, which a half-cleaner cascade
// sorts.
__device__ __forceinline__ uint64_t wave_merge_top64(uint64_t a, uint64_t b_rev) {
  const int lane = threadIdx.x & 63;
  uint64_t c = a > b_rev ? a : b_rev;
#pragma unroll
  for (int j = 32; j > 0; j >>= 1) {
    const uint64_t o = __shfl_xor(c, j);
    c = (lane & j) == 0 ? (o > c ? o : c) : (o < c ? o : c);
  }
  return c;
}

// A lower bound of the 16th largest of the wave's 64 lane values, exact to
// the top 16 bits of its order-preserving key (all of a bf16 value): the
// bits are fixed from the top, each kept if at least 16 lanes reach it (a
// ballot and a popcount per bit; no shuffles).  Two values per lane (the two
// sides) are searched together, so the two dependency chains overlap.
__device__ __forceinline__ uint32_t order_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
__device__ __forceinline__ void wave_16th_bound2(float x, float y, float &bx, float &by) {
  const uint32_t kx = order_key(x), ky = order_key(y);
  uint32_t px = 0, py = 0;
#pragma unroll
  for (int b = 31; b >= 16; --b) {
    const uint32_t cx = px | (1u << b), cy = py | (1u << b);
    const int nx = __popcll(__ballot(kx >= cx)), ny = __popcll(__ballot(ky >= cy));
    px = nx >= 16 ? cx : px;
    py = ny >= 16 ? cy : py;
  }
  bx = key_float(px);
  by = key_float(py);
}

// The 64 best keys of a wave's candidate buffer (its first cnt of kWCap
// entries, LDS), sorted descending, one per lane (0 past cnt): each group of
// 64 entries is sorted across the lanes and merged into the running 64 (lane
// l of group g takes entry 64 g + l).  Registers and shuffles only; not
// inlined, so that its registers do not add to the streaming loop's.
template <typename X> using Lds = __attribute__((address_space(3))) X *;
template <typename X> __device__ __forceinline__ Lds<X> lds(X *p) { return (Lds<X>)p; }

static_assert(kWCap == 4 * 64, "four groups of 64 entries");
__device__ __attribute__((noinline)) uint64_t wave_best64(Lds<const uint64_t> buf, int cnt) {
  const int lane = threadIdx.x & 63;
  uint64_t r = wave_sort_desc(lane < cnt ? entry_key(buf[lane]) : (uint64_t)0);
  for (int g = 1; g < 4 && 64 * g < cnt; ++g) {   // (cnt is wave-uniform)
    const int e = 64 * g + lane;
    const uint64_t b = wave_sort_desc(e < cnt ? entry_key(buf[e]) : (uint64_t)0);
    r = wave_merge_top64(r, __shfl(b, 63 - lane));
  }
  return r;
}

// Per side and wave: the value threshold, the key threshold (0 = none) and
// the number of entries in the wave's candidate buffer.
struct CandState {
  uint64_t tkey;
  float thr;
  int cnt;
};

// Filter a wave's scnt staged vectors (as loaded, with the id of each one's
// first element) against the threshold -- and the key threshold after a
// compaction -- and append the elements that pass to its candidate buffer,
// one element per lane at a time.  A full buffer is cut to its 64 best, which
// sets the key threshold.  (Inlined: as a call it costs more in saved
// registers than its copies cost in code.)
template <typename T, int VEC>
__device__ __forceinline__ CandState topk_flush(Lds<uint64_t> wbuf, Lds<const u32x4> stage,
                                                Lds<const int> sid, int scnt, int64_t hi,
                                                CandState st) {
  using Raw = typename RawOf<T>::type;
  const int lane = threadIdx.x & 63;
  const float th = uniform_f(st.thr);
  for (int b0 = 0; b0 < scnt; b0 += 64) {
    const int e = b0 + lane;
    const bool ok = e < scnt;
    const Raw q = __builtin_bit_cast(Raw, ok ? stage[e] : u32x4{0u, 0u, 0u, 0u});
    const int bid = ok ? sid[e] : 0;
#pragma unroll
    for (int j = 0; j < VEC; ++j) {
      const float x = elem(q, j);
      const int id = bid + j;
      bool p = ok && x >= th && (int64_t)id < hi;
      if (st.tkey != 0ull) p = p && topk_key(x, id) > st.tkey;
      uint64_t m = __ballot(p);
      if (m == 0ull) continue;
      if (st.cnt + 64 > kWCap) {
        // buffer full: keep its 64 best, filter this element again (each
        // lane reads its four entries before any lane writes)
        const uint64_t kb = wave_best64(wbuf, st.cnt);
        wbuf[lane] = make_entry(key_value(kb), key_id(kb));
        st.tkey = uniform_u64(__shfl(kb, 63));
        st.cnt = 64;
        st.thr = uniform_f(fmaxf(st.thr, key_value(st.tkey)));
        p = p && topk_key(x, id) > st.tkey;
        m = __ballot(p);
        if (m == 0ull) continue;
      }
      const int at = st.cnt + (int)__builtin_amdgcn_mbcnt_hi(
          (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (p) wbuf[at] = make_entry(x, id);
      st.cnt += __popcll(m);
    }
  }
  return st;
}

template <typename T, int VEC, int U, bool ALIGNED, bool TWO, bool TOPK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(TOPK && ALIGNED && sizeof(T) == 2 ? 4 : 1))) void logits_partial_kernel(
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

  constexpr int kSCap = 64 * U > 128 ? 64 * U : 128;   // staged vectors per wave and side
  static_assert(kSCap >= 64 * U, "a round's vectors fit after a flush");
  __shared__ TopkShared<kSCap> sh_storage[1];
  TopkShared<kSCap> &sh = sh_storage[0];
  __shared__ RowState waves[kWaves];
  const int lane = threadIdx.x & 63;
  // the wave index in a scalar register: the per-wave LDS bases become
  // scalars and leave the vector registers to the streaming loop
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  // per side, uniform over the wave: value threshold, key threshold (0 = none)
  // and candidates in the wave's buffer
  float thr[2] = {kNegInf, kNegInf};
  uint64_t tkey[2] = {0ull, 0ull};
  int cnt[2] = {0, 0};    // candidates in the wave's buffer
  int scnt[2] = {0, 0};   // vectors staged by the wave
  if constexpr (TOPK) {
    if (threadIdx.x < 2 * kWaves) (&sh.bound[0][0])[threadIdx.x] = kNegInf;
    __syncthreads();
  }

  // Inside the loop every element costs one fma before its exp2: its
  // exponent is e = x L2E - o against the offset o = ref(m) L2E (f32), and
  // t sums w (e_a - e_b), the log2-scaled difference against both offsets
  // (exact arithmetic would give L2E ((a - ref_a) - (b - ref_b)) + (r_a - r_b),
  // r = ref(m) L2E - o).  fold_offsets converts the sums back after the loop.
  // The maxima ma, mb (so the offsets) are the wave's in the plain kernels
  // and the lane's in the top-k kernels, whose bounds need the lanes' own.
  float ma = kNegInf, sa = 0.f, t = 0.f, mb = kNegInf, sb = 0.f;
  // argmax ids; in the top-k loop, the round in which the lane's maximum rose
  int ia = kNoId, ib = kNoId;

  constexpr int kStride = kThreads * VEC;
  constexpr int kRound = kStride * U;   // ids per round
  // every thread runs the same number of rounds so the block can synchronise;
  // offsets from lo fit 32 bits (a split spans at most 2^28 + 7 ids)
  const int len = (int)(hi - lo);
  const int rounds = (len + kRound - 1) / kRound;
  const int tofs = (int)threadIdx.x * VEC;   // the thread's first offset in a round

  // Rounds r + 1 .. r + DEPTH - 1 are loaded while round r is processed
  // (three rounds in flight for bf16 with top-k, whose rounds are one vector
  // per side: two would leave too few bytes in flight per CU).  Aligned rows
  // are read through buffer resources over the whole vectors of [lo, hi):
  // loads past them return zeros and touch no memory, so the loop carries no
  // bounds checks; the last round masks offsets past hi to -inf and reads a
  // vector that straddles hi element by element.
  using Raw = typename RawOf<T>::type;
  constexpr int DEPTH = (TOPK && sizeof(T) == 2) ? 3 : 2;
  Raw qa[DEPTH][U], qb[DEPTH][U];   // round r in slot r % DEPTH
  const int nvec = len / VEC * VEC;   // ids in whole vectors
  __amdgpu_buffer_rsrc_t rsa, rsb;
  if constexpr (ALIGNED) {
    rsa = __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(ra + lo), (short)0,
                                            nvec * (int)sizeof(T), 0x00020000);
    rsb = __builtin_amdgcn_make_buffer_rsrc(const_cast<T *>(rb + lo), (short)0,
                                            nvec * (int)sizeof(T), 0x00020000);
  }
  // Load round r into slot sl.  Rounds past the last one load nothing (zeros
  // from the buffer resources, -inf from the checked path), so the loop
  // fetches DEPTH rounds ahead without conditions.
  auto fetch = [&](int r, int sl) {
    const int e0 = r * kRound + tofs;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (ALIGNED) {
        const int o = (e0 + u * kStride) * (int)sizeof(T);
        qa[sl][u] = __builtin_bit_cast(Raw, __builtin_amdgcn_raw_buffer_load_b128(rsa, o, 0, kNonTemporal));
        if (TWO) qb[sl][u] = __builtin_bit_cast(Raw, __builtin_amdgcn_raw_buffer_load_b128(rsb, o, 0, kNonTemporal));
      } else {
        qa[sl][u] = load_raw<T, VEC, false>(ra, lo + e0 + u * kStride, hi);
        if (TWO) qb[sl][u] = load_raw<T, VEC, false>(rb, lo + e0 + u * kStride, hi);
      }
    }
  };

  // Raise the value thresholds from the lanes' running maxima: each wave
  // publishes the 16th largest of its 64 (distinct elements, so at least 16
  // of its elements reach it) and takes the smallest of the four waves'
  // latest values, which at least 64 elements reach.  Published values only
  // grow, so reading another wave's older value is still valid: no barrier.
  auto update = [&]() __attribute__((always_inline)) {
    float b16[2];
    wave_16th_bound2(ma, mb, b16[0], b16[1]);   // (mb unused with one side)
    // Relaxed workgroup-scope atomics on LDS addresses: plain LDS reads and
    // writes with no fence (another wave may read an older, smaller value,
    // which is still valid).  Volatile accesses would keep generic addresses
    // and become flat operations, whose wait also drains this wave's
    // prefetched row loads.
#pragma unroll
    for (int side = 0; side < NS; ++side)
      if (lane == 0)
        __hip_atomic_store(lds(&sh.bound[side][wave]), b16[side], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
    for (int side = 0; side < NS; ++side) {
      const Lds<float> bd = lds(sh.bound[side]);
      float b = __hip_atomic_load(bd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
      for (int w = 1; w < kWaves; ++w)
        b = fminf(b, __hip_atomic_load(bd + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
      thr[side] = uniform_f(fmaxf(thr[side], b));
    }
  };

  // Filter the wave's staged vectors of one side (topk_flush).
  auto flush = [&](int side) {
    CandState st{tkey[side], thr[side], cnt[side]};
    st = topk_flush<T, VEC>(lds(sh.buf[side][wave]), lds<const u32x4>(sh.stage[side][wave]),
                            lds<const int>(sh.sid[side][wave]), scnt[side], hi, st);
    tkey[side] = uniform_u64(st.tkey);
    thr[side] = uniform_f(st.thr);
    cnt[side] = __builtin_amdgcn_readfirstlane(st.cnt);
    scnt[side] = 0;
  };

  // One round: elements lo + r * kRound + tofs + u * kStride + j of the
  // vectors ca[u], cb[u].  Values are unpacked where they are used, one
  // vector at a time, so that only the packed round stays in registers.
  // `lim` is the number of valid offsets from the thread's first one (only
  // the last round can have fewer than kRound).
  auto process = [&](int r, const Raw (&ca)[U], const Raw (&cb)[U], bool ragged,
                     int lim) __attribute__((always_inline)) {
    const int id0 = (int)lo + r * kRound + tofs;   // id of element (0, 0)
    float vma[U], vmb[U];   // per-vector maxima
    float bma = kNegInf, bmb = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      vma[u] = kNegInf; vmb[u] = kNegInf;
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        vma[u] = fmaxf(vma[u], elem(ca[u], j));
        if (TWO) vmb[u] = fmaxf(vmb[u], elem(cb[u], j));
      }
      bma = fmaxf(bma, vma[u]);
      if (TWO) bmb = fmaxf(bmb, vmb[u]);
    }
    // Lowest id in this batch whose value equals m (m is one of its
    // non-NaN values): one bit per element, then the lowest set bit -- no
    // per-element id arithmetic, which the compiler would otherwise keep
    // live across the loop.
    auto first_id = [&](const Raw (&c)[U], float m) -> int {
      static_assert(U * VEC <= 32, "one bit per element of a round");
      uint32_t bits = 0;
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < VEC; ++j) bits |= (elem(c[u], j) == m ? 1u : 0u) << (u * VEC + j);
      const int k = __builtin_ctz(bits);
      return id0 + (k / VEC) * kStride + (k % VEC);
    };
    if constexpr (!TOPK) {
      // Plain kernels: the sums are taken against the wave's maximum, so a
      // round costs one compare and a ballot per side, and the rebase and
      // the argmax search run only when the wave's maximum rises (a handful
      // of times per row for typical logits; with a maximum per lane some
      // lane's rose in nearly every round).  Lanes that hold the new maximum
      // locate its lowest id in this batch; the others drop theirs, which
      // the merge never takes from a smaller maximum.  Later rounds that
      // only equal the maximum hold larger ids and change nothing.
      if (__ballot(bma > ma)) {
        const float m = wave_max_uniform(bma);
        const float o = m * kL2E, oa = ref_of(ma) * kL2E;
        const float f = ma == kNegInf ? 0.f : exp2_fast(oa - o);
        if (TWO && sa != 0.f) t = fmaf(-sa, o - oa, t);
        t *= f; sa *= f;
        ia = bma == m ? first_id(ca, m) : kNoId;
        ma = m;
      }
      if (TWO && __ballot(bmb > mb)) {
        const float m = wave_max_uniform(bmb);
        const float o = m * kL2E, ob = ref_of(mb) * kL2E;
        if (sa != 0.f) t = fmaf(sa, o - ob, t);
        sb *= mb == kNegInf ? 0.f : exp2_fast(ob - o);
        ib = bmb == m ? first_id(cb, m) : kNoId;
        mb = m;
      }
    } else {
      // Top-k kernels: the lane's own maximum (the bound needs them).  A
      // rise rebases the lane's sums and records the round; the id is
      // located after the loop, so the many early rounds in which some
      // lane's maximum rises cost the wave no per-element search.  (Measured:
      // the wave's maximum here, with the lanes' kept beside it for the
      // bound, was slower -- this kernel sits at its register limit.)
      if (bma > ma) {
        const float o = bma * kL2E, oa = ref_of(ma) * kL2E;
        const float f = ma == kNegInf ? 0.f : exp2_fast(oa - o);
        if (TWO && sa != 0.f) t = fmaf(-sa, o - oa, t);
        t *= f; sa *= f; ma = bma; ia = r;
      }
      if (TWO && bmb > mb) {
        const float o = bmb * kL2E, ob = ref_of(mb) * kL2E;
        if (sa != 0.f) t = fmaf(sa, o - ob, t);
        sb *= mb == kNegInf ? 0.f : exp2_fast(ob - o);
        mb = bmb; ib = r;
      }
    }
    if constexpr (TOPK) {
      {   // rounds 0, 1, 2, 3, 5, 7, 11, 15, 23, 31, ...: r + 1 = 2^k or 3 * 2^k
        const int x = r + 1, y = x / 3;
        if ((x & (x - 1)) == 0 || (x % 3 == 0 && (y & (y - 1)) == 0)) update();
      }
      // stage the vectors whose maximum reaches the threshold; their elements
      // are filtered in batches (flush), so the common path has no
      // per-element work and a single branch per vector and side
#pragma unroll
      for (int side = 0; side < NS; ++side) {
        const float th = uniform_f(thr[side]);
        bool c[U];
        uint64_t any = 0ull;
#pragma unroll
        for (int u = 0; u < U; ++u) {
          c[u] = (side ? vmb[u] : vma[u]) >= th;
          any |= __ballot(c[u]);
        }
        if (any == 0ull) continue;
        if (scnt[side] + 64 * U > kSCap) flush(side);   // room for this round's vectors
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint64_t m = __ballot(c[u]);
          if (m == 0ull) continue;
          const int at = scnt[side] + (int)__builtin_amdgcn_mbcnt_hi(
              (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (c[u]) {
            sh.stage[side][wave][at] = __builtin_bit_cast(u32x4, side ? cb[u] : ca[u]);
            sh.sid[side][wave][at] = id0 + u * kStride;
          }
          scnt[side] += __popcll(m);
        }
      }
    }
    const float oa = ref_of(ma) * kL2E, ob = ref_of(mb) * kL2E;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float xa[VEC], xb[VEC];
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        xa[j] = elem(ca[u], j);
        if (TWO) xb[j] = elem(cb[u], j);
      }
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float ea = fmaf(xa[j], kL2E, -oa);
        const float w = exp2_fast(ea);
        sa += w;
        if (TWO) {
          const float eb = fmaf(xb[j], kL2E, -ob);
          // e_a - e_b is clamped below so that a -inf reference id (w = 0)
          // adds exactly 0 even when the candidate id is -inf too.
          t = fmaf(w, fmaxf(ea - eb, -kFltMax), t);
          sb += exp2_fast(eb);
        }
      }
    }
  };

  // Round r's packed vectors, with the range end applied in the last round
  // (offsets past hi -> -inf; the vector that straddles hi read element by
  // element), then processed.
  auto run = [&](int r, int sl, bool last) __attribute__((always_inline)) {
    Raw ca[U], cb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) { ca[u] = qa[sl][u]; cb[u] = qb[sl][u]; }
    if (!last) {
      fetch(r + DEPTH, sl);
      process(r, ca, cb, false, kRound);
      return;
    }
    const int lim = len - (r * kRound + tofs);   // valid offsets from the thread's first
    const bool ragged = len < (r + 1) * kRound;
    if (ALIGNED && ragged) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int o = u * kStride;
        if (o < lim && o + VEC > lim && r * kRound + tofs + o >= nvec) {
          // the vector that straddles hi (past the buffer's whole vectors)
          const int64_t pos = lo + r * kRound + tofs + o;
#pragma unroll
          for (int j = 0; j < VEC; ++j)
            if (o + j < lim) {
              set_elem(ca[u], j, ra[pos + j]);
              if (TWO) set_elem(cb[u], j, rb[pos + j]);
            }
        }
#pragma unroll
        for (int j = 0; j < VEC; ++j)
          if (o + j >= lim) {
            set_neg_inf(ca[u], j);
            if (TWO) set_neg_inf(cb[u], j);
          }
      }
    }
    process(r, ca, cb, ragged, lim);
  };

  if (rounds > 0) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) fetch(d, d);
    int r = 0;
    for (; r + DEPTH < rounds; r += DEPTH) {   // none of these rounds is the last
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) run(r + d, d, false);
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)   // the 1 .. DEPTH rounds left
      if (r + d < rounds) run(r + d, d, r + d == rounds - 1);
  }

  if constexpr (TOPK) {
    // Last threshold from the final maxima and the remaining staged
    // vectors.  At least 64 elements of the range reach the threshold, so
    // the range's top 64 do too: entries below it are dropped (most of the
    // buffer, whose early entries met lower thresholds).  The survivors --
    // cut to the wave's 64 best only when more remain -- form the wave's
    // list in its staging area, which is free now.
    update();
#pragma unroll
    for (int side = 0; side < NS; ++side) {
      flush(side);
      uint64_t *wbuf = sh.buf[side][wave];
      const float th = uniform_f(thr[side]);
      int n2 = 0;
      for (int g = 0; g < kWCap / 64 && 64 * g < cnt[side]; ++g) {
        // compacting forward: an entry moves to an index at most its own,
        // and every lane has read its group's entry before any lane writes
        const int e = 64 * g + lane;
        const uint64_t en = e < cnt[side] ? wbuf[e] : 0ull;
        const bool keep = e < cnt[side] && __uint_as_float((uint32_t)en) >= th;
        const uint64_t m = __ballot(keep);
        const int at = n2 + (int)__builtin_amdgcn_mbcnt_hi(
            (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
        if (keep) wbuf[at] = en;
        n2 += __popcll(m);
      }
      uint64_t *lst = reinterpret_cast<uint64_t *>(sh.stage[side][wave]);
      if (n2 > 64) {
        const uint64_t k = wave_best64(lds<const uint64_t>(wbuf), n2);
        lst[lane] = make_entry(key_value(k), key_id(k));
        n2 = 64;
      } else if (lane < n2) {
        lst[lane] = wbuf[lane];
      }
      if (lane == 0) sh.lcount[side][wave] = n2;
    }
  }
  if constexpr (TOPK) {
      // locate: each side's argmax is the lowest id holding its maximum in
      // the round where the maximum last rose (ia, ib hold that round, kNoId
      // while a side has seen only -inf): that round's vectors are read again
      // -- as the loop read them, ids past hi as -inf -- and the lowest
      // element equal to the maximum is taken (one bit per element, then the
      // lowest set bit).  Only lanes that hold the wave's maximum can supply
      // the merged argmax, so only they read (a lane's read fetches a whole
      // cache line, which all 64 lanes would pay for); the others drop their
      // id, which the merge never takes from a smaller maximum.
    auto locate = [&](const T *rowp, int rr, float m) -> int {
      static_assert(U * VEC <= 32, "one bit per element of a round");
      const int id0 = (int)lo + rr * kRound + tofs;
      uint32_t bits = 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const Raw c = load_raw<T, VEC, ALIGNED>(rowp, (int64_t)id0 + u * kStride, hi);
#pragma unroll
        for (int j = 0; j < VEC; ++j) bits |= (elem(c, j) == m ? 1u : 0u) << (u * VEC + j);
      }
      const int k = __builtin_ctz(bits);
      return id0 + (k / VEC) * kStride + (k % VEC);
    };
    float wa = ma, wb = mb;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      wa = fmaxf(wa, __shfl_xor(wa, o));
      if (TWO) wb = fmaxf(wb, __shfl_xor(wb, o));
    }
    if (ia != kNoId) ia = ma == wa ? locate(ra, ia, ma) : kNoId;
    if (TWO && ib != kNoId) ib = mb == wb ? locate(rb, ib, mb) : kNoId;
  }
  {   // fold_offsets: back to sums against ref(ma), ref(mb) and t in nats.
      // The exact product ref(m) L2E is o + r (r = fma(ref, L2E, -o), exact
      // and below half an ulp of o): every weight taken against o is 2^r too
      // large, and e_a - e_b carries r_a - r_b besides L2E times the
      // difference of the shifted logits.
    const float oa = ref_of(ma) * kL2E, ob = ref_of(mb) * kL2E;
    const float ra = fmaf(ref_of(ma), kL2E, -oa), rb = fmaf(ref_of(mb), kL2E, -ob);
    const float ga = exp2_fast(-ra);
    sa *= ga;
    sb *= exp2_fast(-rb);
    if (TWO && sa != 0.f) t = fmaf(t, ga, -(ra - rb) * sa) / kL2E;
  }
  RowState s;
  s.ma = ma; s.sa = sa; s.t = t; s.mb = mb; s.sb = sb; s.ia = ia; s.ib = ib;
  s = wave_merge(s);
  if (lane == 0) waves[wave] = s;

  // After a block barrier the closing work is spread over the waves: with
  // top-k, wave s < NS gathers side s's four lists and selects their 64 best
  // while the next wave merges the four waves' row states (in wave order);
  // without, wave 0 merges.  (A wave that left early would free nothing: the
  // block's LDS stays allocated until its last wave ends.)
  __syncthreads();
  if (wave == (TOPK ? NS : 0)) {
    if (lane == 0) {
      RowState r = waves[0];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) r = merge(r, waves[w]);
      part[row * splits + split] = r;
    }
  }
  if constexpr (TOPK) {
    if (wave < NS) {
      const int side = wave;
      uint64_t *scr = sh.buf[side][wave];   // this wave's own buffer, free now
      int nt = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const int c = sh.lcount[side][w];
        if (lane < c) scr[nt + lane] = reinterpret_cast<const uint64_t *>(sh.stage[side][w])[lane];
        nt += c;
      }
      const uint64_t k = wave_best64(lds<const uint64_t>(scr), nt);
      topk_keys[((row * splits + split) * 2 + side) * 64 + lane] = k;
    }
  }
}

__device__ __forceinline__ RowStateD shfl_xor_d(const RowStateD &s, int m) {
  RowStateD o;
  o.ma = __shfl_xor(s.ma, m); o.mb = __shfl_xor(s.mb, m);
  o.sa = __shfl_xor(s.sa, m); o.t = __shfl_xor(s.t, m); o.sb = __shfl_xor(s.sb, m);
  o.ia = __shfl_xor(s.ia, m); o.ib = __shfl_xor(s.ib, m);
  return o;
}

// One group of 2^lg lanes per row (2^lg >= splits, a divisor of the wave):
// lane k loads split k's state (the empty state past the last split), the
// group merges them in f64 by a butterfly in split order (the lower split
// always first, so every lane computes the same bits), and lane 0 finishes
// the row.  The target logits are loaded first, so that their latency
// overlaps the merge.
template <typename T>
__global__ __launch_bounds__(256) void finalize_rows_kernel(
    const RowState *__restrict__ part, int splits, int lg, int64_t n, const T *__restrict__ ref,
    const T *__restrict__ cand, int64_t ld_ref, int64_t ld_cand, int64_t v,
    const int32_t *__restrict__ target, RowsOut out, double *__restrict__ lse_d /*[2][n]*/,
    float *__restrict__ target_lp) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid >> lg;
  const int k = (int)(gid & ((1 << lg) - 1));
  const bool live = row < n;
  bool tok = false;
  float za = 0.f, zb = 0.f;
  if (live && k == 0 && target) {
    const int32_t tg = target[row];
    tok = tg >= 0 && (int64_t)tg < v;
    if (tok) {
      za = to_f32(ref[row * ld_ref + tg]);
      zb = to_f32(cand[row * ld_cand + tg]);
    }
  }
  RowStateD s = live && k < splits ? to_d(part[row * splits + k]) : empty_state_d();
  for (int m = 1; m < (1 << lg); m <<= 1) {
    const RowStateD o = shfl_xor_d(s, m);
    s = (k & m) ? merge_d(o, s) : merge_d(s, o);
  }
  if (!live || k != 0) return;
  double la, lb;
  const RowResult r = finish_d(s, &la, &lb);
  if (lse_d) { lse_d[row] = la; lse_d[n + row] = lb; }
  if (out.kl) out.kl[row] = r.kl;
  if (out.lse_ref) out.lse_ref[row] = r.lse_a;
  if (out.lse_cand) out.lse_cand[row] = r.lse_b;
  if (out.argmax_ref) out.argmax_ref[row] = r.ia;
  if (out.argmax_cand) out.argmax_cand[row] = r.ib;
  if (target) {
    const float nan = __builtin_nanf("");
    if (out.nll_ref) out.nll_ref[row] = tok ? (float)(la - (double)za) : nan;
    if (out.nll_cand) out.nll_cand[row] = tok ? (float)(lb - (double)zb) : nan;
    if (target_lp) target_lp[row] = tok ? (float)((double)za - la) : nan;
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

// Without top-k only (both sides).
template <typename T, int VEC, int U>
hipError_t launch_partial_plain(const LogitsArgs &a, RowState *part) {
  if (a.aligned) return launch_partial_t<T, VEC, U, true, true, false>(a, part, nullptr);
  return launch_partial_t<T, VEC, U, false, true, false>(a, part, nullptr);
}

static_assert(kMaxSplits <= 64, "a row's group of finalize lanes fits in one wave");

template <typename T>
hipError_t launch_finalize(const LogitsArgs &a, const RowState *part, double *lse_d,
                           float *target_lp) {
  int lg = 0;
  while ((1 << lg) < a.splits) ++lg;   // splits <= kMaxSplits = 64: a group fits a wave
  const int64_t threads = a.n << lg;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL((finalize_rows_kernel<T>), dim3(blocks), dim3(256), 0, a.stream, part,
                     a.splits, lg, a.n, (const T *)a.ref, (const T *)a.cand, a.ld_ref, a.ld_cand,
                     a.v, a.target, a.out, lse_d, target_lp);
  return hipGetLastError();
}

}  // namespace

int logits_vec_elems(int dtype) { return dtype == 0 ? Vec<float>::N : Vec<uint16_t>::N; }

hipError_t launch_logits_state(const LogitsArgs &a, RowState *part, uint64_t *topk_keys) {
  if (a.dtype == 0) return launch_partial<float, 4, 4>(a, part, topk_keys);
  // bf16 with top-k: one vector per side and round, so that the kernel fits four blocks per
  // CU (registers and LDS); measured 3-4 % faster than two
  if (topk_keys || !a.two) return launch_partial<uint16_t, 8, 1>(a, part, topk_keys);
  return launch_partial_plain<uint16_t, 8, 2>(a, part);
}

hipError_t launch_logits_finalize(const LogitsArgs &a, const RowState *part, double *lse_d,
                                  float *target_lp) {
  if (a.dtype == 0) return launch_finalize<float>(a, part, lse_d, target_lp);
  return launch_finalize<uint16_t>(a, part, lse_d, target_lp);
}

}  // namespace kld

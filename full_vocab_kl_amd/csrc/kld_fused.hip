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
// Grid: one block per (vocab tile, position tile).  Position tiles are
// grouped 16 at a time and the groups run one after the other, so the hidden
// states in use stay cache-resident at any number of positions.  Within a
// group, consecutive hardware block ids are dealt round-robin over the 8
// XCDs; the block id is remapped so that each XCD receives a contiguous range
// of tiles, position tiles fastest, so all position tiles of one head tile run
// together on one XCD and the head tile is fetched from HBM about once per
// group into that XCD's L2.
#include <type_traits>

#include "kld.h"
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

// f32 max / median of three without operand canonicalisation (fmaxf in IEEE
// mode quiets signalling NaNs first; values produced by MFMA never are).
__device__ __forceinline__ float vmax2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float vmed3(float a, float b, float c) {
  float r;
  asm("v_med3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

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

// Position tiles are taken in groups of kGroupTiles: every vocabulary tile of
// one group runs before the next group starts (blocks are dispatched in id
// order), so the hidden states the resident blocks read -- one group, 16 x
// 256 rows x d -- stay in the 256 MB cache however many positions the call
// scores, and the head streams once per group.  Within a group the XCD-aware
// order above applies.  kGroupTiles is a multiple of 8, so every group starts
// on XCD 0.  Returns (vocabulary tile, position tile).
constexpr int kGroupTiles = 16;
static_assert(kGroupTiles % kXcds == 0, "groups start on XCD 0");
__device__ __forceinline__ int2 tile_of_block(int b, int npt, int nvt) {
  const int per = nvt * kGroupTiles;           // blocks of a full group
  const int ngroups = (npt + kGroupTiles - 1) / kGroupTiles;
  int g = b / per;
  if (g > ngroups - 1) g = ngroups - 1;
  const int gp = min(kGroupTiles, npt - g * kGroupTiles);   // position tiles of group g
  const int L = logical_block(b - g * per, nvt * gp);
  return make_int2(L / gp, g * kGroupTiles + L % gp);
}

// Buffer resource over `bytes` bytes at p (raw addressing, no stride): loads
// at offsets past the range return zero and touch no memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
  const int num = bytes <= 0 ? 0 : (bytes >= 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, num, 0x00020000);
}

// Online log-sum-exp state of one candidate column over part of a tile:
// maximum m, s = sum e^(z - m) and u = the same sum over the unlisted ids.
struct Lsu {
  float m, s, u;
};
__device__ __forceinline__ Lsu lsu_merge(const Lsu &a, const Lsu &b) {
  const float m = fmaxf(a.m, b.m);
  const float fa = a.m == kNegInf ? 0.f : exp2_fast((a.m - ref_of(m)) * kL2E);
  const float fb = b.m == kNegInf ? 0.f : exp2_fast((b.m - ref_of(m)) * kL2E);
  return Lsu{m, fmaf(a.s, fa, b.s * fb), fmaf(a.u, fa, b.u * fb)};
}

struct SparseIn;
template <typename Acc>
__device__ __forceinline__ void sparse_epilogue(Acc &acc, const struct SparseIn &sp, float *part,
                                                void *smem, int64_t v, int64_t v0, int vt,
                                                int64_t p0, int64_t n, int64_t nvt, int64_t npad,
                                                int wv, int wp, int fr, int fh, bool vtail);

// Epilogue modes: KL state of a (reference, candidate) pair per position,
// the same with top-64 candidates, or one-sided scoring of candidate
// positions against stored sparse records (256 positions per block: the two
// 128-row halves of the hidden unit are two position blocks of the
// candidate).
enum { kModeKl = 0, kModeTopk = 1, kModeSparse = 2 };

// Listed ids of a position, sorted by id, for the sparse mode: sid[pos][e]
// the id, sslot[pos][e] its slot in the record (bit 15: a repeat of the
// previous id), rp[pos][t] the first entry with id >= 256 t.
struct SparseIn {
  const int32_t *sid;
  const uint16_t *sslot;
  const uint16_t *rp;
  float *zl;   // [n][512] listed logits out
};

template <int MODE>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(1, 1)))
void fused_head_kernel(const uint16_t *__restrict__ W, const uint16_t *__restrict__ Hr,
                       const uint16_t *__restrict__ Hc, int64_t v, int64_t d, int64_t n, int npt,
                       int64_t npad, int64_t nvt, float *__restrict__ part,
                       uint64_t *__restrict__ ckeys, float *__restrict__ resid,
                       uint64_t *__restrict__ rinfo, uint64_t *__restrict__ tkeys, SparseIn sp) {
  constexpr bool TOPK = MODE == kModeTopk;
  constexpr bool SPARSE = MODE == kModeSparse;
  constexpr int PB = SPARSE ? 2 * BP : BP;   // positions per block
  // The five ring slots (160 KB, the whole LDS) are separate LDS objects, so
  // that the compiler knows the loads into one slot never touch the fragment
  // reads of another and can interleave the two (with one array it kept
  // every read ahead of every later load).
  __shared__ u32x4 lds0[UCHUNKS], lds1[UCHUNKS], lds2[UCHUNKS], lds3[UCHUNKS], lds4[UCHUNKS];
  auto slot_ptr = [&](int slot) -> u32x4 * {
    return slot == 0 ? lds0 : slot == 1 ? lds1 : slot == 2 ? lds2 : slot == 3 ? lds3 : lds4;
  };
  static_assert(sizeof(u32x4) * UCHUNKS * NSLOT == kFusedLds, "ring = all of LDS");
  u32x4 *const smem = lds0;   // epilogue exchange area (after the loop)

  const int2 tile = tile_of_block((int)blockIdx.x, npt, (int)nvt);
  const int vt = tile.x, pt = tile.y;
  const int64_t v0 = (int64_t)vt * BV, p0 = (int64_t)pt * PB;
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
    const int q = SPARSE ? r : (r & (BP - 1));
    const int64_t rh = p0 + q < n ? q : n - 1 - p0;
    vo_w[j] = (uint32_t)(rw * d * 2 + cl * 16);
    vo_h[j] = (uint32_t)(rh * d * 2 + cl * 16);
  }
  const uint16_t *wbase = W + v0 * d;
  const uint16_t *hbase = (SPARSE || wave_u >= 2 ? Hc : Hr) + p0 * d;
  const int64_t wbytes = (v - v0) * d * 2, hbytes = (n - p0) * d * 2;
  const int KT = (int)((d + BK - 1) / BK);
  const bool ktail = (d % BK) != 0;

  // Issue loads j0 .. j0 + cnt - 1 of the head (H = false) or hidden unit of
  // stage st into ring slot `slot`.  The resource starts at the stage's first
  // element, so offsets past the end of the operand -- the K tail of its last
  // row, and stages past the last one -- fetch nothing.  (Byte counts are
  // clamped to 2^31 - 1, far beyond the 256 rows a block reads.)
  const uint32_t wb32 = (uint32_t)(wbytes < 0x7fffffff ? wbytes : 0x7fffffff);
  const uint32_t hb32 = (uint32_t)(hbytes < 0x7fffffff ? hbytes : 0x7fffffff);
  auto issue = [&](int st, bool H, int j0, int cnt, int slot) {
    const int rem = (int)(H ? hb32 : wb32) - st * (BK * 2);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>((H ? hbase : wbase) + (int64_t)st * BK), (short)0,
        __builtin_amdgcn_readfirstlane(rem > 0 ? rem : 0), 0x00020000);
    u32x4 *dst = slot_ptr(slot) + wave_u * (UCHUNKS / 4);
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
  // Per-lane byte offsets of the fragment reads within a slot.  A row
  // wv*128 + vs*32 + fr and B row sd*128 + wp*64 + pg*32 + fr share their
  // swizzle key with the row 64 (resp. 128) below, so the lane offset depends
  // only on (K step, vs & 1) or (K step, pg); the rest is a constant.
  uint32_t offA[4][2], offB[4][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int ra = wv * 128 + x * 32 + fr, rb = wp * 64 + x * 32 + fr;
      offA[ks][x] = (uint32_t)(ra * CH + ((2 * ks + fh) ^ swz_key(ra))) * 16;
      offB[ks][x] = (uint32_t)(rb * CH + ((2 * ks + fh) ^ swz_key(rb))) * 16;
    }
  // The LDS read offset field reaches 64 KB past the address register, so
  // every lane offset is also kept biased by 64 KB and 128 KB (opaque to the
  // compiler, which would otherwise fold the bias back into a VALU op per
  // read): a read of slot k uses the copy biased by 64 KB * (k / 2), and the
  // rest of the slot base (slots are laid out in order, 32 KB apart) is an
  // immediate.  Any other layout only costs the VALU ops back.
  uint32_t offA1[4][2], offB1[4][2], offA2[4][2], offB2[4][2];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      offA1[ks][x] = offA[ks][x] + 65536u;
      offB1[ks][x] = offB[ks][x] + 65536u;
      offA2[ks][x] = offA[ks][x] + 131072u;
      offB2[ks][x] = offB[ks][x] + 131072u;
      asm volatile("" : "+v"(offA1[ks][x]), "+v"(offB1[ks][x]), "+v"(offA2[ks][x]), "+v"(offB2[ks][x]));
    }
  auto lane_off = [&](bool a, int slot, int ks, int x) -> uint32_t {
    const int g = slot >> 1;
    return a ? (g == 0 ? offA[ks][x] : g == 1 ? offA1[ks][x] - 65536u : offA2[ks][x] - 131072u)
             : (g == 0 ? offB[ks][x] : g == 1 ? offB1[ks][x] - 65536u : offB2[ks][x] - 131072u);
  };
  auto load_frags = [&](int slot_w, int slot_h, int ks, Frags &f) {
    const char *sw = reinterpret_cast<const char *>(slot_ptr(slot_w));
    const char *sh = reinterpret_cast<const char *>(slot_ptr(slot_h));
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
      for (int sd = 0; sd < 2; ++sd)
        f.b[pg][sd] = *reinterpret_cast<const bf16x8 *>(sh + lane_off(false, slot_h, ks, pg) + sd * (BP * CH * 16));
#pragma unroll
    for (int vs = 0; vs < 4; ++vs)
      f.a[vs] = *reinterpret_cast<const bf16x8 *>(sw + lane_off(true, slot_w, ks, vs & 1) + (vs >> 1) * (64 * CH * 16));
  };
  // 16 MFMAs per K step.  Consecutive MFMAs share an operand: the two sides
  // of one position group run back to back, and the (pg, sd) order reverses
  // for odd vs, so only one operand changes at each step (slightly faster
  // under the power limit this loop runs at than restarting at pg 0).
  auto mfma = [&](const Frags &f) {
#pragma unroll
    for (int vs = 0; vs < 4; ++vs)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int qq = (vs & 1) ? 3 - q : q;
        const int pg = qq >> 1, sd = qq & 1;
        acc[vs][pg][sd] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[vs], f.b[pg][sd], acc[vs][pg][sd], 0, 0, 0);
      }
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
  // 16 MFMAs interleaved with 8 LDS fragment reads and 4 global loads; the
  // scheduling fence after each K step keeps the pattern from being merged
  // across the steps of the unrolled stages.
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
    __builtin_amdgcn_sched_barrier(0);   // keep each K step's mix within the step
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
  issue(0, false, 0, ULOADS, 0);
  issue(0, true, 0, ULOADS, 1);
  issue(1, false, 0, ULOADS, 2);
  issue(1, true, 0, ULOADS, 3);
  wait_vmcnt<2 * ULOADS>();   // stage 0 has landed
  block_barrier();
  load_frags(0, 1, 0, f0);
  load_frags(0, 1, 1, f1);
  // One stage; R = s % 5 is a compile-time constant in the unrolled loop, so
  // every slot index (and LDS offset) below is one too.
  auto stage = [&](int s, auto R) {
    constexpr int r = decltype(R)::value;
    constexpr int sw = (2 * r) % NSLOT, sh = (2 * r + 1) % NSLOT;           // stage s
    constexpr int nw = (2 * r + 2) % NSLOT, nh = (2 * r + 3) % NSLOT;       // stage s + 1
    constexpr int lw = (2 * r + 4) % NSLOT, lh = (2 * r + 5) % NSLOT;       // stage s + 2
    load_frags(sw, sh, 2, f2);
    issue(s + 2, false, 0, ULOADS / 2, lw);
    mfma(f0);
    interleave();
    load_frags(sw, sh, 3, f3);
    issue(s + 2, false, ULOADS / 2, ULOADS / 2, lw);
    mfma(f1);
    interleave();
    wait_vmcnt<ULOADS>();
    wait_lgkm0();
    block_barrier();
    load_frags(nw, nh, 0, f0);
    issue(s + 2, true, 0, ULOADS / 2, lh);
    mfma(f2);
    interleave();
    load_frags(nw, nh, 1, f1);
    issue(s + 2, true, ULOADS / 2, ULOADS / 2, lh);
    mfma(f3);
    interleave();
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  int s = 0;
  for (; s + NSLOT < KT; s += NSLOT) {
    stage(s, I0{});
    stage(s + 1, I1{});
    stage(s + 2, I2{});
    stage(s + 3, I3{});
    stage(s + 4, I4{});
  }
  if (s + 1 < KT) { stage(s, I0{}); ++s; }
  if (s + 1 < KT) { stage(s, I1{}); ++s; }
  if (s + 1 < KT) { stage(s, I2{}); ++s; }
  if (s + 1 < KT) { stage(s, I3{}); ++s; }
  {   // last stage, s = KT - 1
    const int sw = (2 * s) % NSLOT, sh = (2 * s + 1) % NSLOT;
    load_frags(sw, sh, 2, f2);
    load_frags(sw, sh, 3, f3);
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
  if constexpr (SPARSE) {
    sparse_epilogue(acc, sp, part, smem, v, v0, vt, p0, n, nvt, npad, wv, wp, fr, fh, vtail);
    return;
  }
  RowState *xch = reinterpret_cast<RowState *>(smem);          // [2 pos waves][2 pg][32]
  float *rx = reinterpret_cast<float *>(xch + 2 * 2 * 32);       // [2 sides][2][2][32]
  float *qx = rx + 2 * 2 * 2 * 32;                                 // same shape
  int *gx = reinterpret_cast<int *>(qx + 2 * 2 * 2 * 32);          // same shape
#pragma unroll
  for (int pg = 0; pg < 2; ++pg) {
    if (vtail) {
      const int lim = (int)(v - v0) - (wv * 128 + 4 * fh);   // lane offsets >= lim are past v
#pragma unroll
      for (int vs = 0; vs < 4; ++vs)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * vs + 8 * (i >> 2) + (i & 3) >= lim) {
            acc[vs][pg][0][i] = kNegInf;
            acc[vs][pg][1][i] = kNegInf;
          }
    }
    // Group by group (the 16 ids of (lane, vs), ascending in vs and in id):
    // per side the maximum m1 with its lowest id and, with top-k, the second
    // largest value m2; the group's partial state relative to its own maxima,
    // merged into the lane's state in id order.  With top-k, every group
    // maximum is written as a candidate key at once, and per side the two
    // largest m2 are kept with the group of the largest.
    const int64_t pos = p0 + wp * 64 + pg * 32 + fr;
    float a1[2] = {kNegInf, kNegInf}, a2[2] = {kNegInf, kNegInf};
    int i1[2] = {0, 0};
    RowState st = empty_state();
#pragma unroll
    for (int vs = 0; vs < 4; ++vs) {
      // the group's 2 x 16 values, pinned in VGPRs here so that only one
      // group is held outside the accumulators at a time
      float xs[2][16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        xs[0][i] = acc[vs][pg][0][i];
        xs[1][i] = acc[vs][pg][1][i];
        asm volatile("" : "+v"(xs[0][i]), "+v"(xs[1][i]));
      }
      // Group maxima by v_max3 (the accumulators never hold signalling NaNs,
      // so the canonicalising moves that fmaxf implies are not needed); with
      // top-k the second value by v_med3 (m1 >= m2: med3(m1, m2, x) is the
      // new second largest).  Then the lowest id of each side's maximum, the
      // two sides' compare chains interleaved.
      float m1[2], m2[2];
#pragma unroll
      for (int sd = 0; sd < 2; ++sd) {
        const float *x = xs[sd];
        if constexpr (TOPK) {
          float x1 = kNegInf, x2 = kNegInf;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            x2 = vmed3(x1, x2, x[i]);
            x1 = vmax2(x1, x[i]);
          }
          m1[sd] = x1; m2[sd] = x2;
        } else {
          const float a = vmax3(x[0], x[1], x[2]), b = vmax3(x[3], x[4], x[5]);
          const float c = vmax3(x[6], x[7], x[8]), d = vmax3(x[9], x[10], x[11]);
          const float e = vmax3(x[12], x[13], x[14]);
          m1[sd] = vmax2(vmax3(a, b, c), vmax3(d, e, x[15]));
          m2[sd] = kNegInf;
        }
      }
      int k[2] = {kNoId, kNoId};
#pragma unroll
      for (int i = 15; i >= 0; --i)
#pragma unroll
        for (int sd = 0; sd < 2; ++sd)
          if (xs[sd][i] == m1[sd]) k[sd] = 32 * vs + 8 * (i >> 2) + (i & 3);
      int id[2];
#pragma unroll
      for (int sd = 0; sd < 2; ++sd) {
        const float x1 = m1[sd], x2 = m2[sd];
        id[sd] = x1 == kNegInf ? kNoId : (int)(vb + k[sd]);
        if constexpr (TOPK) {   // (positions n .. npad - 1 are padding: no branch needed)
          ckeys[(((int64_t)sd * nvt + vt) * npad + pos) * 16 + (wv * 2 + fh) * 4 + vs] =
              x1 == kNegInf ? 0ull : topk_key(x1, id[sd]);
          if (x2 > a1[sd]) { a2[sd] = a1[sd]; a1[sd] = x2; i1[sd] = vs; }
          else { a2[sd] = fmaxf(a2[sd], x2); }
        }
      }
      const float ra = ref_of(m1[0]), rb = ref_of(m1[1]);
      float sa = 0.f, sb = 0.f, t = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float x = xs[0][i] - ra, y = xs[1][i] - rb;
        const float w = exp2_fast(x * kL2E);
        sa += w;
        t = fmaf(w, fmaxf(x - y, -kFltMax), t);
        sb += exp2_fast(y * kL2E);
      }
      // the group's sums are complete here, before the next group is read
      asm volatile("" : "+v"(sa), "+v"(sb), "+v"(t));
      RowState g;
      g.ma = m1[0]; g.sa = sa; g.t = t; g.mb = m1[1]; g.sb = sb; g.ia = id[0]; g.ib = id[1];
      st = vs == 0 ? g : merge(st, g);
    }
    // lanes l and l ^ 32 hold the same position (interleaved ids)
    const RowState o = shfl_xor_state(st, 32);
    st = fh == 0 ? merge(st, o) : merge(o, st);
    // Per side: the largest group second value r2 (the tile residual), the
    // group g2 that holds it (lowest group index among equals) and the
    // largest second value q2 of the other groups.
    float r2[2] = {kNegInf, kNegInf}, q2[2] = {kNegInf, kNegInf};
    int g2[2] = {0, 0};
    if constexpr (TOPK) {
#pragma unroll
      for (int sd = 0; sd < 2; ++sd) {
        const int ga = wv * 8 + fh * 4 + i1[sd];
        const float b1 = __shfl_xor(a1[sd], 32), b2 = __shfl_xor(a2[sd], 32);
        const int gb = __shfl_xor(ga, 32);
        const bool aw = a1[sd] > b1 || (a1[sd] == b1 && ga < gb);
        r2[sd] = aw ? a1[sd] : b1;
        g2[sd] = aw ? ga : gb;
        q2[sd] = aw ? fmaxf(a2[sd], b1) : fmaxf(b2, a1[sd]);
      }
    }
    if (wv == 1 && fh == 0) {
      xch[(wp * 2 + pg) * 32 + fr] = st;
      if (TOPK) {
#pragma unroll
        for (int sd = 0; sd < 2; ++sd) {
          rx[((sd * 2 + wp) * 2 + pg) * 32 + fr] = r2[sd];
          qx[((sd * 2 + wp) * 2 + pg) * 32 + fr] = q2[sd];
          gx[((sd * 2 + wp) * 2 + pg) * 32 + fr] = g2[sd];
        }
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
#pragma unroll
        for (int sd = 0; sd < 2; ++sd) {
          const int xi = ((sd * 2 + wp) * 2 + pg) * 32 + fr;
          const float b1 = rx[xi], b2 = qx[xi];
          const int gb = gx[xi];
          const bool aw = r2[sd] > b1 || (r2[sd] == b1 && g2[sd] < gb);
          const int64_t ti = ((int64_t)sd * nvt + vt) * npad + pos;
          resid[ti] = aw ? r2[sd] : b1;
          rinfo[ti] = (uint64_t)__float_as_uint(aw ? fmaxf(q2[sd], b1) : fmaxf(b2, r2[sd])) |
                      ((uint64_t)(uint32_t)(aw ? g2[sd] : gb) << 32);
        }
        // the tile's largest candidate key per side (the maximum and its
        // lowest id), position-major for the selection
        tkeys[((int64_t)0 * npad + pos) * nvt + vt] = st.ma == kNegInf ? 0ull : topk_key(st.ma, st.ia);
        tkeys[((int64_t)1 * npad + pos) * nvt + vt] = st.mb == kNegInf ? 0ull : topk_key(st.mb, st.ib);
      }
    }
    __syncthreads();
  }
}

// Sparse-mode epilogue.  Column (pg, sd) of a lane is candidate position
// p0 + 128 sd + 64 wp + 32 pg + (lane & 31); the lane holds its ids
// vb + 32 vs + 8 (i / 4) + (i % 4).  For each column: the record's listed ids
// that fall in this lane's part of the tile are marked in a 64-bit mask (bit
// 16 vs + i) and their logits written to zl at their record slots; then the
// lane's maximum, its sum and its sum over unmarked ids, merged with lane
// l ^ 32 and with the other vocabulary wave, give the tile's partial state
// (planes m, s, u of part[3][nvt][npad]).
template <typename Acc>
__device__ __forceinline__ void sparse_epilogue(Acc &acc, const SparseIn &sp, float *part,
                                                void *smem, int64_t v, int64_t v0, int vt,
                                                int64_t p0, int64_t n, int64_t nvt, int64_t npad,
                                                int wv, int wp, int fr, int fh, bool vtail) {
  Lsu *xch = reinterpret_cast<Lsu *>(smem);   // [2 pos waves][2 sd][32]
  const int64_t plane = nvt * npad;
#pragma unroll
  for (int pg = 0; pg < 2; ++pg) {
    if (vtail) {
      const int lim = (int)(v - v0) - (wv * 128 + 4 * fh);
#pragma unroll
      for (int vs = 0; vs < 4; ++vs)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * vs + 8 * (i >> 2) + (i & 3) >= lim) {
            acc[vs][pg][0][i] = kNegInf;
            acc[vs][pg][1][i] = kNegInf;
          }
    }
    Lsu st[2];
#pragma unroll
    for (int sd = 0; sd < 2; ++sd) {
      const int64_t pos = p0 + sd * BP + wp * 64 + pg * 32 + fr;
      uint64_t lm = 0;
      if (pos < n) {
        const uint16_t *rr = sp.rp + pos * (nvt + 1) + vt;
        const int e0 = rr[0], e1 = rr[1];
        for (int e = e0; e < e1; ++e) {
          const uint16_t sl = sp.sslot[pos * KLD_GOLDEN_TOPK + e];
          const int idl = sp.sid[pos * KLD_GOLDEN_TOPK + e] - (int)v0;
          if ((sl & 0x8000) || (idl >> 7) != wv || ((idl >> 2) & 1) != fh) continue;
          const int k = ((idl >> 5) & 3) * 16 + ((idl >> 3) & 3) * 4 + (idl & 3);
          lm |= 1ull << k;
          float z = 0.f;
#pragma unroll
          for (int vs = 0; vs < 4; ++vs)
#pragma unroll
            for (int i = 0; i < 16; ++i) z = k == vs * 16 + i ? acc[vs][pg][sd][i] : z;
          sp.zl[pos * KLD_GOLDEN_TOPK + (sl & 0x1ff)] = z;
        }
      }
      float m = kNegInf;
#pragma unroll
      for (int vs = 0; vs < 4; ++vs)
#pragma unroll
        for (int i = 0; i < 16; i += 2) m = vmax3(m, acc[vs][pg][sd][i], acc[vs][pg][sd][i + 1]);
      const float r = ref_of(m);
      float ssum = 0.f, usum = 0.f;
#pragma unroll
      for (int vs = 0; vs < 4; ++vs)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float w = exp2_fast((acc[vs][pg][sd][i] - r) * kL2E);
          ssum += w;
          usum += ((lm >> (vs * 16 + i)) & 1ull) ? 0.f : w;
        }
      st[sd] = Lsu{m, ssum, usum};
      // lanes l and l ^ 32 hold the same position (interleaved ids)
      const Lsu o{__shfl_xor(st[sd].m, 32), __shfl_xor(st[sd].s, 32), __shfl_xor(st[sd].u, 32)};
      st[sd] = fh == 0 ? lsu_merge(st[sd], o) : lsu_merge(o, st[sd]);
    }
    if (wv == 1 && fh == 0) {
#pragma unroll
      for (int sd = 0; sd < 2; ++sd) xch[(wp * 2 + sd) * 32 + fr] = st[sd];
    }
    __syncthreads();
    if (wv == 0 && fh == 0) {
#pragma unroll
      for (int sd = 0; sd < 2; ++sd) {
        const int64_t pos = p0 + sd * BP + wp * 64 + pg * 32 + fr;
        if (pos < n) {
          const Lsu t = lsu_merge(st[sd], xch[(wp * 2 + sd) * 32 + fr]);
          float *q = part + (int64_t)vt * npad + pos;
          q[0] = t.m;
          q[plane] = t.s;
          q[2 * plane] = t.u;
        }
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

// Merge the partial states of each position over the vocabulary tiles.
// Block = 8 positions x 32 groups; group g takes tiles g, g + 32, ...  Pass 1:
// the maxima (and lowest-id argmax) of both sides over all tiles.  Pass 2:
// every tile's sums moved to those maxima (one f64 exp per side and tile, no
// running rebase) and added in f64; the 32 group results are combined in a
// fixed order through LDS.  (Many groups and small blocks: a window must
// spread over every CU.)
constexpr int FP = 8, FG = 32;
__global__ __launch_bounds__(FP * FG) void fused_finalize_kernel(
    const float *__restrict__ part, int64_t nvt, int64_t npad, int64_t n,
    const float *__restrict__ zt, const int32_t *__restrict__ target, RowsOut out,
    double *__restrict__ lse_d) {
  struct Mx { float ma, mb; int ia, ib; };
  struct Sm { double sa, t, sb; };
  __shared__ Mx rm[FG][FP];
  __shared__ Sm rs[FG][FP];
  const int pl = threadIdx.x % FP, g = threadIdx.x / FP;
  const int64_t pos = (int64_t)blockIdx.x * FP + pl;
  const int64_t plane = nvt * npad;
  const bool live = pos < n;
  // pass 1: maxima
  Mx m = {kNegInf, kNegInf, kNoId, kNoId};
  if (live) {
    for (int64_t vt = g; vt < nvt; vt += FG) {
      const float *q = part + vt * npad + pos;
      const float xa = q[0], xb = q[3 * plane];
      const int ja = __float_as_int(q[5 * plane]), jb = __float_as_int(q[6 * plane]);
      if (beats(xa, ja, m.ma, m.ia)) { m.ma = xa; m.ia = ja; }
      if (beats(xb, jb, m.mb, m.ib)) { m.mb = xb; m.ib = jb; }
    }
  }
  rm[g][pl] = m;
  __syncthreads();
  m = rm[0][pl];
  for (int i = 1; i < FG; ++i) {
    const Mx o = rm[i][pl];
    if (beats(o.ma, o.ia, m.ma, m.ia)) { m.ma = o.ma; m.ia = o.ia; }
    if (beats(o.mb, o.ib, m.mb, m.ib)) { m.mb = o.mb; m.ib = o.ib; }
  }
  // pass 2: sums at the final offsets
  const double ra = (double)ref_of(m.ma), rb = (double)ref_of(m.mb);
  Sm sm = {0.0, 0.0, 0.0};
  if (live) {
    for (int64_t vt = g; vt < nvt; vt += FG) {
      const float *q = part + vt * npad + pos;
      const float xa = q[0], xsa = q[plane], xt = q[2 * plane], xb = q[3 * plane], xsb = q[4 * plane];
      const double oa = (double)ref_of(xa), ob = (double)ref_of(xb);
      const double fa = xa == kNegInf ? 0.0 : exp(oa - ra), fb = xb == kNegInf ? 0.0 : exp(ob - rb);
      const double tt = xsa == 0.f ? (double)xt : fma((double)xsa, (rb - ob) - (ra - oa), (double)xt);
      sm.sa += (double)xsa * fa;
      sm.t += tt * fa;
      sm.sb += (double)xsb * fb;
    }
  }
  rs[g][pl] = sm;
  __syncthreads();
  if (g == 0 && live) {
    RowStateD s;
    s.ma = m.ma; s.mb = m.mb; s.ia = m.ia; s.ib = m.ib;
    s.sa = rs[0][pl].sa; s.t = rs[0][pl].t; s.sb = rs[0][pl].sb;
    for (int i = 1; i < FG; ++i) { s.sa += rs[i][pl].sa; s.t += rs[i][pl].t; s.sb += rs[i][pl].sb; }
    double la, lb;
    const RowResult r = finish_d(s, &la, &lb);
    if (lse_d) {
      lse_d[pos] = la;
      lse_d[n + pos] = lb;
    }
    out.kl[pos] = r.kl;
    if (out.lse_ref) out.lse_ref[pos] = r.lse_a;
    if (out.lse_cand) out.lse_cand[pos] = r.lse_b;
    if (out.argmax_ref) out.argmax_ref[pos] = r.ia;
    if (out.argmax_cand) out.argmax_cand[pos] = r.ib;
    if (target) {
      if (out.nll_ref) out.nll_ref[pos] = (float)(la - (double)zt[pos]);
      if (out.nll_cand) out.nll_cand[pos] = (float)(lb - (double)zt[n + pos]);
    }
  }
}

// Exact top-64 of one (position, side) from the fused kernel's candidates.
//
// Candidates: for every vocabulary tile, the maximum of each of its 16
// groups (key = value bits, then complemented id).  Every id that is not a
// candidate is <= its tile's residual (the largest second-largest value of
// the tile's groups).
//  A. Tile maxima (the largest of a tile's 16 keys) are cut to the 64
//     largest, in chunks through a sorted LDS buffer.  A candidate of any
//     other tile is below 64 larger tile maxima, so the top 64 candidates lie
//     in these 64 tiles: their 1024 keys are sorted and the first 64 kept.
//     T = the 64th key.
//  B. Any tile whose residual reaches T's value may hide an id that belongs
//     in the top 64 (or fewer than 64 candidates exist): its 256 logits are
//     recomputed here from W and h (f32 dot products), its old candidates
//     are dropped, and the running top 64 is re-cut.  Only the 64 tiles of A
//     can qualify: every other tile's residual is at most its maximum, which
//     is below T, or equal to T's value only with larger ids.  On generic
//     inputs no tile is flagged; degenerate inputs (exact ties across many
//     ids) only cost time.
//  C. Write ids and fp16 log-probs lp = z - lse.
constexpr int TK = 256;

__global__ __launch_bounds__(TK) void fused_topk_kernel(
    const uint64_t *__restrict__ ckeys, const float *__restrict__ resid,
    const uint64_t *__restrict__ rinfo, const uint64_t *__restrict__ tkeys, int64_t nvt,
    int64_t npad,
    int64_t n, const uint16_t *__restrict__ W, const uint16_t *__restrict__ Hr,
    const uint16_t *__restrict__ Hc, int64_t v, int64_t d, const double *__restrict__ lse_d,
    TopkOut out) {
  const int64_t pos = blockIdx.x >> 1;
  const int side = blockIdx.x & 1;
  int32_t *ids = side ? out.ids_cand : out.ids_ref;
  uint16_t *lp = side ? out.lp_cand : out.lp_ref;
  if ((!ids && !lp) || pos >= n) return;

  __shared__ uint64_t buf[64 + TK];
  __shared__ uint32_t hist[256];
  __shared__ __align__(8) uint32_t sh[6];
  __shared__ int tiles[64];
  __shared__ int sh_nflag;
  __shared__ int flagged[TK];

  const uint64_t *base = ckeys + ((int64_t)side * nvt * npad + pos) * 16;
  const int64_t tstride = npad * 16;
  const int tid = threadIdx.x;

  // ---- A1: the 64 largest tile maxima, in chunks of 3 TK tiles plus the
  // running 64 (buf[0..63]).
  const uint64_t *tk = tkeys + ((int64_t)side * npad + pos) * nvt;
  if (tid < 64) buf[tid] = 0ull;
  __syncthreads();
  for (int64_t c0 = 0; c0 < nvt; c0 += 3 * TK) {
    uint64_t k4[4];
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int64_t t = c0 + q * TK + tid;
      k4[q] = t < nvt ? tk[t] : 0ull;
    }
    k4[3] = tid < 64 ? buf[tid] : 0ull;
    __syncthreads();
    block_select64<4>(k4, buf, hist, sh);
  }
  // ---- A2: the 64 largest of those tiles' 16 candidates each
  if (tid < 64) tiles[tid] = buf[tid] == 0ull ? -1 : (int)((uint32_t)key_id(buf[tid]) / BV);
  __syncthreads();
  uint64_t T;
  {
    uint64_t k4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = q * TK + tid;
      const int t = tiles[i >> 4];
      k4[q] = t < 0 ? 0ull : base[(int64_t)t * tstride + (i & 15)];
    }
    T = block_select64<4>(k4, buf, hist, sh);
  }
  const float tval = key_value(T);

  // ---- B: recompute what may hide a missing id: when T is unset, every tile;
  // else, among the 64 tiles of A, each tile whose residual reaches T -- only
  // the group that holds the residual when no other group's second value
  // reaches T, else the whole tile.
  const uint16_t *h = (side ? Hc : Hr) + pos * d;
  const int64_t nscan = T == 0ull ? nvt : 64;
  for (int64_t r0 = 0; r0 < nscan; r0 += TK) {
    if (tid == 0) sh_nflag = 0;
    __syncthreads();
    const int64_t vt = T == 0ull ? r0 + tid : (tid < 64 ? tiles[tid] : -1);
    if (r0 + tid < nscan && vt >= 0) {
      const int64_t ti = ((int64_t)side * nvt + vt) * npad + pos;
      if (T == 0ull) {
        flagged[atomicAdd(&sh_nflag, 1)] = (int)vt;
      } else if (resid[ti] >= tval) {
        const uint64_t info = rinfo[ti];
        const int grp = __uint_as_float((uint32_t)info) < tval ? (int)(info >> 32) : -1;
        flagged[atomicAdd(&sh_nflag, 1)] = (int)vt | ((grp + 1) << 24);
      }
    }
    __syncthreads();
    const int nf = sh_nflag;
    for (int f = 0; f < nf; ++f) {
      const int64_t t0 = (int64_t)(flagged[f] & 0xffffff) * BV;   // the tile's first id
      const int grp = (flagged[f] >> 24) - 1;                     // -1: the whole tile
      // Offset in the tile of row q of group g: ids of group (wv, fh, vs) are
      // 128 wv + 4 fh + 32 vs + 8 (i / 4) + i % 4, i = 0..15.
      auto grp_off = [](int g, int q) {
        return (g >> 3) * 128 + ((g >> 2) & 1) * 4 + (g & 3) * 32 + 8 * (q >> 2) + (q & 3);
      };
      auto grp_of = [](int off) { return ((off >> 7) & 1) * 8 + ((off >> 2) & 1) * 4 + ((off >> 5) & 3); };
      // drop the recomputed ids' old candidates from the running top 64
      if (tid < 64) {
        const int64_t id = key_id(buf[tid]);
        if (buf[tid] != 0ull && id >= t0 && id < t0 + BV && (grp < 0 || grp_of((int)(id - t0)) == grp))
          buf[tid] = 0ull;
      }
      // the logits: wave w computes a quarter of the rows, four at a time;
      // lane l sums elements 8 l .. 8 l + 7 of every 512 in order, then the 64
      // lane sums are added in a fixed butterfly order.
      const int nrows = grp < 0 ? BV : 16;
      {
        const int wv = tid >> 6, ln = tid & 63;
        const int per = nrows / 4;
        for (int r = 0; r < per; r += 4) {
          float z4[4] = {0.f, 0.f, 0.f, 0.f};
          const uint16_t *w4[4];
          int64_t j4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int row = wv * per + r + q;
            j4[q] = t0 + (grp < 0 ? row : grp_off(grp, row));
            w4[q] = W + (j4[q] < v ? j4[q] : v - 1) * d;
          }
          for (int64_t e = (int64_t)ln * 8; e < d; e += 512) {
            const u32x4 qh = *reinterpret_cast<const u32x4 *>(h + e);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const u32x4 qw = *reinterpret_cast<const u32x4 *>(w4[q] + e);
#pragma unroll
              for (int c = 0; c < 4; ++c) {
                z4[q] = fmaf(__uint_as_float(qw[c] << 16), __uint_as_float(qh[c] << 16), z4[q]);
                z4[q] = fmaf(__uint_as_float(qw[c] & 0xffff0000u), __uint_as_float(qh[c] & 0xffff0000u), z4[q]);
              }
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) {
              const float o = __shfl_xor(z4[q], m);
              z4[q] = (ln & m) == 0 ? z4[q] + o : o + z4[q];
            }
          }
          if (ln < 4) {
            const float z = ln == 0 ? z4[0] : ln == 1 ? z4[1] : ln == 2 ? z4[2] : z4[3];
            const int64_t j = ln == 0 ? j4[0] : ln == 1 ? j4[1] : ln == 2 ? j4[2] : j4[3];
            buf[64 + wv * per + r + ln] = j < v ? topk_key(z, (int)j) : 0ull;
          }
        }
      }
      if (tid >= nrows) buf[64 + tid] = 0ull;
      __syncthreads();
      uint64_t k2[2] = {buf[64 + tid], tid < 64 ? buf[tid] : 0ull};
      __syncthreads();
      block_select64<2>(k2, buf, hist, sh);
    }
    __syncthreads();
  }

  // ---- C: ids and log-probs, in descending key order (bitonic sort of the
  // 64 selected keys across the lanes of wave 0)
  if (tid < 64) {
    const uint64_t k = wave_sort_desc(buf[tid]);
    const double l = lse_d[(int64_t)side * n + pos];
    if (ids) ids[pos * 64 + tid] = key_id(k);
    if (lp) lp[pos * 64 + tid] = f32_to_f16_bits((float)((double)key_value(k) - l));
  }
}

// Sparse-mode preparation, one block per position: the record's 512 ids
// sorted by (id, slot) (bitonic in LDS), a repeat of an id marked on its
// later slots and aliased to the first, the first entry of every 256-id
// vocabulary tile (binary search), and a flag for ids outside [0, v).
constexpr int SK = KLD_GOLDEN_TOPK;

__global__ __launch_bounds__(SK) void sparse_prep_kernel(const int32_t *__restrict__ ids,
                                                         int64_t n, int64_t v, int64_t nvt,
                                                         int32_t *__restrict__ sid,
                                                         uint16_t *__restrict__ sslot,
                                                         uint16_t *__restrict__ alias,
                                                         uint16_t *__restrict__ rp,
                                                         int32_t *__restrict__ bad) {
  __shared__ uint64_t key[SK];
  __shared__ int32_t sidl[SK];
  __shared__ int any_bad;
  const int64_t pos = blockIdx.x;
  const int t = threadIdx.x;
  if (t == 0) any_bad = 0;
  __syncthreads();
  const int32_t id = ids[pos * SK + t];
  if (id < 0 || (int64_t)id >= v) any_bad = 1;
  // order-preserving key of (signed id, slot)
  key[t] = ((uint64_t)((uint32_t)id ^ 0x80000000u) << 32) | (uint32_t)t;
  __syncthreads();
  for (int size = 2; size <= SK; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (t < SK / 2) {
        const int i = 2 * t - (t & (stride - 1));
        const int j = i + stride;
        const bool up = (i & size) == 0;
        const uint64_t a = key[i], b = key[j];
        if ((b < a) == up) {
          key[i] = b;
          key[j] = a;
        }
      }
      __syncthreads();
    }
  }
  const uint64_t k = key[t];
  const int32_t my = (int32_t)((uint32_t)(k >> 32) ^ 0x80000000u);
  const int slot = (int)(uint32_t)k;
  sidl[t] = my;
  __syncthreads();
  const bool rep = t > 0 && sidl[t - 1] == my;
  int first = t;
  while (first > 0 && sidl[first - 1] == my) --first;
  sid[pos * SK + t] = my;
  sslot[pos * SK + t] = (uint16_t)(slot | (rep ? 0x8000 : 0));
  alias[pos * SK + slot] = (uint16_t)(uint32_t)key[first];
  for (int64_t vt = t; vt <= nvt; vt += SK) {
    const int64_t lo_id = vt * BV;
    int lo = 0, hi = SK;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)sidl[mid] < lo_id) lo = mid + 1; else hi = mid;
    }
    rp[pos * (nvt + 1) + vt] = (uint16_t)lo;
  }
  if (t == 0) bad[pos] = any_bad;
}

// The 513-cell score of each position from the sparse-mode partial states:
// one wave per position merges its tiles (maxima, then the sums moved to the
// overall maximum in f64), giving lse and the candidate's unlisted mass q_T;
// then sums p_i (lp_i - (z_i - lse)) over the 512 listed cells and
// p_T (ln p_T - ln q_T) in f64 in a fixed order.
__global__ __launch_bounds__(256) void sparse_finalize_kernel(
    const float *__restrict__ part, int64_t nvt, int64_t npad, int64_t n,
    const float *__restrict__ zl, const uint16_t *__restrict__ alias,
    const int32_t *__restrict__ bad, const float *__restrict__ lp, const float *__restrict__ rec,
    float *__restrict__ kl) {
  const int64_t pos = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (pos >= n) return;
  const int64_t plane = nvt * npad;
  float m = kNegInf;
  for (int64_t t = lane; t < nvt; t += 64) m = fmaxf(m, part[t * npad + pos]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  const double r = (double)ref_of(m);
  double s = 0.0, u = 0.0;
  for (int64_t t = lane; t < nvt; t += 64) {
    const float mt = part[t * npad + pos];
    if (mt == kNegInf) continue;
    const double f = exp((double)mt - r);
    s += (double)part[plane + t * npad + pos] * f;
    u += (double)part[2 * plane + t * npad + pos] * f;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    s += __shfl_xor(s, o);
    u += __shfl_xor(u, o);
  }
  const double lse = r + log(s);
  const double q_t = u / s;
  double acc = 0.0;
  int inf = 0;
  for (int i = lane; i < SK; i += 64) {
    const double l = (double)lp[pos * SK + i];
    const double p = exp(l);
    if (p == 0.0) continue;
    const float z = zl[pos * SK + alias[pos * SK + i]];
    if (z == kNegInf) { inf = 1; continue; }
    acc += p * (l - ((double)z - lse));
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    acc += __shfl_xor(acc, o);
    inf |= __shfl_xor(inf, o);
  }
  if (lane == 0) {
    const double p_t = (double)rec[pos * 3 + 2];
    if (p_t > 0.0) {
      if (q_t == 0.0) inf = 1;
      else acc += p_t * (log(p_t) - log(q_t));
    }
    const bool nan_in = bad[pos] || !(s > 0.0) || s != s || m != m || m == __builtin_huge_valf();
    kl[pos] = nan_in ? __builtin_nanf("") : inf ? __builtin_huge_valf() : (float)acc;
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
  hipError_t e;   // the kernel's 160 KB of LDS is static: no launch attribute to set
  const int64_t nblocks = g.nvt * g.npt;
  e = record(a.ev.start, a.stream);
  if (e != hipSuccess) return e;
  if (tk)
    hipLaunchKernelGGL(fused_head_kernel<kModeTopk>, dim3((unsigned)nblocks), dim3(NT),
                       0, a.stream, a.W, a.h_ref, a.h_cand, a.v, a.d,
                       a.n, (int)g.npt, g.npad, g.nvt, w.part, w.ckeys, w.resid, w.rinfo, w.tkeys,
                       SparseIn{});
  else
    hipLaunchKernelGGL(fused_head_kernel<kModeKl>, dim3((unsigned)nblocks), dim3(NT),
                       0, a.stream, a.W, a.h_ref, a.h_cand, a.v, a.d,
                       a.n, (int)g.npt, g.npad, g.nvt, w.part, nullptr, nullptr, nullptr, nullptr,
                       SparseIn{});
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
                     w.resid, w.rinfo, w.tkeys, g.nvt, g.npad, a.n, a.W, a.h_ref, a.h_cand, a.v, a.d, w.lse,
                     a.topk);
  return hipGetLastError();
}

SparseGeom sparse_geom(int64_t n, int64_t v) {
  SparseGeom g;
  g.nvt = (v + BV - 1) / BV;
  g.npt = (n + 2 * BP - 1) / (2 * BP);
  g.npad = g.npt * 2 * BP;
  return g;
}

hipError_t launch_coarse_fused(const CoarseFusedArgs &a, const SparseWs &w) {
  const SparseGeom g = sparse_geom(a.n, a.v);
  hipLaunchKernelGGL(sparse_prep_kernel, dim3((unsigned)a.n), dim3(SK), 0, a.stream, a.ids, a.n,
                     a.v, g.nvt, w.sid, w.sslot, w.alias, w.rp, w.bad);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = record(a.ev.start, a.stream);
  if (e != hipSuccess) return e;
  SparseIn sp{w.sid, w.sslot, w.rp, w.zl};
  hipLaunchKernelGGL(fused_head_kernel<kModeSparse>, dim3((unsigned)(g.nvt * g.npt)), dim3(NT), 0,
                     a.stream, a.W, a.h_cand, a.h_cand, a.v, a.d, a.n, (int)g.npt, g.npad, g.nvt,
                     w.part, nullptr, nullptr, nullptr, nullptr, sp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = record(a.ev.stop, a.stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sparse_finalize_kernel, dim3((unsigned)((a.n + 3) / 4)), dim3(256), 0,
                     a.stream, w.part, g.nvt, g.npad, a.n, w.zl, w.alias, w.bad, a.lp, a.rec,
                     a.kl);
  return hipGetLastError();
}

}  // namespace kld

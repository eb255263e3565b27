// C ABI of libkld: argument validation (fail-closed, before any launch),
// workspace layout and kernel dispatch.  See include/kld.h for the contract.
#include "kld.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "kld_device.hpp"
#include "kld_launch.hpp"

using namespace kld;

// Workspace of kld_from_logits_noalloc (see device_scratch below).
static __device__ __align__(256) unsigned char scratch[KLD_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
// Every pointer argument must be aligned to its element size (NULL passes);
// workspaces to 16 bytes.
inline bool al(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline bool rows_aligned(const kld_rows *o) {
  return al(o->kl, 4) && al(o->nll_ref, 4) && al(o->nll_cand, 4) && al(o->lse_ref, 4) &&
         al(o->lse_cand, 4) && al(o->argmax_ref, 4) && al(o->argmax_cand, 4);
}
inline bool topk_aligned(const kld_topk *t) {
  return !t || (al(t->ids_ref, 4) && al(t->ids_cand, 4) && al(t->lp_ref, 2) && al(t->lp_cand, 2));
}

// Workspace carving: a bump allocator over the caller's buffer.
struct Carver {
  char *base;
  size_t used = 0;
  explicit Carver(void *b) : base((char *)b) {}
  template <typename T> T *take(size_t count) {
    used = round_up(used, kAlign);
    T *p = base ? (T *)(base + used) : nullptr;
    used += count * sizeof(T);
    return p;
  }
};

// ---- logits path geometry --------------------------------------------------
// Splits per row so that the grid holds about 4096 blocks (16 per CU; the
// nearest whole number of splits, so 4080 rows take one split each rather
// than two half-rows), each streaming at least 4096 ids; chunk is a multiple
// of 8 ids so that 16-byte vectors never straddle a split for either dtype.
struct LogitsGeom {
  int splits;
  int64_t chunk;
};

LogitsGeom logits_geom(int64_t n, int64_t v) {
  int64_t want = n > 0 ? (4096 + n / 2) / n : 1;
  if (want < 1) want = 1;
  if (want > kMaxSplits) want = kMaxSplits;
  int64_t max_splits = (v + 4095) / 4096;
  if (max_splits < 1) max_splits = 1;
  if (want > max_splits) want = max_splits;
  // a split spans at most kMaxChunk ids (its byte offsets fit 32 bits)
  const int64_t min_splits = (v + kMaxChunk - 1) / kMaxChunk;
  if (want < min_splits) want = min_splits;
  if (want < 1) want = 1;
  int64_t chunk = (v + want - 1) / want;
  chunk = (chunk + 7) / 8 * 8;
  LogitsGeom g;
  g.chunk = chunk;
  g.splits = (int)((v + chunk - 1) / chunk);
  return g;
}

struct LogitsWs {
  RowState *part;
  uint64_t *keys;   // with top-k
  double *lse;      // with top-k
};

LogitsWs logits_carve(int64_t n, int64_t v, bool topk, Carver *c) {
  const LogitsGeom g = logits_geom(n, v);
  LogitsWs w;
  w.part = c->take<RowState>((size_t)n * g.splits);
  w.keys = topk ? c->take<uint64_t>((size_t)n * g.splits * 2 * 64) : nullptr;
  w.lse = topk ? c->take<double>((size_t)2 * n) : nullptr;
  return w;
}

size_t logits_workspace(int64_t n, int64_t v, int flags, Carver *c) {
  logits_carve(n, v, (flags & KLD_FLAG_TOPK) != 0, c);
  return round_up(c->used, kAlign);
}

FusedWs fused_carve(int64_t n, int64_t v, bool topk, Carver *c) {
  const FusedGeom g = fused_geom(n, v);
  FusedWs w;
  w.part = c->take<float>((size_t)7 * g.nvt * g.npad);
  w.zt = c->take<float>((size_t)2 * n);
  w.lse = c->take<double>((size_t)2 * n);
  w.ckeys = topk ? c->take<uint64_t>((size_t)2 * g.nvt * g.npad * 16) : nullptr;
  w.resid = topk ? c->take<float>((size_t)2 * g.nvt * g.npad) : nullptr;
  w.rinfo = topk ? c->take<uint64_t>((size_t)2 * g.nvt * g.npad) : nullptr;
  w.tkeys = topk ? c->take<uint64_t>((size_t)2 * g.npad * g.nvt) : nullptr;
  return w;
}

SparseWs sparse_carve(int64_t n, int64_t v, Carver *c) {
  const SparseGeom g = sparse_geom(n, v);
  SparseWs w;
  w.part = c->take<float>((size_t)3 * g.nvt * g.npad);
  w.zl = c->take<float>((size_t)n * KLD_GOLDEN_TOPK);
  w.sid = c->take<int32_t>((size_t)n * KLD_GOLDEN_TOPK);
  w.sslot = c->take<uint16_t>((size_t)n * KLD_GOLDEN_TOPK);
  w.alias = c->take<uint16_t>((size_t)n * KLD_GOLDEN_TOPK);
  w.rp = c->take<uint16_t>((size_t)n * (g.nvt + 1));
  w.bad = c->take<int32_t>((size_t)n);
  return w;
}

size_t fused_workspace(int64_t n, int64_t v, int flags, Carver *c) {
  fused_carve(n, v, (flags & KLD_FLAG_TOPK) != 0, c);
  return round_up(c->used, kAlign);
}

inline hipStream_t as_stream(void *s) { return (hipStream_t)s; }

Events events_of(const kld_launch_opts *o) {
  Events e;
  if (o) { e.start = (hipEvent_t)o->main_start; e.stop = (hipEvent_t)o->main_stop; }
  return e;
}

// ---- kld_from_logits: validation and launch, shared by the workspace and
// the allocation-free entry points ------------------------------------------
kld_status check_from_logits(const void *ref, const void *cand, int dtype, int64_t n, int64_t v,
                             int64_t ld_ref, int64_t ld_cand, const int32_t *target,
                             const kld_rows *out, const kld_topk *topk) {
  if (dtype != KLD_F32 && dtype != KLD_BF16) return KLD_EDTYPE;
  if (n < 0 || v < 0) return KLD_EINVAL;
  if (!out) return KLD_EINVAL;
  if (n == 0) return KLD_OK;
  if (v < 1 || v > 0x7fffffffLL) return KLD_ESHAPE;
  if (!ref || !cand || !out->kl) return KLD_EINVAL;
  if (ld_ref < v || ld_cand < v) return KLD_ESHAPE;
  if ((out->nll_ref || out->nll_cand) && !target) return KLD_EINVAL;
  if (topk && v < KLD_TOPK) return KLD_ESHAPE;
  const size_t esize = dtype == KLD_F32 ? 4 : 2;
  if (!al(ref, esize) || !al(cand, esize) || !al(target, 4) || !rows_aligned(out) ||
      !topk_aligned(topk))
    return KLD_EUNSUPPORTED;
  return KLD_OK;
}

kld_status run_from_logits(const void *ref, const void *cand, int dtype, int64_t n, int64_t v,
                           int64_t ld_ref, int64_t ld_cand, const int32_t *target,
                           const kld_rows *out, const kld_topk *topk, void *ws, void *stream,
                           const kld_launch_opts *opts) {
  const size_t esize = dtype == KLD_F32 ? 4 : 2;
  const LogitsGeom g = logits_geom(n, v);
  LogitsArgs a;
  a.ref = ref; a.cand = cand; a.dtype = dtype; a.n = n; a.v = v;
  a.ld_ref = ld_ref; a.ld_cand = ld_cand; a.chunk = g.chunk; a.splits = g.splits;
  a.aligned = aligned16(ref) && aligned16(cand) && (ld_ref * esize) % 16 == 0 &&
              (ld_cand * esize) % 16 == 0;
  a.two = true;
  a.target = target;
  a.out = RowsOut{out->kl, out->nll_ref, out->nll_cand, out->lse_ref, out->lse_cand,
                  out->argmax_ref, out->argmax_cand};
  a.stream = as_stream(stream);
  a.ev = events_of(opts);

  Carver c(ws);
  const LogitsWs w = logits_carve(n, v, topk != nullptr, &c);
  if (launch_logits_state(a, w.part, w.keys) != hipSuccess) return KLD_EHIP;
  if (launch_logits_finalize(a, w.part, w.lse, nullptr) != hipSuccess) return KLD_EHIP;
  if (topk) {
    const TopkOut to{topk->ids_ref, topk->lp_ref, topk->ids_cand, topk->lp_cand};
    if (launch_topk_merge(w.keys, g.splits, 2, n, w.lse, to, a.stream) != hipSuccess)
      return KLD_EHIP;
  }
  return KLD_OK;
}

// ---- the allocation-free variant's scratch ---------------------------------
// The workspace of kld_from_logits_noalloc is this file-scope device array:
// every GPU the library runs on holds its own copy (at its own address) until
// the process ends.  Host code never uses the array's name as an address (on
// the host it is only a stand-in); the device address is looked up once per
// device, with that device current, and kept.  Nothing in the logits path
// needs the workspace cleared: every partial state and candidate key is
// written before it is read.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

hipError_t device_scratch(void **ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidValue;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

const char *kld_status_str(int s) {
  switch (s) {
    case KLD_OK: return "KLD_OK";
    case KLD_EINVAL: return "KLD_EINVAL: null pointer or negative count";
    case KLD_ESHAPE: return "KLD_ESHAPE: inconsistent sizes";
    case KLD_EDTYPE: return "KLD_EDTYPE: unknown dtype";
    case KLD_EWORKSPACE: return "KLD_EWORKSPACE: workspace missing, too small or not 16-byte aligned";
    case KLD_EUNSUPPORTED: return "KLD_EUNSUPPORTED: valid request the library does not serve (alignment, d % 8)";
    case KLD_EHIP: return "KLD_EHIP: HIP runtime error";
    case KLD_ETOOBIG:
      return "KLD_ETOOBIG: the request needs more workspace than the static scratch of "
             "kld_from_logits_noalloc holds";
    default: return "KLD_UNKNOWN";
  }
}

int kld_abi_version(void) { return KLD_ABI_VERSION; }

size_t kld_workspace_size(int op, int64_t n, int64_t v, int64_t d, int flags) {
  if (n < 0 || v < 0 || d < 0) return 0;
  Carver c(nullptr);
  switch (op) {
    case KLD_OP_FROM_LOGITS: return logits_workspace(n, v, flags, &c);
    case KLD_OP_TOPK_EXPORT: return logits_workspace(n, v, KLD_FLAG_TOPK, &c);
    case KLD_OP_FUSED_HEAD: return fused_workspace(n, v, flags, &c);
    case KLD_OP_SUMMARY: return round_up(summary_workspace_bytes(n), kAlign);
    case KLD_OP_PAIRED: return round_up(paired_workspace_bytes(n, v), kAlign);
    case KLD_OP_COARSE_FUSED: sparse_carve(n, v, &c); return round_up(c.used, kAlign);
    case KLD_OP_COARSE_KL: {
      if (n == 0 || v == 0) return 0;
      const CoarseGeom g = coarse_geom(n, v);
      return round_up((size_t)n * g.splits * coarse_state_bytes(), kAlign);
    }
    default: return 0;
  }
}

kld_status kld_from_logits(const void *ref, const void *cand, int dtype, int64_t n, int64_t v,
                           int64_t ld_ref, int64_t ld_cand, const int32_t *target,
                           const kld_rows *out, const kld_topk *topk, void *ws, size_t ws_bytes,
                           void *stream, const kld_launch_opts *opts) {
  const kld_status st = check_from_logits(ref, cand, dtype, n, v, ld_ref, ld_cand, target, out, topk);
  if (st != KLD_OK || n == 0) return st;
  const size_t need = kld_workspace_size(KLD_OP_FROM_LOGITS, n, v, 0, topk ? KLD_FLAG_TOPK : 0);
  if (!ws || ws_bytes < need || !aligned16(ws)) return KLD_EWORKSPACE;
  return run_from_logits(ref, cand, dtype, n, v, ld_ref, ld_cand, target, out, topk, ws, stream,
                         opts);
}

kld_status kld_from_logits_noalloc(const void *ref, const void *cand, int dtype, int64_t n,
                                   int64_t v, int64_t ld_ref, int64_t ld_cand,
                                   const int32_t *target, const kld_rows *out,
                                   const kld_topk *topk, void *stream,
                                   const kld_launch_opts *opts) {
  const kld_status st = check_from_logits(ref, cand, dtype, n, v, ld_ref, ld_cand, target, out, topk);
  if (st != KLD_OK || n == 0) return st;
  const size_t need = kld_workspace_size(KLD_OP_FROM_LOGITS, n, v, 0, topk ? KLD_FLAG_TOPK : 0);
  if (need == 0 || need > (size_t)KLD_NOALLOC_SCRATCH_BYTES) return KLD_ETOOBIG;
  void *ws = nullptr;
  if (device_scratch(&ws) != hipSuccess) return KLD_EHIP;
  return run_from_logits(ref, cand, dtype, n, v, ld_ref, ld_cand, target, out, topk, ws, stream,
                         opts);
}

kld_status kld_fused_head(const uint16_t *W, int64_t v, int64_t d, const uint16_t *h_ref,
                          const uint16_t *h_cand, int64_t n, const int32_t *target,
                          const kld_rows *out, const kld_topk *topk, void *ws, size_t ws_bytes,
                          void *stream, const kld_launch_opts *opts) {
  if (n < 0 || v < 0 || d < 0) return KLD_EINVAL;
  if (!out) return KLD_EINVAL;
  if (n == 0) return KLD_OK;
  if (v < 1 || v > 0x7fffffffLL || d < 1 || d > (1 << 20)) return KLD_ESHAPE;
  if (!W || !h_ref || !h_cand || !out->kl) return KLD_EINVAL;
  if ((out->nll_ref || out->nll_cand) && !target) return KLD_EINVAL;
  if (topk && v < KLD_TOPK) return KLD_ESHAPE;
  if (d % 8 != 0 || !aligned16(W) || !aligned16(h_ref) || !aligned16(h_cand) || !al(target, 4) ||
      !rows_aligned(out) || !topk_aligned(topk))
    return KLD_EUNSUPPORTED;
  const size_t need = kld_workspace_size(KLD_OP_FUSED_HEAD, n, v, d, topk ? KLD_FLAG_TOPK : 0);
  if (!ws || ws_bytes < need || !aligned16(ws)) return KLD_EWORKSPACE;

  Carver c(ws);
  const FusedWs w = fused_carve(n, v, topk != nullptr, &c);
  FusedArgs a;
  a.W = W; a.h_ref = h_ref; a.h_cand = h_cand; a.v = v; a.d = d; a.n = n; a.target = target;
  a.out = RowsOut{out->kl, out->nll_ref, out->nll_cand, out->lse_ref, out->lse_cand,
                  out->argmax_ref, out->argmax_cand};
  a.topk = topk ? TopkOut{topk->ids_ref, topk->lp_ref, topk->ids_cand, topk->lp_cand}
                : TopkOut{nullptr, nullptr, nullptr, nullptr};
  a.stream = as_stream(stream);
  a.ev = events_of(opts);
  if (launch_fused(a, w) != hipSuccess) return KLD_EHIP;
  return KLD_OK;
}

kld_status topk_export(const void *logits, int dtype, int64_t n, int64_t v, int64_t ld, int k,
                       int32_t *ids, uint16_t *lp, const int32_t *target, float *target_lp,
                       void *ws, size_t ws_bytes, void *stream) {
  if (dtype != KLD_F32 && dtype != KLD_BF16) return KLD_EDTYPE;
  if (n < 0 || v < 0) return KLD_EINVAL;
  if (k != KLD_TOPK) return KLD_ESHAPE;
  if (n == 0) return KLD_OK;
  if (v < KLD_TOPK || v > 0x7fffffffLL || ld < v) return KLD_ESHAPE;
  if (!logits || !ids || !lp) return KLD_EINVAL;
  if (target_lp && !target) return KLD_EINVAL;
  const size_t esize = dtype == KLD_F32 ? 4 : 2;
  if (!al(logits, esize) || !al(ids, 4) || !al(lp, 2) || !al(target, 4) || !al(target_lp, 4))
    return KLD_EUNSUPPORTED;
  if (!ws || ws_bytes < kld_workspace_size(KLD_OP_TOPK_EXPORT, n, v, 0, KLD_FLAG_TOPK) ||
      !aligned16(ws))
    return KLD_EWORKSPACE;
  const LogitsGeom g = logits_geom(n, v);
  LogitsArgs a;
  a.ref = logits; a.cand = logits; a.dtype = dtype; a.n = n; a.v = v;
  a.ld_ref = ld; a.ld_cand = ld; a.chunk = g.chunk; a.splits = g.splits;
  a.aligned = aligned16(logits) && (ld * esize) % 16 == 0;
  a.two = false;
  a.target = target;
  a.out = RowsOut{nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
  a.stream = as_stream(stream);
  Carver c(ws);
  const LogitsWs w = logits_carve(n, v, true, &c);
  if (launch_logits_state(a, w.part, w.keys) != hipSuccess) return KLD_EHIP;
  if (launch_logits_finalize(a, w.part, w.lse, target_lp) != hipSuccess) return KLD_EHIP;
  const TopkOut to{ids, lp, nullptr, nullptr};
  if (launch_topk_merge(w.keys, g.splits, 1, n, w.lse, to, a.stream) != hipSuccess) return KLD_EHIP;
  return KLD_OK;
}

kld_status kld_golden_export(const void *logits, int dtype, int64_t n, int64_t v, int64_t ld,
                             const int32_t *target, int k, int32_t *ids, float *lp, float *rec,
                             void *stream) {
  if (dtype != KLD_F32 && dtype != KLD_BF16) return KLD_EDTYPE;
  if (n < 0 || v < 0) return KLD_EINVAL;
  if (k != KLD_GOLDEN_TOPK) return KLD_ESHAPE;
  if (n == 0) return KLD_OK;
  if (n > 0x7fffffffLL || v < KLD_GOLDEN_TOPK || v > 0x7fffffffLL || ld < v) return KLD_ESHAPE;
  if (!logits || !ids || !lp || !rec) return KLD_EINVAL;
  const size_t esize = dtype == KLD_F32 ? 4 : 2;
  if (!al(logits, esize) || !al(target, 4) || !al(ids, 4) || !al(lp, 4) || !al(rec, 4))
    return KLD_EUNSUPPORTED;
  const bool aligned = aligned16(logits) && (ld * esize) % 16 == 0;
  if (launch_golden_export(logits, dtype, n, v, ld, aligned, target, ids, lp, rec,
                           as_stream(stream)) != hipSuccess)
    return KLD_EHIP;
  return KLD_OK;
}

kld_status kld_coarse_kl(const void *cand, int dtype, int64_t n, int64_t v, int64_t ld,
                         const int32_t *ids, const float *lp, const float *rec, int k, float *kl,
                         void *ws, size_t ws_bytes, void *stream) {
  if (dtype != KLD_F32 && dtype != KLD_BF16) return KLD_EDTYPE;
  if (n < 0 || v < 0) return KLD_EINVAL;
  if (k != KLD_GOLDEN_TOPK) return KLD_ESHAPE;
  if (n == 0) return KLD_OK;
  if (n > 0x7fffffffLL || v < KLD_GOLDEN_TOPK || v > 0x7fffffffLL || ld < v) return KLD_ESHAPE;
  if (!cand || !ids || !lp || !rec || !kl) return KLD_EINVAL;
  const size_t esize = dtype == KLD_F32 ? 4 : 2;
  if (!al(cand, esize) || !al(ids, 4) || !al(lp, 4) || !al(rec, 4) || !al(kl, 4))
    return KLD_EUNSUPPORTED;
  if (!ws || ws_bytes < kld_workspace_size(KLD_OP_COARSE_KL, n, v, 0, 0) || !aligned16(ws))
    return KLD_EWORKSPACE;
  const bool aligned = aligned16(cand) && (ld * esize) % 16 == 0;
  if (launch_coarse_kl(cand, dtype, n, v, ld, aligned, ids, lp, rec, kl, ws, as_stream(stream)) !=
      hipSuccess)
    return KLD_EHIP;
  return KLD_OK;
}

kld_status kld_coarse_fused(const uint16_t *W, int64_t v, int64_t d, const uint16_t *h_cand,
                            int64_t n, const int32_t *ids, const float *lp, const float *rec, int k,
                            float *kl, void *ws, size_t ws_bytes, void *stream,
                            const kld_launch_opts *opts) {
  if (n < 0 || v < 0 || d < 0) return KLD_EINVAL;
  if (k != KLD_GOLDEN_TOPK) return KLD_ESHAPE;
  if (n == 0) return KLD_OK;
  if (n > 0x7fffffffLL || v < KLD_GOLDEN_TOPK || v > 0x7fffffffLL || d < 1 || d > (1 << 20))
    return KLD_ESHAPE;
  if (!W || !h_cand || !ids || !lp || !rec || !kl) return KLD_EINVAL;
  if (d % 8 != 0 || !aligned16(W) || !aligned16(h_cand) || !al(ids, 4) || !al(lp, 4) ||
      !al(rec, 4) || !al(kl, 4))
    return KLD_EUNSUPPORTED;
  if (!ws || ws_bytes < kld_workspace_size(KLD_OP_COARSE_FUSED, n, v, d, 0) || !aligned16(ws))
    return KLD_EWORKSPACE;
  Carver c(ws);
  const SparseWs w = sparse_carve(n, v, &c);
  CoarseFusedArgs a;
  a.W = W; a.h_cand = h_cand; a.v = v; a.d = d; a.n = n;
  a.ids = ids; a.lp = lp; a.rec = rec; a.kl = kl;
  a.stream = as_stream(stream);
  a.ev = events_of(opts);
  if (launch_coarse_fused(a, w) != hipSuccess) return KLD_EHIP;
  return KLD_OK;
}

kld_status kld_paired_bootstrap(const double *sum_a, const double *sum_b, const int64_t *count,
                                int64_t nctx, const int32_t *cluster, int64_t nclust,
                                const int32_t *draws, int64_t nrep, const double *quantiles,
                                int nq, double *replicates, double *out, void *ws,
                                size_t ws_bytes, void *stream) {
  if (nctx < 0 || nclust < 0 || nrep < 0 || nq < 0) return KLD_EINVAL;
  if (nq > KLD_MAX_QUANTILES || nrep > KLD_MAX_REPLICATES || nclust > (1LL << 28))
    return KLD_ESHAPE;
  if (nrep > 0 && nclust == 0) return KLD_ESHAPE;
  if (!out || (nctx > 0 && (!sum_a || !sum_b || !count || !cluster)) ||
      (nrep > 0 && (!draws || !replicates)) || (nq > 0 && !quantiles))
    return KLD_EINVAL;
  if (!al(sum_a, 8) || !al(sum_b, 8) || !al(count, 8) || !al(cluster, 4) || !al(draws, 4) ||
      !al(replicates, 8) || !al(out, 8))
    return KLD_EUNSUPPORTED;
  PairedQuantiles qs;
  qs.count = nq;
  for (int i = 0; i < KLD_MAX_QUANTILES; ++i) {
    const double q = i < nq ? quantiles[i] : 0.0;
    if (!(q >= 0.0 && q <= 1.0)) return KLD_EINVAL;
    qs.q[i] = q;
  }
  if ((nclust > 0 || nrep > 0) &&
      (!ws || ws_bytes < kld_workspace_size(KLD_OP_PAIRED, nclust, nrep, 0, 0)))
    return KLD_EWORKSPACE;
  if ((nclust > 0 || nrep > 0) && !aligned16(ws)) return KLD_EWORKSPACE;   // 16-byte entries
  if (launch_paired_bootstrap(sum_a, sum_b, count, nctx, cluster, nclust, draws, nrep, qs,
                              replicates, out, ws, as_stream(stream)) != hipSuccess)
    return KLD_EHIP;
  return KLD_OK;
}

kld_status kld_window_summary(const float *kl, int64_t n, const int64_t *offsets, int64_t nseg,
                              int64_t score_from, const float *thresholds, int nthr,
                              double *seg_sum, int64_t *seg_count, int64_t *seg_exceed,
                              double *totals, void *stream) {
  if (n < 0 || nseg < 0 || score_from < 0 || nthr < 0) return KLD_EINVAL;
  if (nthr > KLD_MAX_THRESHOLDS || nseg > 0x7fffffffLL) return KLD_ESHAPE;
  if (!offsets || !totals || (nseg > 0 && (!seg_sum || !seg_count)) ||
      (nthr > 0 && (!thresholds || (nseg > 0 && !seg_exceed))))
    return KLD_EINVAL;
  if (n > 0 && !kl) return KLD_EINVAL;
  if (!al(kl, 4) || !al(offsets, 8) || !al(seg_sum, 8) || !al(seg_count, 8) ||
      !al(seg_exceed, 8) || !al(totals, 8))
    return KLD_EUNSUPPORTED;
  WindowThresholds thr;
  thr.count = nthr;
  for (int t = 0; t < KLD_MAX_THRESHOLDS; ++t) thr.value[t] = t < nthr ? thresholds[t] : 0.f;
  if (launch_window_summary(kl, n, offsets, nseg, score_from, thr, seg_sum, seg_count, seg_exceed,
                            totals, as_stream(stream)) != hipSuccess)
    return KLD_EHIP;
  return KLD_OK;
}

kld_status kld_topk_tail(const int32_t *ids_p, const uint16_t *lp_p, const int32_t *ids_q,
                         const uint16_t *lp_q, int64_t n, int k, int64_t v, float *kl_tail,
                         void *stream) {
  if (n < 0 || v < 0) return KLD_EINVAL;
  if (k != KLD_TOPK) return KLD_ESHAPE;
  if (n == 0) return KLD_OK;
  if (v <= KLD_TOPK || v > 0x7fffffffLL) return KLD_ESHAPE;
  if (!ids_p || !lp_p || !ids_q || !lp_q || !kl_tail) return KLD_EINVAL;
  if (!al(ids_p, 4) || !al(lp_p, 2) || !al(ids_q, 4) || !al(lp_q, 2) || !al(kl_tail, 4))
    return KLD_EUNSUPPORTED;
  if (launch_topk_tail(ids_p, lp_p, ids_q, lp_q, n, v, kl_tail, as_stream(stream)) != hipSuccess)
    return KLD_EHIP;
  return KLD_OK;
}

kld_status kld_summary(const float *kl, const int32_t *argmax_ref, const int32_t *argmax_cand,
                       const float *nll_ref, const float *nll_cand, int64_t n,
                       const double *quantiles, int nq, double *out, void *ws, size_t ws_bytes,
                       void *stream) {
  if (n < 0 || nq < 0) return KLD_EINVAL;
  if (!out) return KLD_EINVAL;
  if (n == 0) return KLD_OK;
  if (n > 0x7fffffffLL || nq > KLD_MAX_QUANTILES) return KLD_ESHAPE;
  if (!kl || (nq > 0 && !quantiles)) return KLD_EINVAL;
  if ((argmax_ref == nullptr) != (argmax_cand == nullptr)) return KLD_EINVAL;
  if ((nll_ref == nullptr) != (nll_cand == nullptr)) return KLD_EINVAL;
  SummaryArgs a;
  a.ranks.count = 2 * nq;
  a.qs.count = nq;
  for (int i = 0; i < nq; ++i) {
    const double q = quantiles[i];
    if (!(q >= 0.0 && q <= 1.0)) return KLD_ESHAPE;
    const double h = q * (double)(n - 1);
    int64_t lo = (int64_t)h;
    if (lo > n - 1) lo = n - 1;
    const int64_t hi = lo + 1 < n ? lo + 1 : n - 1;
    a.ranks.rank[2 * i] = (uint32_t)lo;
    a.ranks.rank[2 * i + 1] = (uint32_t)hi;
    a.qs.frac[i] = h - (double)lo;
  }
  if (!al(kl, 4) || !al(argmax_ref, 4) || !al(argmax_cand, 4) || !al(nll_ref, 4) ||
      !al(nll_cand, 4) || !al(out, 8))
    return KLD_EUNSUPPORTED;
  if (!ws || ws_bytes < kld_workspace_size(KLD_OP_SUMMARY, n, 0, 0, 0) || !aligned16(ws))
    return KLD_EWORKSPACE;
  a.kl = kl; a.argmax_ref = argmax_ref; a.argmax_cand = argmax_cand;
  a.nll_ref = nll_ref; a.nll_cand = nll_cand; a.n = n; a.out = out;
  a.stream = as_stream(stream);
  if (launch_summary(a, ws) != hipSuccess) return KLD_EHIP;
  return KLD_OK;
}

}  // extern "C"

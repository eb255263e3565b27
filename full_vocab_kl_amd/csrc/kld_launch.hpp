// Host-side launch interface between the C ABI (kld_api.cpp) and the kernel
// translation units.  Internal to libkld.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kld {

struct RowState;

struct RowsOut {
  float *kl, *nll_ref, *nll_cand, *lse_ref, *lse_cand;
  int32_t *argmax_ref, *argmax_cand;
};

struct TopkOut {
  int32_t *ids_ref;
  uint16_t *lp_ref;
  int32_t *ids_cand;
  uint16_t *lp_cand;
};

// ---- logits path ---------------------------------------------------------
struct Events {
  hipEvent_t start = nullptr, stop = nullptr;
};
inline hipError_t record(hipEvent_t e, hipStream_t s) { return e ? hipEventRecord(e, s) : hipSuccess; }

struct LogitsArgs {
  const void *ref, *cand;
  int dtype;              // 0 f32, 1 bf16
  int64_t n, v, ld_ref, ld_cand;
  int64_t chunk;          // ids per split (multiple of the vector width)
  int splits;
  bool aligned;           // both row sets 16-byte aligned
  bool two;               // both sides (false: reference only, top-k export)
  const int32_t *target;
  RowsOut out;
  hipStream_t stream;
  Events ev;
};
int logits_vec_elems(int dtype);
// topk_keys: NULL, or [n][splits][2][64] per-split best keys (sorted, 0-padded)
hipError_t launch_logits_state(const LogitsArgs &a, RowState *part, uint64_t *topk_keys);
// lse_d: NULL or [2][n] f64 log-sum-exp; target_lp: NULL or [n] ref log-prob of the target
hipError_t launch_logits_finalize(const LogitsArgs &a, const RowState *part, double *lse_d,
                                  float *target_lp);

// ---- top-k merge and tail KLD -----------------------------------------------
constexpr int kTopkMergeMax = 4096;   // splits * 64 candidate keys per row and side
constexpr int kMaxSplits = kTopkMergeMax / 64;
constexpr int64_t kMaxChunk = int64_t(1) << 28;   // ids per split, so 4-byte logits stay below 2^30 bytes
static_assert((int64_t(0x7fffffff) + kMaxChunk - 1) / kMaxChunk <= kMaxSplits, "every v fits");
hipError_t launch_topk_merge(const uint64_t *keys, int splits, int nsides, int64_t n,
                             const double *lse_d, const TopkOut &out, hipStream_t stream);
hipError_t launch_topk_tail(const int32_t *ids_p, const uint16_t *lp_p, const int32_t *ids_q,
                            const uint16_t *lp_q, int64_t n, int64_t v, float *kl_tail,
                            hipStream_t stream);

// ---- fused head path ------------------------------------------------------
struct FusedArgs {
  const uint16_t *W, *h_ref, *h_cand;
  int64_t v, d, n;
  const int32_t *target;
  RowsOut out;
  TopkOut topk;           // all NULL: no top-k export
  hipStream_t stream;
  Events ev;
};
struct FusedGeom {
  int64_t nvt, npt, npad;   // vocabulary tiles, position tiles, padded positions
};
FusedGeom fused_geom(int64_t n, int64_t v);
struct FusedWs {
  float *part;        // 7 * nvt * npad partial-state planes
  float *zt;          // 2 * n target logits
  double *lse;        // 2 * n log-sum-exp (top-k only)
  uint64_t *ckeys;    // 2 * nvt * npad * 16 candidate keys (top-k only)
  float *resid;       // 2 * nvt * npad tile residuals (top-k only)
  uint64_t *rinfo;    // 2 * nvt * npad: runner-up group residual | residual group << 32
  uint64_t *tkeys;    // 2 * npad * nvt tile-maximum keys, position-major (top-k only)
};
hipError_t launch_fused(const FusedArgs &a, const FusedWs &w);

// candidate hidden states scored against stored golden records through the
// shared head (sparse mode of the fused kernel)
struct CoarseFusedArgs {
  const uint16_t *W, *h_cand;
  int64_t v, d, n;
  const int32_t *ids;
  const float *lp, *rec;
  float *kl;
  hipStream_t stream;
  Events ev;
};
struct SparseGeom {
  int64_t nvt, npt, npad;   // vocabulary tiles, 256-position tiles, padded positions
};
SparseGeom sparse_geom(int64_t n, int64_t v);
struct SparseWs {
  float *part;        // 3 * nvt * npad partial-state planes (m, s, unlisted s)
  float *zl;          // n * 512 listed logits
  int32_t *sid;       // n * 512 listed ids sorted by id
  uint16_t *sslot;    // n * 512 their record slots (bit 15: repeated id)
  uint16_t *alias;    // n * 512 slot of the first occurrence of each slot's id
  uint16_t *rp;       // n * (nvt + 1) first sorted entry of each vocabulary tile
  int32_t *bad;       // n flags: an id outside [0, v)
};
hipError_t launch_coarse_fused(const CoarseFusedArgs &a, const SparseWs &w);

// ---- summary ---------------------------------------------------------------
constexpr int kSummaryMaxRanks = 32;   // two order statistics per quantile, <= 16 quantiles
struct SummaryRanks {
  int count;
  uint32_t rank[kSummaryMaxRanks];
};
struct SummaryQuantiles {
  int count;
  double frac[kSummaryMaxRanks / 2];
};
struct SummaryArgs {
  const float *kl;
  const int32_t *argmax_ref, *argmax_cand;
  const float *nll_ref, *nll_cand;
  int64_t n;
  SummaryRanks ranks;
  SummaryQuantiles qs;
  double *out;
  hipStream_t stream;
};
size_t summary_workspace_bytes(int64_t n);
hipError_t launch_summary(const SummaryArgs &a, void *ws);

// scored-window statistics (kld_window.hip)
struct WindowThresholds {
  float value[16];
  int count;
};
// paired comparison with a cluster bootstrap (kld_paired.hip)
struct PairedQuantiles {
  double q[16];
  int count;
};
size_t paired_workspace_bytes(int64_t nclust, int64_t nrep);
hipError_t launch_paired_bootstrap(const double *sum_a, const double *sum_b, const int64_t *count,
                                   int64_t nctx, const int32_t *cluster, int64_t nclust,
                                   const int32_t *draws, int64_t nrep, const PairedQuantiles &qs,
                                   double *reps, double *out, void *ws, hipStream_t stream);
hipError_t launch_window_summary(const float *kl, int64_t n, const int64_t *offsets, int64_t nseg,
                                 int64_t score_from, const WindowThresholds &thr, double *seg_sum,
                                 int64_t *seg_count, int64_t *seg_exceed, double *totals,
                                 hipStream_t stream);

// golden records and the 513-cell score (kld_golden.hip)
hipError_t launch_golden_export(const void *logits, int dtype, int64_t n, int64_t v, int64_t ld,
                                bool aligned, const int32_t *target, int32_t *ids, float *lp,
                                float *rec, hipStream_t stream);
struct CoarseGeom {
  int splits;
  int64_t chunk;
};
CoarseGeom coarse_geom(int64_t n, int64_t v);
size_t coarse_state_bytes();   // per (row, range) partial state in the workspace
hipError_t launch_coarse_kl(const void *cand, int dtype, int64_t n, int64_t v, int64_t ld,
                            bool aligned, const int32_t *ids, const float *lp, const float *rec,
                            float *kl, void *part_ws, hipStream_t stream);

}  // namespace kld

// spec_internal.h -- launch descriptors shared by the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

namespace specv {

constexpr int kModeSoftmax = 0;
constexpr int kModeArgmax = 1;
constexpr int kMaxChunks = 512;   // V <= 512 * 4096 logits
constexpr int kMaxGamma = 64;     // gamma_max bound (one finalize thread per position)

// fused single-kernel path limits (larger problems take the multi-kernel path)
constexpr int kMaxSlicesFused = 64;    // V <= 64 * 4096
constexpr int kMaxTeamsFused = 4096;   // target rows
constexpr int kMaxReqFused = 1024;     // requests
constexpr int kFusedWgsPerCu = 8;       // resident streaming workgroups per CU (64 VGPRs, 19.7 KB LDS)
constexpr int kMaxMembers = 32;        // streaming workgroups of one target row (two slices each)
constexpr int kFuSample = 0;           // draft logits, temperature > 0
constexpr int kFuTokenOnly = 1;        // token-only draft, temperature > 0
constexpr int kFuGreedy = 2;           // temperature 0

// Header at the start of every workspace (the multi-kernel path's offset-check flag; the
// filtered path's count of units sent to the dense recomputation).
constexpr size_t kHeaderBytes = 256;
constexpr size_t kHdrCuBad = 0;                                     // i32
constexpr size_t kHdrOvfN = 4;                                      // i32

// How a logical row index maps onto the caller's arrays (see resolve_row).
struct RowMap {
  const void* tgt;
  int64_t tgt_ld;
  const void* drf;          // nullptr: no draft / q rows
  int64_t drf_ld;
  const int32_t* cu;        // request mode: [B + 1] draft-row offsets; nullptr: plain rows
  int B;                    // requests, or rows in plain-row mode
  int G;                    // gamma_max (request mode)
  int n_draft_rows;         // cu[B] as stated by the caller (request mode)
  const int* cu_bad;        // request mode: set when cu is not a valid exclusive prefix
  const float* thr;         // per logical row: filter threshold (a logit below it is masked);
                            // nullptr: unfiltered
};

// spec_row_stats outputs written by the combine kernel (plain-row mode).
struct RowStatsOut {
  int enabled;
  float* max_logit;
  int32_t* argmax;
  float* log_z;
  float* entropy_bits;
  float* max_prob;
  int32_t* kept_count;
};

struct SlicePart;
struct RowStat;
struct Part4;
struct TeamStat;

struct DenseLaunch {
  RowMap map;
  int dt, V, n_slices, n_slots;
  float c;                  // log2(e) / T (0 when greedy)
  int greedy, want_argmax, pair, vec;
  int want_kl;              // the pair pass also gathers the KL divergences' sums
  SlicePart* part;
  RowStat* rs;
  double* smass;            // [n_slots][n_slices] sum over the slice of [p - q]_+
  double* amass;            // [n_slots][n_slices] sum over the slice of min(p, q)
  double* kmass;            // [n_slots][n_slices][4] sum p (l_p - l_q), sum q (l_q - l_p), and the
                            // counts of p > 0 = q, q > 0 = p (the KL divergences' support)
  RowStatsOut rso;
  hipEvent_t ev_start, ev_stop;   // optional: bracket the streaming pass (benchmark timing)
};

struct PosStatsOut {
  float* p_y;
  float* q_y;
  float* one_minus_tv;
  float* draft_entropy_bits;
  float* draft_max_prob;
  float* target_entropy_bits;
  float* target_max_prob;
  float* kl_pq;
  float* kl_qp;
  float* l1;
  float* accept_prob;
  float* expected_committed;   // [B]
};

struct FinalizeArgs {
  RowMap map;
  int V, n_slices, greedy;
  int vec;                  // rows 16-byte aligned (vector loads when rows are read again)
  float c;
  double inv_t;             // 1 / T (T > 0)
  uint64_t seed, step;
  const int32_t* tokens;
  const RowStat* rs;
  const SlicePart* part;
  const double* smass;
  const double* amass;
  const double* kmass;
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  float* out_req_stats;
  int32_t* out_status;
  PosStatsOut st;
};

struct ResidualArgs {
  RowMap map;               // plain-row mode, B = R
  int V, n_slices, greedy;
  float c;
  uint64_t seed, step;
  const double* uniforms;
  const RowStat* rs;
  const SlicePart* part;
  const double* smass;
  int32_t* out_token;
  double* out_mass;
  int32_t* out_status;
};

struct FusedArgs {
  const void* tgt;
  int64_t tgt_ld;
  const void* drf;
  int64_t drf_ld;
  const int32_t* cu;
  const int32_t* tokens;
  int B, G, V, n_s, n_draft_rows, n_teams, n_tickets, mode, want_t_ent;
  unsigned spin_limit;
  uint32_t tag;         // this call's record tag (never 0)
  float c;
  uint64_t seed, step;
  uint64_t* part;       // [n_teams][2 rows][n_s] 16-byte tagged slice records
  uint64_t* smass;      // [n_teams][n_s][4 waves] tagged residual masses
  uint32_t* arrive;     // [n_teams][kMaxMembers] a member's flag: the call's tag once its records are out
  float* ylog;          // [n_draft_rows][2]: each draft token's logit in its target and draft row
  const float* thr;     // filtered calls off the sparse path, uniform batches only: per logical row
                        // 2 (b (G + 1) + i) + kind (kind 0 target, 1 draft) the filter threshold,
                        // a logit below it masked; nullptr: unfiltered
  int ragged;           // 1 unless every request has G draft rows: a dispatch place then finds its
                        // request among the offsets instead of from its place
  int poll_delay;       // wait before the first team poll, in 10 ns ticks
  int tail_wgs;         // the launch's last generation (one workgroup per resident slot), which
                        // waits half the poll delay
  int poll_pause;       // pause between team polls, in units of 128 cycles
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  float* out_req_stats;
  int32_t* out_status;
  PosStatsOut st;
};

hipError_t launch_fused(const FusedArgs& a, int dt, int vec, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);

// Launch a kernel; with both events given they are recorded by the dispatch itself around the
// kernel (start and end of its execution), so that their interval holds no launch gap.
template <typename K, typename... Args>
inline void launch_timed(K kernel, dim3 grid, dim3 block, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1,
                         Args... args) {
  if (ev0 && ev1) hipExtLaunchKernelGGL(kernel, grid, block, 0, st, ev0, ev1, 0, args...);
  else hipLaunchKernelGGL(kernel, grid, block, 0, st, args...);
}

// ---------------------------------------------------------------- filtered (top-k / top-p) path

constexpr int kKeepMax = 512;          // largest top-k set (k plus boundary ties) a row may keep
constexpr int kFilterMaxK = 256;       // largest top_k the sparse path accepts

struct CandEntry {       // a candidate logit of a slice
  float v;
  int x;                 // token index
};
struct CandHead {        // one (row, slice): candidates stored / found, threshold digits, flags
  int stored, total;
  uint32_t th;
  int flags;
};
struct KeptEntry {       // a kept token of a row, in index order
  int x, pad;
  double p;
};
struct RowStat2 {        // a row's filtered distribution
  int n, flags;          // kept entries; kFlag* bits
  float m;               // max logit
  int argmax;
  int kept_finite, pad;  // kept entries with a finite logit
  double log_z, entropy, max_prob, z;
};

// The dense recomputation of what the sparse filtered path cannot hold: a row whose top-k set
// (k plus its boundary ties) exceeds kKeepMax, or a slice that had to drop tied candidates the
// row keeps.  The sparse path's last kernel lists such units (requests, or plain rows) in
// device memory; these kernels then run the dense threshold path on the listed units only
// (every workgroup reads the list's length and leaves when it is zero).
struct FallbackRows {
  RowMap map;               // map.thr = thr
  int V, n_slices, n_lr;    // n_lr: logical rows of the whole call
  int unit_lr;              // logical rows per listed unit: 2 (G + 1) per request, 2 per plain row
  int k;                    // top_k
  float top_p;
  double cthr;              // log2(e) / T for the threshold search
  float c;                  // log2(e) / T
  int want_argmax;          // argmax and kept counts in the row statistics (spec_row_stats)
  float* thr;               // [n_lr]
  SlicePart* part;          // [n_lr][n_slices]
  RowStat* rs;              // [n_lr]
  RowStatsOut rso;
  const int* list;          // listed units
  const int* list_n;        // their number
};

struct FilterArgs {
  const void* tgt;
  int64_t tgt_ld;
  const void* drf;
  int64_t drf_ld;
  const int32_t* cu;
  const int32_t* tokens;
  int B, G, V, n_s, n_draft_rows, n_teams, n_slots, mode, k, cap;
  int n_l;                // candidate lists per row (set by the launchers; n_l <= n_s)
  float top_p;
  double c, inv_t;        // c = log2(e) / T
  uint64_t seed, step;
  CandEntry* cand;        // [n_slots][n_l][cap] (sized for n_s lists); a bf16 list holds one 32-bit word per entry
  CandHead* chead;        // [n_slots][n_l] (sized for n_s)
  KeptEntry* kept;        // [n_slots][kKeepMax]
  RowStat2* rstat;        // [n_slots]
  int32_t* out_tokens;
  int32_t* out_num_accepted;
  float* out_req_stats;
  int32_t* out_status;
  PosStatsOut st;
  // units the sparse sets cannot hold, for the dense recomputation (requests, or plain rows)
  int* ovf_list;            // [B]
  int* ovf_n;               // zeroed by the first kernel, one increment per listed unit
  int* cu_bad0;             // the dense path's offset flag, zeroed by the first kernel
  // plain rows (spec_row_stats / spec_residual_sample): target row r pairs with draft row r
  int direct;
  const double* uniforms;   // residual draws: [rows][3] injected uniforms, or nullptr (Philox)
  double* out_mass;
  RowStatsOut rso;
};

// Candidate slots of one list for top-k = k.  A list's candidates are its logits at or above
// the k-th largest of its 256 per-thread maxima (32 logits per thread), so for a row of i.i.d.
// values their expected count is 8192 (1 - q^(1/32)) with q = (256.5 - k) / 257, the expected
// quantile of that order statistic: 56 at k = 50, 175 at k = 128, about 1450 at k = 256.  The
// slots hold that count plus five standard deviations of it (and never fewer than k + 32), so
// that a list rarely takes the exact select, which reads the list again.
inline int filter_cap(int k) {
  const double q = (256.5 - (double)k) / 257.0;
  const double c = 8192.0 * (1.0 - pow(q > 0.0 ? q : 1e-9, 1.0 / 32.0));
  const int need = (int)ceil(c + 5.0 * sqrt(c));
  const int cap = need > k + 32 ? need : k + 32;
  return (cap < 8192 ? cap : 8192) + 15 & ~15;
}
hipError_t launch_filter(const FilterArgs& a, int dt, int vec, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
// Plain filtered rows: what = 0, the statistics of n_teams rows (a.rso); what = 1, one residual
// draw per row pair (target row r, draft row r or none).
hipError_t launch_filter_rows(const FilterArgs& a, int dt, int vec, int what, hipStream_t st);
hipError_t launch_check_cu(const int32_t* cu, int B, int G, int n_draft_rows, int* cu_bad, hipStream_t st);
size_t fused_record_bytes();

hipError_t launch_dense(const DenseLaunch& L, hipStream_t st);
// The dense recomputation of listed units: per logical row the threshold, slice statistics and
// row statistics; then per listed request the pair sums and the finalize (a.map and the arrays
// of `a` as the dense path carves them), or per listed plain row the pair sums and the
// residual draw.
hipError_t launch_fallback_rows(const FallbackRows& f, int dt, int vec, hipStream_t st);
hipError_t launch_fallback_requests(const FallbackRows& f, const FinalizeArgs& a, int want_kl, int dt, int vec,
                                    hipStream_t st);
hipError_t launch_fallback_residual(const FallbackRows& f, const ResidualArgs& a, double* amass, int dt, int vec,
                                    hipStream_t st);
// Filter thresholds of logical rows 0..n_lr-1 of `m` into thr[n_lr] (c = log2(e) / T).
hipError_t launch_threshold(const RowMap& m, int dt, int vec, int V, int n_lr, int k, float top_p, double c,
                            float* thr, hipStream_t st);
hipError_t launch_finalize(const FinalizeArgs& a, int dt, hipStream_t st);
hipError_t launch_select_gamma(int B, const float* req_stats, const float* comp, const float* w1, const float* b1,
                               const float* w2, float b2, int32_t* out_gamma, float* out_expected, hipStream_t st);
hipError_t launch_residual_finalize(const ResidualArgs& a, int dt, hipStream_t st);
hipError_t launch_stream_read(const void* buf, int64_t n16, uint32_t* sink, hipStream_t st, hipEvent_t ev0,
                              hipEvent_t ev1);

// ---------------------------------------------------------------- fused LM head

struct HeadRec {          // a row's partials over one 256-column tile of l = h W^T
  float m;                // maximum
  int amax;               // lowest arg-max; -1 none, -2 a NaN or +inf logit
  double s, w;            // sum e and sum e t with e = 2^t, t = (l - m) c (fp64: a peaked row's
                          // sum is 1 plus a little, which fp32 would round away)
};
struct HeadArgs {
  const void* hidden;     // [R, D] bf16, row stride h_ld
  int64_t h_ld;
  const void* weight;     // [V, D] bf16, row stride w_ld
  int64_t w_ld;
  int R, V, D, n_rt, n_ct, greedy;
  float c;                // log2(e) / T
  double inv_t;
  const int32_t* tokens;  // [R] or nullptr
  HeadRec* rec;           // [R][n_ct]
  float* ly;              // [R]: the logit of tokens[r]
  float* max_logit;
  int32_t* argmax;
  float* log_z;
  float* entropy_bits;
  float* max_prob;
  float* p_tok;
};
constexpr int kHeadCols = 256;   // vocabulary columns per tile
hipError_t launch_head(const HeadArgs& a, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);

size_t slice_part_bytes();
size_t row_stat_bytes();

}  // namespace specv

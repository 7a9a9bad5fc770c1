// spec_api.hip -- the C ABI of libspecverify: argument checks, workspace carving, launches.
// Declarations and their documentation are in include/spec_verify.h.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "spec_device.h"
#include "spec_internal.h"
#include "spec_verify.h"

using namespace specv;

namespace {

constexpr size_t kAlign = 256;

// A call's options (spec_call_options, every field defaulted when the pointer is NULL).  The
// single kernel's team wait gives up after spin_limit polls; a member waits poll_delay 10-ns
// ticks after publishing before its first poll and pauses poll_pause x 128 cycles after a
// failed one (device-scope polls compete with the row stream, so few and late polls are
// cheaper than early ones).
struct Opts {
  bool multi;            // every kernel of the multi-kernel path (filtered: the dense threshold path)
  unsigned spin_limit;
  int poll_delay, poll_pause;
  hipEvent_t ev0, ev1;   // bracket the streaming kernel, or none
};
Opts resolve(const spec_call_options* o) {
  Opts r;
  r.multi = o != nullptr && o->path == SPEC_PATH_MULTI_KERNEL;
  r.spin_limit = (o == nullptr || o->spin_limit < 0) ? (1u << 18)
                 : (unsigned)(o->spin_limit > 0x7fffffff ? 0x7fffffff : o->spin_limit);
  r.poll_delay = (o == nullptr || o->poll_delay <= 0) ? 400 : o->poll_delay;
  r.poll_pause = (o == nullptr || o->poll_pause <= 0) ? 8 : o->poll_pause;
  r.ev0 = o ? (hipEvent_t)o->profile_start : nullptr;
  r.ev1 = o ? (hipEvent_t)o->profile_stop : nullptr;
  return r;
}
// NULL or a valid path; both profile events or neither.
bool opts_valid(const spec_call_options* o) {
  if (o == nullptr) return true;
  if (o->path != SPEC_PATH_AUTO && o->path != SPEC_PATH_MULTI_KERNEL) return false;
  return (o->profile_start == nullptr) == (o->profile_stop == nullptr);
}

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int n_chunks(int V) { return (V + kChunk - 1) / kChunk; }

bool filter_on(int V, const spec_sampling_params& sp) {
  return sp.temperature > 0.f && ((sp.top_k > 0 && sp.top_k < V) || sp.top_p < 1.f);
}

// log2(e) / T, the scale of every exponent 2^(l c - ref) (0 when greedy).
float exp2_scale(const spec_sampling_params& sp) {
  return sp.temperature > 0.f ? (float)(1.4426950408889634 / (double)sp.temperature) : 0.f;
}

// Sampling parameters: temperature finite and >= 0, top_p > 0 (NaN rejected).
int check_params(const spec_sampling_params& sp) {
  if (!(sp.temperature >= 0.f) || !isfinite(sp.temperature)) return SPEC_ERR_INVALID;
  if (!(sp.top_p > 0.f)) return SPEC_ERR_INVALID;
  return SPEC_OK;
}

int elem_bytes(spec_dtype dt) { return dt == SPEC_BF16 ? 2 : 4; }

bool aligned16(const void* p, int64_t ld, spec_dtype dt) {
  return p == nullptr || (((uintptr_t)p % 16) == 0 && ((ld * elem_bytes(dt)) % 16) == 0);
}

struct Carve {
  char* base;
  size_t off = kHeaderBytes;
  template <typename T>
  T* take(size_t bytes) {
    T* p = (T*)(base + off);
    off += align_up(bytes);
    return p;
  }
};

// The multi-kernel arrays, in the order dense_arrays_bytes counts them.
struct DenseArrays {
  SlicePart* part;
  RowStat* rs;
  double *smass, *amass, *kmass;
};
DenseArrays carve_dense(Carve& cv, int64_t n_slots, int ns) {
  DenseArrays d;
  d.part = cv.take<SlicePart>((size_t)(2 * n_slots) * ns * slice_part_bytes());
  d.rs = cv.take<RowStat>((size_t)(2 * n_slots) * row_stat_bytes());
  d.smass = cv.take<double>((size_t)n_slots * ns * sizeof(double));
  d.amass = cv.take<double>((size_t)n_slots * ns * sizeof(double));
  d.kmass = cv.take<double>((size_t)n_slots * ns * 4 * sizeof(double));
  return d;
}

PosStatsOut pos_out(const spec_pos_stats& p) {
  PosStatsOut o;
  o.p_y = p.p_y;
  o.q_y = p.q_y;
  o.one_minus_tv = p.one_minus_tv;
  o.draft_entropy_bits = p.draft_entropy_bits;
  o.draft_max_prob = p.draft_max_prob;
  o.target_entropy_bits = p.target_entropy_bits;
  o.target_max_prob = p.target_max_prob;
  o.kl_pq = p.kl_pq;
  o.kl_qp = p.kl_qp;
  o.l1 = p.l1;
  o.accept_prob = p.accept_prob;
  o.expected_committed = p.expected_committed;
  return o;
}

// The dense recomputation of the units the sparse path lists: arrays carved after the sparse
// ones, the list's length in the workspace header (both zeroed by the sparse path's first
// kernel).
FallbackRows fallback_rows(Carve& cv, char* ws, const RowMap& map, int64_t n_units, int64_t n_slots, int unit_lr,
                           int V, const spec_sampling_params& sp, int want_argmax, DenseArrays& d) {
  const int ns = n_chunks(V);
  FallbackRows f;
  memset(&f, 0, sizeof(f));
  d = carve_dense(cv, n_slots, ns);
  f.thr = cv.take<float>((size_t)(2 * n_slots) * sizeof(float));
  f.list = cv.take<int>((size_t)n_units * sizeof(int));
  f.list_n = (const int*)(ws + kHdrOvfN);
  f.map = map;
  f.map.cu_bad = (const int*)(ws + kHdrCuBad);
  f.map.thr = f.thr;
  f.V = V;
  f.n_slices = ns;
  f.n_lr = (int)(2 * n_slots);
  f.unit_lr = unit_lr;
  f.k = sp.top_k;
  f.top_p = sp.top_p;
  f.cthr = 1.4426950408889634 / (double)sp.temperature;
  f.c = exp2_scale(sp);
  f.want_argmax = want_argmax;
  f.part = d.part;
  f.rs = d.rs;
  return f;
}

// Arrays of the multi-kernel path for n_slots slots (2 logical rows each).
size_t dense_arrays_bytes(int64_t n_slots, int V) {
  const int64_t n_lr = 2 * n_slots;
  const int64_t ns = n_chunks(V);
  return align_up((size_t)(n_lr * ns) * slice_part_bytes()) + align_up((size_t)n_lr * row_stat_bytes()) +
         2 * align_up((size_t)(n_slots * ns) * sizeof(double)) + align_up((size_t)(n_slots * ns * 4) * sizeof(double));
}
// Workspace of the multi-kernel path, after the header.
size_t dense_bytes(int64_t n_slots, int V) { return kHeaderBytes + dense_arrays_bytes(n_slots, V); }

// Workspace of the fused path for n_teams target rows, after the header.
size_t fused_bytes(int64_t n_teams, int V) {
  const int64_t ns = n_chunks(V);
  return kHeaderBytes + align_up((size_t)(n_teams * ns * 2) * fused_record_bytes()) +
         align_up((size_t)(n_teams * ns * 4) * sizeof(uint64_t)) + align_up((size_t)(n_teams * kMaxMembers) * 4) +
         align_up((size_t)n_teams * 2 * sizeof(float));
}

// Tags of the fused kernel's workspace records: one per call, unique within the process,
// never 0 (a zero-filled workspace holds no valid record).
std::atomic<uint32_t> g_call_seq{0};
uint32_t next_tag() {
  uint32_t t;
  do { t = g_call_seq.fetch_add(1, std::memory_order_relaxed) + 1; } while (t == 0);
  return t;
}

// The fused single-kernel path covers these shapes; the rest takes the multi-kernel path.
bool fused_ok(int B, int V, int gamma_max) {
  return B <= kMaxReqFused && (int64_t)B * (gamma_max + 1) <= kMaxTeamsFused && n_chunks(V) <= kMaxSlicesFused;
}

// The sparse filtered path: T > 0 with top-k on (1 <= k <= 256, k < V; top-p optional), the
// fused path's shape limits.  Every other filtered call (top-p alone, a larger k, larger
// shapes) takes the dense threshold path, as does every filtered call asked to take the
// multi-kernel path.
bool filter_supported(int B, int V, int gamma_max, const spec_sampling_params& sp) {
  return sp.temperature > 0.f && sp.top_k >= 1 && sp.top_k < V && sp.top_k <= kFilterMaxK && B <= kMaxReqFused &&
         (int64_t)B * (gamma_max + 1) <= kMaxTeamsFused && n_chunks(V) <= kMaxSlicesFused;
}
// The same sparse path for plain rows (spec_row_stats, spec_residual_sample): R rows, or R row
// pairs, each one team of its own.
bool filter_rows_supported(int R, int V, const spec_sampling_params& sp) {
  return sp.temperature > 0.f && sp.top_k >= 1 && sp.top_k < V && sp.top_k <= kFilterMaxK &&
         n_chunks(V) <= kMaxSlicesFused && (int64_t)R * n_chunks(V) <= 0x3fffffff;
}
// Thresholds of the dense filtered path: one float per logical row.
size_t thr_bytes(int64_t n_slots) { return align_up((size_t)(2 * n_slots) * sizeof(float)); }
// The sparse path's dense recomputation of listed units: the multi-kernel arrays and thresholds
// for n_slots slots, and the list of up to n_units units.
size_t fallback_bytes(int64_t n_units, int64_t n_slots, int V) {
  return dense_arrays_bytes(n_slots, V) + thr_bytes(n_slots) + align_up((size_t)n_units * sizeof(int));
}
size_t filter_bytes(int64_t n_slots, int V, int k) {
  const int64_t ns = n_chunks(V);
  return kHeaderBytes + align_up((size_t)(n_slots * ns * filter_cap(k)) * sizeof(CandEntry)) +
         align_up((size_t)(n_slots * ns) * sizeof(CandHead)) + align_up((size_t)n_slots * kKeepMax * sizeof(KeptEntry)) +
         align_up((size_t)n_slots * sizeof(RowStat2));
}


// Launch descriptor of the sparse path over R plain rows (p rows as targets, q rows, if any,
// as their draft rows), its arrays carved from the workspace.
FilterArgs plain_filter_args(int R, int V, const void* p, int64_t p_ld, const void* q, int64_t q_ld,
                             const spec_sampling_params& sp, Carve& cv) {
  FilterArgs f;
  memset(&f, 0, sizeof(f));
  const int ns = n_chunks(V);
  f.tgt = p;
  f.tgt_ld = p_ld;
  f.drf = q;
  f.drf_ld = q_ld;
  f.B = R;
  f.V = V;
  f.n_s = ns;
  f.n_teams = R;
  f.n_draft_rows = q ? R : 0;
  f.n_slots = q ? 2 * R : R;
  f.k = sp.top_k;
  f.cap = filter_cap(sp.top_k);
  f.top_p = sp.top_p;
  f.c = 1.4426950408889634 / (double)sp.temperature;
  f.inv_t = 1.0 / (double)sp.temperature;
  f.direct = 1;
  f.cand = cv.take<CandEntry>((size_t)f.n_slots * ns * f.cap * sizeof(CandEntry));
  f.chead = cv.take<CandHead>((size_t)f.n_slots * ns * sizeof(CandHead));
  f.kept = cv.take<KeptEntry>((size_t)f.n_slots * kKeepMax * sizeof(KeptEntry));
  f.rstat = cv.take<RowStat2>((size_t)f.n_slots * sizeof(RowStat2));
  return f;
}

}  // namespace

namespace specv {
// The matrix-rate kernel's launcher (spec_head.hip), used only by spec_mfma_rate.
hipError_t launch_mfma_rate(int mode, int iters, int workgroups, float* sink, hipStream_t st, hipEvent_t ev0,
                            hipEvent_t ev1);
}  // namespace specv

extern "C" {

const char* spec_status_string(int code) {
  switch (code) {
    case SPEC_OK: return "ok";
    case SPEC_ERR_INVALID: return "invalid argument";
    case SPEC_ERR_UNSUPPORTED: return "unsupported combination";
    case SPEC_ERR_WORKSPACE: return "workspace too small";
    case SPEC_ERR_LAUNCH: return "HIP launch failed";
    case SPEC_ERR_SCRATCH_LIMIT: return "call needs more workspace than the no-allocation scratch holds";
    case SPEC_STATUS_NONFINITE: return "non-finite logits";
    case SPEC_STATUS_BAD_TOKEN: return "draft token out of range";
    case SPEC_STATUS_ZERO_Q: return "draft probability of the draft token is zero";
    case SPEC_STATUS_RESIDUAL_EMPTY: return "empty residual, drawn from p";
    case SPEC_STATUS_TIMEOUT: return "bounded wait expired";
    case SPEC_STATUS_FILTER_OVERFLOW: return "filtered row too large for the sparse path (recomputed densely)";
    case SPEC_STATUS_BAD_GAMMA: return "inconsistent draft offsets";
    default: return "unknown code";
  }
}

// Workspace sizes cover every path a call can take (with any options), so a caller sizes once.
size_t spec_verify_workspace_bytes(int B, int V, int gamma_max, spec_dtype dt, spec_sampling_params sp) {
  (void)dt;
  if (B <= 0 || V <= 0 || gamma_max < 0) return 0;
  const int64_t n_slots = (int64_t)B * (gamma_max + 1);
  const size_t dense = dense_bytes(n_slots, V);
  if (filter_on(V, sp)) {
    const size_t thr = dense + thr_bytes(n_slots);
    // the fused path with thresholds (uniform bf16 batches) needs the thresholds ahead of its arrays
    const size_t fthr = fused_bytes(n_slots, V) + thr_bytes(n_slots);
    const size_t off_sparse = thr > fthr ? thr : fthr;
    if (!filter_supported(B, V, gamma_max, sp)) return off_sparse;
    const size_t sparse = filter_bytes((int64_t)B * (2 * gamma_max + 1), V, sp.top_k) + fallback_bytes(B, n_slots, V);
    return sparse > off_sparse ? sparse : off_sparse;
  }
  const size_t fused = fused_bytes(n_slots, V);
  return dense > fused ? dense : fused;
}

size_t spec_row_stats_workspace_bytes(int R, int V, spec_dtype dt, spec_sampling_params sp) {
  (void)dt;
  if (R <= 0 || V <= 0) return 0;
  if (!filter_on(V, sp)) return dense_bytes(R, V);
  const size_t thr = dense_bytes(R, V) + thr_bytes(R);
  if (!filter_rows_supported(R, V, sp)) return thr;
  const size_t sparse = filter_bytes(R, V, sp.top_k) + fallback_bytes(R, R, V);
  return sparse > thr ? sparse : thr;
}

size_t spec_residual_sample_workspace_bytes(int R, int V, spec_dtype dt, spec_sampling_params sp) {
  (void)dt;
  if (R <= 0 || V <= 0) return 0;
  if (!filter_on(V, sp)) return dense_bytes(R, V);
  const size_t thr = dense_bytes(R, V) + thr_bytes(R);
  if (!filter_rows_supported(R, V, sp)) return thr;
  const size_t sparse = filter_bytes(2 * (int64_t)R, V, sp.top_k) + fallback_bytes(R, R, V);
  return sparse > thr ? sparse : thr;
}

int spec_verify_batch_ex(int B, int V, int gamma_max, spec_dtype dt, const void* target_logits, int64_t target_ld,
                         const void* draft_logits, int64_t draft_ld, const int32_t* draft_tokens,
                         const int32_t* cu_draft, int n_draft_rows, spec_sampling_params sp, uint64_t seed,
                         uint64_t step, int32_t* out_tokens, int32_t* out_num_accepted, spec_pos_stats pos_stats,
                         float* out_req_stats, int32_t* out_status, void* workspace, size_t workspace_bytes,
                         void* hip_stream, const spec_call_options* options) {
  if (B < 0 || V <= 0 || gamma_max < 0 || gamma_max > kMaxGamma) return SPEC_ERR_INVALID;
  if (dt != SPEC_F32 && dt != SPEC_BF16) return SPEC_ERR_INVALID;
  if (!opts_valid(options)) return SPEC_ERR_INVALID;
  if (V > kMaxChunks * kChunk) return SPEC_ERR_UNSUPPORTED;
  if (check_params(sp) != SPEC_OK) return SPEC_ERR_INVALID;
  if (B == 0) return SPEC_OK;
  if (n_draft_rows < 0 || (int64_t)n_draft_rows > (int64_t)B * gamma_max) return SPEC_ERR_INVALID;
  if (!target_logits || target_ld < V || !cu_draft || !out_tokens || !out_num_accepted || !out_status)
    return SPEC_ERR_INVALID;
  if (n_draft_rows > 0 && !draft_tokens) return SPEC_ERR_INVALID;
  if (draft_logits && draft_ld < V) return SPEC_ERR_INVALID;
  if ((int64_t)B * (gamma_max + 1) * 2 > (int64_t)INT32_MAX / 2) return SPEC_ERR_INVALID;
  const Opts op = resolve(options);
  const bool greedy = sp.temperature == 0.f;
  const bool filtered = filter_on(V, sp);
  const bool sparse = filtered && !op.multi && filter_supported(B, V, gamma_max, sp);
  const size_t need = spec_verify_workspace_bytes(B, V, gamma_max, dt, sp);
  if (need > 0 && (!workspace || workspace_bytes < need)) return SPEC_ERR_WORKSPACE;
  if (((uintptr_t)workspace % kAlign) != 0) return SPEC_ERR_INVALID;

  const hipStream_t st = (hipStream_t)hip_stream;
  const int n_slots = B * (gamma_max + 1);
  const int ns = n_chunks(V);
  const void* drf = greedy ? nullptr : draft_logits;
  const PosStatsOut po = pos_out(pos_stats);
  const bool want_kl = pos_stats.kl_pq != nullptr || pos_stats.kl_qp != nullptr;

  RowMap map;
  memset(&map, 0, sizeof(map));
  map.tgt = target_logits;
  map.tgt_ld = target_ld;
  map.drf = drf;
  map.drf_ld = draft_ld;
  map.cu = cu_draft;
  map.B = B;
  map.G = gamma_max;
  map.n_draft_rows = n_draft_rows;

  // the multi-kernel path's finalize arguments (also those of the sparse path's dense
  // recomputation); the arrays are filled in where they are carved
  FinalizeArgs fa;
  memset(&fa, 0, sizeof(fa));
  fa.V = V;
  fa.n_slices = ns;
  fa.greedy = greedy;
  fa.c = exp2_scale(sp);
  fa.inv_t = greedy ? 0.0 : 1.0 / (double)sp.temperature;
  fa.seed = seed;
  fa.step = step;
  fa.tokens = draft_tokens;
  fa.out_tokens = out_tokens;
  fa.out_num_accepted = out_num_accepted;
  fa.out_req_stats = out_req_stats;
  fa.out_status = out_status;
  fa.st = po;

  char* ws = (char*)workspace;
  const int dtc = dt == SPEC_BF16 ? kDtBF16 : kDtF32;
  const bool vec = aligned16(target_logits, target_ld, dt) && aligned16(drf, draft_ld, dt);
  fa.vec = vec ? 1 : 0;
  if (sparse) {
    FilterArgs f;
    memset(&f, 0, sizeof(f));
    f.tgt = target_logits;
    f.tgt_ld = target_ld;
    f.drf = drf;
    f.drf_ld = draft_ld;
    f.cu = cu_draft;
    f.tokens = draft_tokens;
    f.B = B;
    f.G = gamma_max;
    f.V = V;
    f.n_s = ns;
    f.n_draft_rows = n_draft_rows;
    f.n_teams = n_draft_rows + B;
    f.mode = drf ? kFuSample : kFuTokenOnly;
    f.n_slots = f.n_teams + (drf ? n_draft_rows : 0);
    f.k = sp.top_k;
    f.cap = filter_cap(sp.top_k);
    f.top_p = sp.top_p;
    f.c = 1.4426950408889634 / (double)sp.temperature;
    f.inv_t = 1.0 / (double)sp.temperature;
    f.seed = seed;
    f.step = step;
    Carve cv{ws};
    f.cand = cv.take<CandEntry>((size_t)f.n_slots * ns * f.cap * sizeof(CandEntry));
    f.chead = cv.take<CandHead>((size_t)f.n_slots * ns * sizeof(CandHead));
    f.kept = cv.take<KeptEntry>((size_t)f.n_slots * kKeepMax * sizeof(KeptEntry));
    f.rstat = cv.take<RowStat2>((size_t)f.n_slots * sizeof(RowStat2));
    f.out_tokens = out_tokens;
    f.out_num_accepted = out_num_accepted;
    f.out_req_stats = out_req_stats;
    f.out_status = out_status;
    f.st = po;
    // requests the sparse sets cannot hold are recomputed on the dense threshold path
    DenseArrays d;
    const FallbackRows fb = fallback_rows(cv, ws, map, B, n_slots, 2 * (gamma_max + 1), V, sp, 0, d);
    f.ovf_list = (int*)fb.list;
    f.ovf_n = (int*)(ws + kHdrOvfN);
    f.cu_bad0 = (int*)(ws + kHdrCuBad);
    if (launch_filter(f, dtc, vec, st, op.ev0, op.ev1) != hipSuccess) return SPEC_ERR_LAUNCH;
    fa.map = fb.map;
    fa.rs = d.rs;
    fa.part = d.part;
    fa.smass = d.smass;
    fa.amass = d.amass;
    fa.kmass = d.kmass;
    if (launch_fallback_requests(fb, fa, want_kl ? 1 : 0, dtc, vec, st) != hipSuccess) return SPEC_ERR_LAUNCH;
    return SPEC_OK;
  }
  // filtered calls off the sparse path (top-p alone, a larger k) on a uniform bf16 batch: one
  // threshold per logical row, then the fused path with every logit below its row's threshold
  // masked (a ragged or fp32 batch takes the dense threshold path below)
  const bool masked = filtered && dt == SPEC_BF16 && vec && (int64_t)n_draft_rows == (int64_t)B * gamma_max;
  if ((!filtered || masked) && !want_kl && !op.multi && fused_ok(B, V, gamma_max)) {
    Carve cv{ws};
    const float* thr = nullptr;
    if (masked) {
      int* cu_bad = (int*)(ws + kHdrCuBad);
      if (launch_check_cu(cu_draft, B, gamma_max, n_draft_rows, cu_bad, st) != hipSuccess) return SPEC_ERR_LAUNCH;
      map.cu_bad = cu_bad;
      float* t = cv.take<float>((size_t)(2 * n_slots) * sizeof(float));
      if (launch_threshold(map, dtc, vec, V, 2 * n_slots, sp.top_k, sp.top_p,
                           1.4426950408889634 / (double)sp.temperature, t, st) != hipSuccess)
        return SPEC_ERR_LAUNCH;
      thr = t;
    }
    FusedArgs f;
    memset(&f, 0, sizeof(f));
    f.thr = thr;
    f.tgt = target_logits;
    f.tgt_ld = target_ld;
    f.drf = drf;
    f.drf_ld = draft_ld;
    f.cu = cu_draft;
    f.tokens = draft_tokens;
    f.B = B;
    f.G = gamma_max;
    f.V = V;
    f.n_s = ns;
    f.n_draft_rows = n_draft_rows;
    f.n_teams = n_draft_rows + B;
    f.n_tickets = f.n_teams * ns;
    f.mode = greedy ? kFuGreedy : (drf ? kFuSample : kFuTokenOnly);
    f.want_t_ent = pos_stats.target_entropy_bits != nullptr;
    f.spin_limit = op.spin_limit;
    f.c = exp2_scale(sp);
    f.seed = seed;
    f.step = step;
    f.tag = next_tag();
    f.part = cv.take<uint64_t>((size_t)f.n_teams * ns * 2 * fused_record_bytes());
    f.smass = cv.take<uint64_t>((size_t)f.n_teams * ns * 4 * sizeof(uint64_t));
    f.arrive = cv.take<uint32_t>((size_t)f.n_teams * kMaxMembers * sizeof(uint32_t));
    // every request has G draft rows exactly when the rows number B G (a valid offset array
    // has no request above G): then a team's rows follow from its place
    f.ragged = (int64_t)n_draft_rows == (int64_t)B * gamma_max ? 0 : 1;
    f.ylog = cv.take<float>((size_t)f.n_teams * 2 * sizeof(float));
    f.poll_delay = op.poll_delay;
    {
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
      f.tail_wgs = cus * kFusedWgsPerCu;
    }
    f.poll_pause = op.poll_pause;
    f.out_tokens = out_tokens;
    f.out_num_accepted = out_num_accepted;
    f.out_req_stats = out_req_stats;
    f.out_status = out_status;
    f.st = po;
    const hipError_t e = launch_fused(f, dtc, vec, st, op.ev0, op.ev1);
    return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
  }

  int* cu_bad = (int*)(ws + kHdrCuBad);
  if (launch_check_cu(cu_draft, B, gamma_max, n_draft_rows, cu_bad, st) != hipSuccess) return SPEC_ERR_LAUNCH;
  map.cu_bad = cu_bad;
  Carve cv{ws};
  const DenseArrays d = carve_dense(cv, n_slots, ns);
  DenseLaunch L;
  memset(&L, 0, sizeof(L));
  L.map = map;
  L.dt = dtc;
  L.V = V;
  L.n_slices = ns;
  L.n_slots = n_slots;
  L.c = exp2_scale(sp);
  L.greedy = greedy;
  L.want_argmax = 0;
  L.pair = (!greedy && drf != nullptr) ? 1 : 0;
  L.want_kl = want_kl ? 1 : 0;
  L.vec = vec;
  L.part = d.part;
  L.rs = d.rs;
  L.smass = d.smass;
  L.amass = d.amass;
  L.kmass = d.kmass;
  if (filtered) {
    float* thr = cv.take<float>((size_t)(2 * n_slots) * sizeof(float));
    if (launch_threshold(map, dtc, vec, V, 2 * n_slots, sp.top_k, sp.top_p, 1.4426950408889634 / (double)sp.temperature,
                         thr, st) != hipSuccess)
      return SPEC_ERR_LAUNCH;
    map.thr = thr;
    L.map = map;
  }
  L.rso.enabled = 0;
  L.ev_start = op.ev0;
  L.ev_stop = op.ev1;
  if (launch_dense(L, st) != hipSuccess) return SPEC_ERR_LAUNCH;
  fa.map = map;
  fa.rs = L.rs;
  fa.part = L.part;
  fa.smass = L.smass;
  fa.amass = L.amass;
  fa.kmass = L.kmass;
  if (launch_finalize(fa, L.dt, st) != hipSuccess) return SPEC_ERR_LAUNCH;
  return SPEC_OK;
}

int spec_verify_batch(int B, int V, int gamma_max, spec_dtype dt, const void* target_logits, int64_t target_ld,
                      const void* draft_logits, int64_t draft_ld, const int32_t* draft_tokens, const int32_t* cu_draft,
                      int n_draft_rows, spec_sampling_params sp, uint64_t seed, uint64_t step, int32_t* out_tokens,
                      int32_t* out_num_accepted, spec_pos_stats pos_stats, float* out_req_stats, int32_t* out_status,
                      void* workspace, size_t workspace_bytes, void* hip_stream) {
  return spec_verify_batch_ex(B, V, gamma_max, dt, target_logits, target_ld, draft_logits, draft_ld, draft_tokens,
                              cu_draft, n_draft_rows, sp, seed, step, out_tokens, out_num_accepted, pos_stats,
                              out_req_stats, out_status, workspace, workspace_bytes, hip_stream, nullptr);
}

int spec_row_stats_ex(int R, int V, spec_dtype dt, const void* logits, int64_t ld, spec_sampling_params sp,
                      float* max_logit, int32_t* argmax, float* log_z, float* entropy_bits, float* max_prob,
                      int32_t* kept_count, void* workspace, size_t workspace_bytes, void* hip_stream,
                      const spec_call_options* options) {
  if (R < 0 || V <= 0) return SPEC_ERR_INVALID;
  if (dt != SPEC_F32 && dt != SPEC_BF16) return SPEC_ERR_INVALID;
  if (!opts_valid(options)) return SPEC_ERR_INVALID;
  if (V > kMaxChunks * kChunk) return SPEC_ERR_UNSUPPORTED;
  if (check_params(sp) != SPEC_OK) return SPEC_ERR_INVALID;
  if (R == 0) return SPEC_OK;
  if (!logits || ld < V) return SPEC_ERR_INVALID;
  if ((int64_t)R * 2 > (int64_t)INT32_MAX / 2) return SPEC_ERR_INVALID;
  const size_t need = spec_row_stats_workspace_bytes(R, V, dt, sp);
  if (!workspace || workspace_bytes < need) return SPEC_ERR_WORKSPACE;
  if (((uintptr_t)workspace % kAlign) != 0) return SPEC_ERR_INVALID;
  const Opts op = resolve(options);
  const bool greedy = sp.temperature == 0.f;
  const int ns = n_chunks(V);
  const int dtc = dt == SPEC_BF16 ? kDtBF16 : kDtF32;
  const int vec = aligned16(logits, ld, dt) ? 1 : 0;
  const hipStream_t st = (hipStream_t)hip_stream;
  RowStatsOut rso;
  rso.enabled = 1;
  rso.max_logit = max_logit;
  rso.argmax = argmax;
  rso.log_z = log_z;
  rso.entropy_bits = entropy_bits;
  rso.max_prob = max_prob;
  rso.kept_count = kept_count;

  RowMap map;
  memset(&map, 0, sizeof(map));
  map.tgt = logits;
  map.tgt_ld = ld;
  map.B = R;
  if (filter_on(V, sp) && !op.multi && filter_rows_supported(R, V, sp)) {
    Carve cv{(char*)workspace};
    FilterArgs f = plain_filter_args(R, V, logits, ld, nullptr, 0, sp, cv);
    f.rso = rso;
    // rows the sparse sets cannot hold are recomputed on the dense threshold path
    DenseArrays d;
    FallbackRows fb = fallback_rows(cv, (char*)workspace, map, R, R, 2, V, sp, 1, d);
    fb.rso = rso;
    f.ovf_list = (int*)fb.list;
    f.ovf_n = (int*)((char*)workspace + kHdrOvfN);
    f.cu_bad0 = (int*)((char*)workspace + kHdrCuBad);
    if (launch_filter_rows(f, dtc, vec, 0, st) != hipSuccess) return SPEC_ERR_LAUNCH;
    if (launch_fallback_rows(fb, dtc, vec, st) != hipSuccess) return SPEC_ERR_LAUNCH;
    return SPEC_OK;
  }

  Carve cv{(char*)workspace};
  const DenseArrays d = carve_dense(cv, R, ns);
  DenseLaunch L;
  memset(&L, 0, sizeof(L));
  L.map = map;
  L.dt = dtc;
  L.V = V;
  L.n_slices = ns;
  L.n_slots = R;
  L.c = exp2_scale(sp);
  L.greedy = greedy;
  L.want_argmax = 1;
  L.pair = 0;
  L.vec = vec;
  L.part = d.part;
  L.rs = d.rs;
  L.smass = d.smass;
  L.amass = d.amass;
  L.kmass = d.kmass;
  if (filter_on(V, sp)) {
    float* thr = cv.take<float>((size_t)(2 * R) * sizeof(float));
    if (launch_threshold(map, L.dt, L.vec, V, 2 * R, sp.top_k, sp.top_p, 1.4426950408889634 / (double)sp.temperature,
                         thr, st) != hipSuccess)
      return SPEC_ERR_LAUNCH;
    map.thr = thr;
    L.map = map;
  }
  L.rso = rso;
  L.ev_start = op.ev0;
  L.ev_stop = op.ev1;
  if (launch_dense(L, st) != hipSuccess) return SPEC_ERR_LAUNCH;
  return SPEC_OK;
}

int spec_row_stats(int R, int V, spec_dtype dt, const void* logits, int64_t ld, spec_sampling_params sp,
                   float* max_logit, int32_t* argmax, float* log_z, float* entropy_bits, float* max_prob,
                   int32_t* kept_count, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return spec_row_stats_ex(R, V, dt, logits, ld, sp, max_logit, argmax, log_z, entropy_bits, max_prob, kept_count,
                           workspace, workspace_bytes, hip_stream, nullptr);
}

int spec_residual_sample_ex(int R, int V, spec_dtype dt, const void* p_logits, int64_t p_ld, const void* q_logits,
                            int64_t q_ld, spec_sampling_params sp, const double* uniforms, uint64_t seed,
                            uint64_t step, int32_t* out_token, double* out_mass, int32_t* out_status,
                            void* workspace, size_t workspace_bytes, void* hip_stream,
                            const spec_call_options* options) {
  if (R < 0 || V <= 0) return SPEC_ERR_INVALID;
  if (dt != SPEC_F32 && dt != SPEC_BF16) return SPEC_ERR_INVALID;
  if (!opts_valid(options)) return SPEC_ERR_INVALID;
  if (V > kMaxChunks * kChunk) return SPEC_ERR_UNSUPPORTED;
  if (check_params(sp) != SPEC_OK) return SPEC_ERR_INVALID;
  if (R == 0) return SPEC_OK;
  if (!p_logits || p_ld < V || !out_token || !out_status) return SPEC_ERR_INVALID;
  if (q_logits && q_ld < V) return SPEC_ERR_INVALID;
  if ((int64_t)R * 2 > (int64_t)INT32_MAX / 2) return SPEC_ERR_INVALID;
  const size_t need = spec_residual_sample_workspace_bytes(R, V, dt, sp);
  if (!workspace || workspace_bytes < need) return SPEC_ERR_WORKSPACE;
  if (((uintptr_t)workspace % kAlign) != 0) return SPEC_ERR_INVALID;
  const Opts op = resolve(options);
  const bool greedy = sp.temperature == 0.f;
  const int ns = n_chunks(V);
  const int dtc = dt == SPEC_BF16 ? kDtBF16 : kDtF32;
  const int vec = (aligned16(p_logits, p_ld, dt) && aligned16(q_logits, q_ld, dt)) ? 1 : 0;
  const hipStream_t st = (hipStream_t)hip_stream;

  RowMap map;
  memset(&map, 0, sizeof(map));
  map.tgt = p_logits;
  map.tgt_ld = p_ld;
  map.drf = q_logits;
  map.drf_ld = q_ld;
  map.B = R;
  ResidualArgs ra;
  memset(&ra, 0, sizeof(ra));
  ra.V = V;
  ra.n_slices = ns;
  ra.greedy = greedy;
  ra.c = exp2_scale(sp);
  ra.seed = seed;
  ra.step = step;
  ra.uniforms = uniforms;
  ra.out_token = out_token;
  ra.out_mass = out_mass;
  ra.out_status = out_status;
  if (filter_on(V, sp) && !op.multi && filter_rows_supported(R, V, sp)) {
    Carve cv{(char*)workspace};
    FilterArgs f = plain_filter_args(R, V, p_logits, p_ld, q_logits, q_ld, sp, cv);
    f.uniforms = uniforms;
    f.seed = seed;
    f.step = step;
    f.out_tokens = out_token;
    f.out_mass = out_mass;
    f.out_status = out_status;
    // rows the sparse sets cannot hold are recomputed on the dense threshold path
    DenseArrays d;
    const FallbackRows fb = fallback_rows(cv, (char*)workspace, map, R, R, 2, V, sp, 0, d);
    f.ovf_list = (int*)fb.list;
    f.ovf_n = (int*)((char*)workspace + kHdrOvfN);
    f.cu_bad0 = (int*)((char*)workspace + kHdrCuBad);
    if (launch_filter_rows(f, dtc, vec, 1, st) != hipSuccess) return SPEC_ERR_LAUNCH;
    ra.map = fb.map;
    ra.rs = d.rs;
    ra.part = d.part;
    ra.smass = d.smass;
    if (launch_fallback_residual(fb, ra, d.amass, dtc, vec, st) != hipSuccess) return SPEC_ERR_LAUNCH;
    return SPEC_OK;
  }

  Carve cv{(char*)workspace};
  const DenseArrays d = carve_dense(cv, R, ns);
  DenseLaunch L;
  memset(&L, 0, sizeof(L));
  L.map = map;
  L.dt = dtc;
  L.V = V;
  L.n_slices = ns;
  L.n_slots = R;
  L.c = exp2_scale(sp);
  L.greedy = greedy;
  L.want_argmax = 0;
  L.pair = (!greedy && q_logits != nullptr) ? 1 : 0;
  L.vec = vec;
  L.part = d.part;
  L.rs = d.rs;
  L.smass = d.smass;
  L.amass = d.amass;
  L.kmass = d.kmass;
  if (filter_on(V, sp)) {
    float* thr = cv.take<float>((size_t)(2 * R) * sizeof(float));
    if (launch_threshold(map, L.dt, L.vec, V, 2 * R, sp.top_k, sp.top_p, 1.4426950408889634 / (double)sp.temperature,
                         thr, st) != hipSuccess)
      return SPEC_ERR_LAUNCH;
    map.thr = thr;
    L.map = map;
  }
  L.rso.enabled = 0;
  L.ev_start = op.ev0;
  L.ev_stop = op.ev1;
  if (launch_dense(L, st) != hipSuccess) return SPEC_ERR_LAUNCH;
  ra.map = map;
  ra.rs = L.rs;
  ra.part = L.part;
  ra.smass = L.smass;
  if (launch_residual_finalize(ra, L.dt, st) != hipSuccess) return SPEC_ERR_LAUNCH;
  return SPEC_OK;
}

int spec_residual_sample(int R, int V, spec_dtype dt, const void* p_logits, int64_t p_ld, const void* q_logits,
                         int64_t q_ld, spec_sampling_params sp, const double* uniforms, uint64_t seed,
                         uint64_t step, int32_t* out_token, double* out_mass, int32_t* out_status,
                         void* workspace, size_t workspace_bytes, void* hip_stream) {
  return spec_residual_sample_ex(R, V, dt, p_logits, p_ld, q_logits, q_ld, sp, uniforms, seed, step, out_token,
                                 out_mass, out_status, workspace, workspace_bytes, hip_stream, nullptr);
}

size_t spec_lm_head_workspace_bytes(int R, int V, int D) {
  if (R <= 0 || V <= 0 || D <= 0) return 0;
  const int64_t n_ct = ((int64_t)V + kHeadCols - 1) / kHeadCols;
  return kHeaderBytes + align_up((size_t)R * n_ct * sizeof(HeadRec)) + align_up((size_t)R * sizeof(float));
}

int spec_lm_head_row_stats_ex(int R, int V, int D, const void* hidden, int64_t h_ld, const void* weight,
                              int64_t w_ld, spec_sampling_params sp, const int32_t* tokens, float* max_logit,
                              int32_t* argmax, float* log_z, float* entropy_bits, float* max_prob, float* p_tok,
                              void* workspace, size_t workspace_bytes, void* hip_stream,
                              const spec_call_options* options) {
  if (R < 0 || V <= 0 || D <= 0) return SPEC_ERR_INVALID;
  if (!opts_valid(options)) return SPEC_ERR_INVALID;
  if (check_params(sp) != SPEC_OK) return SPEC_ERR_INVALID;
  if (filter_on(V, sp)) return SPEC_ERR_UNSUPPORTED;
  if (R == 0) return SPEC_OK;
  if (!hidden || !weight || h_ld < D || w_ld < D) return SPEC_ERR_INVALID;
  if (p_tok && !tokens) return SPEC_ERR_INVALID;
  // 16-byte rows: D, the strides and the bases are whole multiples of eight bf16
  if (D % 8 != 0 || h_ld % 8 != 0 || w_ld % 8 != 0 || ((uintptr_t)hidden % 16) != 0 || ((uintptr_t)weight % 16) != 0)
    return SPEC_ERR_UNSUPPORTED;
  // a tile's rows are addressed with 32-bit byte offsets (256 rows x stride x 2 B < 2^31)
  if (h_ld > (1 << 21) || w_ld > (1 << 21)) return SPEC_ERR_UNSUPPORTED;
  const int64_t n_ct = ((int64_t)V + kHeadCols - 1) / kHeadCols;
  if ((int64_t)R * n_ct > (int64_t)INT32_MAX / 2) return SPEC_ERR_INVALID;
  const size_t need = spec_lm_head_workspace_bytes(R, V, D);
  if (!workspace || workspace_bytes < need) return SPEC_ERR_WORKSPACE;
  if (((uintptr_t)workspace % kAlign) != 0) return SPEC_ERR_INVALID;
  const Opts op = resolve(options);
  HeadArgs a;
  memset(&a, 0, sizeof(a));
  a.hidden = hidden;
  a.h_ld = h_ld;
  a.weight = weight;
  a.w_ld = w_ld;
  a.R = R;
  a.V = V;
  a.D = D;
  a.n_ct = (int)n_ct;
  a.greedy = sp.temperature == 0.f ? 1 : 0;
  a.c = exp2_scale(sp);
  a.inv_t = a.greedy ? 0.0 : 1.0 / (double)sp.temperature;
  a.tokens = tokens;
  Carve cv{(char*)workspace};
  a.rec = cv.take<HeadRec>((size_t)R * n_ct * sizeof(HeadRec));
  a.ly = cv.take<float>((size_t)R * sizeof(float));
  a.max_logit = max_logit;
  a.argmax = argmax;
  a.log_z = log_z;
  a.entropy_bits = entropy_bits;
  a.max_prob = max_prob;
  a.p_tok = p_tok;
  const hipError_t e = launch_head(a, (hipStream_t)hip_stream, op.ev0, op.ev1);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}

int spec_lm_head_row_stats(int R, int V, int D, const void* hidden, int64_t h_ld, const void* weight, int64_t w_ld,
                           spec_sampling_params sp, const int32_t* tokens, float* max_logit, int32_t* argmax,
                           float* log_z, float* entropy_bits, float* max_prob, float* p_tok, void* workspace,
                           size_t workspace_bytes, void* hip_stream) {
  return spec_lm_head_row_stats_ex(R, V, D, hidden, h_ld, weight, w_ld, sp, tokens, max_logit, argmax, log_z,
                                   entropy_bits, max_prob, p_tok, workspace, workspace_bytes, hip_stream, nullptr);
}

int spec_select_gamma(int B, const float* req_stats, const float* comp, spec_gamma_mlp w, int32_t* out_gamma,
                      float* out_expected, void* hip_stream) {
  if (B < 0) return SPEC_ERR_INVALID;
  if (B == 0) return SPEC_OK;
  if (!req_stats || !w.w1 || !w.b1 || !w.w2 || !out_gamma) return SPEC_ERR_INVALID;
  const hipError_t e = launch_select_gamma(B, req_stats, comp, w.w1, w.b1, w.w2, w.b2, out_gamma, out_expected,
                                           (hipStream_t)hip_stream);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}

int spec_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* hip_stream) {
  if (bytes < 0 || (bytes > 0 && !buf) || !sink) return SPEC_ERR_INVALID;
  if (bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0) return SPEC_ERR_UNSUPPORTED;
  if (bytes == 0) return SPEC_OK;
  const hipError_t e = launch_stream_read(buf, bytes / 16, sink, (hipStream_t)hip_stream, nullptr, nullptr);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}

int spec_mfma_rate(int mode, int iters, int workgroups, float* sink, void* hip_stream) {
  if (mode < 0 || mode > 2 || iters < 0 || iters > (1 << 20) || workgroups < 0 || workgroups > (1 << 16) || !sink)
    return SPEC_ERR_INVALID;
  if (iters == 0 || workgroups == 0) return SPEC_OK;
  const hipError_t e = launch_mfma_rate(mode, iters, workgroups, sink, (hipStream_t)hip_stream, nullptr, nullptr);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_LAUNCH;
}

}  // extern "C"

// Host stand-ins for the kernel launchers of libspecverify, for a CPU-only build of the C-ABI
// layer (spec_api.hip) under AddressSanitizer and UndefinedBehaviorSanitizer.  No kernel runs:
// each launcher checks that every array the layer carved from the caller's workspace is
// 256-byte aligned and lies inside the workspace, then clears it on the host, so an array that
// reaches past the workspace size the layer reported is a heap overflow for the sanitizer.
// Device pointers of the caller (logits, tokens, outputs) are never touched.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "host_stubs.h"
#include "spec_device.h"
#include "spec_internal.h"

namespace hoststub {
Workspace g_ws = {nullptr, 0};
int g_launches = 0;
int g_errors = 0;

struct Range {
  const char* what;
  const char* lo;
  size_t bytes;
};
std::vector<Range> g_ranges;

int check_disjoint() {
  int bad = 0;
  for (size_t i = 0; i < g_ranges.size(); ++i)
    for (size_t j = i + 1; j < g_ranges.size(); ++j) {
      const Range &a = g_ranges[i], &b = g_ranges[j];
      if (a.lo == b.lo && a.bytes == b.bytes) continue;
      if (a.lo < b.lo + b.bytes && b.lo < a.lo + a.bytes) {
        fprintf(stderr, "carved arrays %s and %s overlap\n", a.what, b.what);
        ++bad;
      }
    }
  g_ranges.clear();
  g_errors += bad;
  return bad;
}

void carved(const char* what, const void* p, size_t bytes, size_t align) {
  if (bytes == 0) return;
  const char* b = (const char*)g_ws.base;
  const char* q = (const char*)p;
  if (q == nullptr || q < b || q + bytes > b + g_ws.bytes) {
    fprintf(stderr, "carved array %s [%p, +%zu) outside the workspace [%p, +%zu)\n", what, p, bytes,
            g_ws.base, g_ws.bytes);
    ++g_errors;
    return;
  }
  if (((uintptr_t)q % align) != 0) {
    fprintf(stderr, "carved array %s at %p is not %zu-byte aligned\n", what, p, align);
    ++g_errors;
  }
  memset((void*)q, 0, bytes);
  g_ranges.push_back({what, q, bytes});
}
}  // namespace hoststub

using hoststub::carved;

namespace specv {

size_t fused_record_bytes() { return 16; }
size_t slice_part_bytes() { return sizeof(SlicePart); }
size_t row_stat_bytes() { return sizeof(RowStat); }

hipError_t launch_fused(const FusedArgs& a, int, int, hipStream_t, hipEvent_t, hipEvent_t) {
  ++hoststub::g_launches;
  carved("fused records", a.part, (size_t)a.n_teams * a.n_s * 2 * 16);
  carved("fused residual masses", a.smass, (size_t)a.n_teams * a.n_s * 4 * sizeof(uint64_t));
  carved("fused arrival flags", a.arrive, (size_t)a.n_teams * kMaxMembers * sizeof(uint32_t));
  carved("fused token logits", a.ylog, (size_t)a.n_teams * 2 * sizeof(float));
  return hipSuccess;
}

hipError_t launch_filter(const FilterArgs& a, int, int, hipStream_t, hipEvent_t, hipEvent_t) {
  ++hoststub::g_launches;
  carved("candidates", a.cand, (size_t)a.n_slots * a.n_s * a.cap * sizeof(CandEntry));
  carved("candidate heads", a.chead, (size_t)a.n_slots * a.n_s * sizeof(CandHead));
  carved("kept sets", a.kept, (size_t)a.n_slots * kKeepMax * sizeof(KeptEntry));
  carved("row statistics", a.rstat, (size_t)a.n_slots * sizeof(RowStat2));
  carved("recompute list", a.ovf_list, (size_t)a.B * sizeof(int));
  carved("recompute count", a.ovf_n, sizeof(int), sizeof(int));     // header fields
  carved("offset flag", a.cu_bad0, sizeof(int), sizeof(int));
  return hipSuccess;
}

hipError_t launch_filter_rows(const FilterArgs& a, int, int, int, hipStream_t) {
  ++hoststub::g_launches;
  carved("candidates", a.cand, (size_t)a.n_slots * a.n_s * a.cap * sizeof(CandEntry));
  carved("candidate heads", a.chead, (size_t)a.n_slots * a.n_s * sizeof(CandHead));
  carved("kept sets", a.kept, (size_t)a.n_slots * kKeepMax * sizeof(KeptEntry));
  carved("row statistics", a.rstat, (size_t)a.n_slots * sizeof(RowStat2));
  carved("recompute list", a.ovf_list, (size_t)a.n_teams * sizeof(int));
  return hipSuccess;
}

hipError_t launch_check_cu(const int32_t*, int, int, int, int* cu_bad, hipStream_t) {
  ++hoststub::g_launches;
  carved("offset flag", cu_bad, sizeof(int), sizeof(int));
  return hipSuccess;
}

hipError_t launch_dense(const DenseLaunch& L, hipStream_t) {
  ++hoststub::g_launches;
  const size_t n_lr = 2 * (size_t)L.n_slots, ns = (size_t)L.n_slices;
  carved("slice partials", L.part, n_lr * ns * sizeof(SlicePart));
  carved("row statistics", L.rs, n_lr * sizeof(RowStat));
  carved("residual masses", L.smass, (size_t)L.n_slots * ns * sizeof(double));
  carved("overlap masses", L.amass, (size_t)L.n_slots * ns * sizeof(double));
  carved("KL sums", L.kmass, (size_t)L.n_slots * ns * 4 * sizeof(double));
  return hipSuccess;
}

hipError_t launch_threshold(const RowMap&, int, int, int, int n_lr, int, float, double, float* thr, hipStream_t) {
  ++hoststub::g_launches;
  carved("thresholds", thr, (size_t)n_lr * sizeof(float));
  return hipSuccess;
}

hipError_t launch_finalize(const FinalizeArgs&, int, hipStream_t) {
  ++hoststub::g_launches;
  return hipSuccess;
}

hipError_t launch_residual_finalize(const ResidualArgs&, int, hipStream_t) {
  ++hoststub::g_launches;
  return hipSuccess;
}

hipError_t launch_fallback_rows(const FallbackRows& f, int, int, hipStream_t) {
  ++hoststub::g_launches;
  const size_t n_lr = (size_t)f.n_lr, ns = (size_t)f.n_slices;
  carved("recompute thresholds", f.thr, n_lr * sizeof(float));
  carved("recompute slice partials", f.part, n_lr * ns * sizeof(SlicePart));
  carved("recompute row statistics", f.rs, n_lr * sizeof(RowStat));
  carved("recompute list", f.list, n_lr / (size_t)f.unit_lr * sizeof(int));
  carved("recompute count", f.list_n, sizeof(int), sizeof(int));
  return hipSuccess;
}

hipError_t launch_fallback_requests(const FallbackRows& f, const FinalizeArgs& a, int, int, int, hipStream_t) {
  launch_fallback_rows(f, 0, 0, nullptr);   // the same kernel recomputes the listed rows
  const size_t n_slots = (size_t)f.n_lr / 2, ns = (size_t)f.n_slices;
  carved("recompute residual masses", a.smass, n_slots * ns * sizeof(double));
  carved("recompute overlap masses", a.amass, n_slots * ns * sizeof(double));
  carved("recompute KL sums", a.kmass, n_slots * ns * 4 * sizeof(double));
  return hipSuccess;
}

hipError_t launch_fallback_residual(const FallbackRows& f, const ResidualArgs& a, double* amass, int, int,
                                    hipStream_t) {
  launch_fallback_rows(f, 0, 0, nullptr);   // the same kernel recomputes the listed rows
  const size_t n_slots = (size_t)f.n_lr / 2, ns = (size_t)f.n_slices;
  carved("recompute residual masses", a.smass, n_slots * ns * sizeof(double));
  carved("recompute overlap masses", amass, n_slots * ns * sizeof(double));
  return hipSuccess;
}

hipError_t launch_select_gamma(int, const float*, const float*, const float*, const float*, const float*, float,
                               int32_t*, float*, hipStream_t) {
  ++hoststub::g_launches;
  return hipSuccess;
}

hipError_t launch_stream_read(const void*, int64_t, uint32_t*, hipStream_t, hipEvent_t, hipEvent_t) {
  ++hoststub::g_launches;
  return hipSuccess;
}

hipError_t launch_mfma_rate(int, int, int, float*, hipStream_t, hipEvent_t, hipEvent_t) {
  ++hoststub::g_launches;
  return hipSuccess;
}

hipError_t launch_head(const HeadArgs& a, hipStream_t, hipEvent_t, hipEvent_t) {
  ++hoststub::g_launches;
  carved("head records", a.rec, (size_t)a.R * a.n_ct * sizeof(HeadRec));
  carved("token logits", a.ly, (size_t)a.R * sizeof(float));
  return hipSuccess;
}

}  // namespace specv

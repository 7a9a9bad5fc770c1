// Drives every C entry point of libspecverify's host layer with the kernel launchers replaced by
// host stand-ins (host_stubs.cpp), built for the CPU under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Valid calls get a host workspace of exactly the size the
// *_workspace_bytes function reports, so every carved array the stand-ins clear must fit it;
// invalid calls must return their documented code without launching anything.  Exits 0 when
// every check holds; the sanitizers abort on a memory or arithmetic fault.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "host_stubs.h"
#include "spec_verify.h"

namespace {

int g_fail = 0;
#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      fprintf(stderr, "FAIL line %d: ", __LINE__);        \
      fprintf(stderr, __VA_ARGS__);                       \
      fprintf(stderr, "\n");                              \
      ++g_fail;                                           \
    }                                                     \
  } while (0)

// Any non-null address stands for a caller's device array: the layer never reads through it.
void* const kDev = (void*)0x100000;

struct HostWs {
  void* p = nullptr;
  size_t n = 0;
  explicit HostWs(size_t bytes) : n(bytes) {
    if (bytes && posix_memalign(&p, 256, bytes) != 0) p = nullptr;
    hoststub::g_ws = {p, bytes};
  }
  ~HostWs() { free(p); }
};

spec_sampling_params params(float t, int k, float p) {
  spec_sampling_params s;
  s.temperature = t;
  s.top_k = k;
  s.top_p = p;
  return s;
}

// One spec_verify_batch call of B requests with gamma_max G (uniform or ragged row count).
void verify(const char* what, int B, int V, int G, int n_draft_rows, spec_sampling_params sp, bool draft,
            const spec_call_options* opt) {
  const size_t need = spec_verify_workspace_bytes(B, V, G, SPEC_BF16, sp);
  HostWs ws(need);
  spec_pos_stats ps;
  memset(&ps, 0, sizeof(ps));
  ps.one_minus_tv = (float*)kDev;
  const int before = hoststub::g_launches;
  const int rc = spec_verify_batch_ex(B, V, G, SPEC_BF16, kDev, V, draft ? kDev : nullptr, V, (int32_t*)kDev,
                                      (int32_t*)kDev, n_draft_rows, sp, 1, 2, (int32_t*)kDev, (int32_t*)kDev, ps,
                                      nullptr, (int32_t*)kDev, ws.p, ws.n, nullptr, opt);
  CHECK(rc == SPEC_OK, "%s: rc %d", what, rc);
  CHECK(hoststub::g_launches > before, "%s: nothing launched", what);
  CHECK(hoststub::check_disjoint() == 0, "%s: carved arrays overlap", what);
  // one byte short is refused before any launch
  const int mid = hoststub::g_launches;
  const int rc2 = spec_verify_batch_ex(B, V, G, SPEC_BF16, kDev, V, draft ? kDev : nullptr, V, (int32_t*)kDev,
                                       (int32_t*)kDev, n_draft_rows, sp, 1, 2, (int32_t*)kDev, (int32_t*)kDev, ps,
                                       nullptr, (int32_t*)kDev, ws.p, ws.n - 1, nullptr, opt);
  CHECK(rc2 == SPEC_ERR_WORKSPACE && hoststub::g_launches == mid, "%s: short workspace rc %d", what, rc2);
}

void row_stats(const char* what, int R, int V, spec_sampling_params sp, const spec_call_options* opt) {
  const size_t need = spec_row_stats_workspace_bytes(R, V, SPEC_BF16, sp);
  HostWs ws(need);
  const int rc = spec_row_stats_ex(R, V, SPEC_BF16, kDev, V, sp, (float*)kDev, (int32_t*)kDev, nullptr, nullptr,
                                   nullptr, (int32_t*)kDev, ws.p, ws.n, nullptr, opt);
  CHECK(rc == SPEC_OK, "%s: rc %d", what, rc);
  CHECK(hoststub::check_disjoint() == 0, "%s: carved arrays overlap", what);
}

void residual(const char* what, int R, int V, spec_sampling_params sp, bool q, const spec_call_options* opt) {
  const size_t need = spec_residual_sample_workspace_bytes(R, V, SPEC_BF16, sp);
  HostWs ws(need);
  const int rc = spec_residual_sample_ex(R, V, SPEC_BF16, kDev, V, q ? kDev : nullptr, V, sp, nullptr, 3, 4,
                                         (int32_t*)kDev, (double*)kDev, (int32_t*)kDev, ws.p, ws.n, nullptr, opt);
  CHECK(rc == SPEC_OK, "%s: rc %d", what, rc);
  CHECK(hoststub::check_disjoint() == 0, "%s: carved arrays overlap", what);
}

}  // namespace

int main() {
  const int Q3 = 151936, L3 = 128256;
  spec_call_options multi;
  memset(&multi, 0, sizeof(multi));
  multi.path = SPEC_PATH_MULTI_KERNEL;
  multi.spin_limit = -1;

  // the five workloads' shapes on their default paths, and on the multi-kernel path
  for (int m = 0; m < 2; ++m) {
    const spec_call_options* o = m ? &multi : nullptr;
    verify("tiny fp32-shaped", 1, 8, 4, 4, params(1.f, 0, 1.f), true, o);
    verify("batch 64, gamma 7", 64, Q3, 7, 64 * 7, params(1.f, 0, 1.f), true, o);
    verify("batch 128 ragged", 128, L3, 8, 640, params(0.7f, 0, 1.f), true, o);
    verify("greedy batch 256", 256, Q3, 7, 256 * 7, params(0.f, 0, 1.f), false, o);
    verify("top-k 50, top-p 0.9, batch 256", 256, Q3, 7, 256 * 7, params(0.7f, 50, 0.9f), true, o);
    verify("top-p alone", 32, Q3, 7, 32 * 7, params(0.7f, 0, 0.9f), true, o);
    verify("top-k 600", 16, Q3, 7, 16 * 7, params(0.7f, 600, 1.f), true, o);
    verify("token-only draft", 16, Q3, 7, 16 * 7, params(1.f, 0, 1.f), false, o);
    verify("filtered token-only draft", 16, Q3, 7, 16 * 7, params(0.7f, 50, 1.f), false, o);
    verify("gamma 0", 8, 5000, 0, 0, params(1.f, 0, 1.f), true, o);
    verify("beyond the single-kernel limits", 1100, 5000, 3, 1100 * 3, params(1.f, 0, 1.f), true, o);
    verify("vocabulary beyond 64 slices", 4, 300000, 3, 12, params(1.f, 0, 1.f), true, o);
    row_stats("row stats", 40, Q3, params(1.f, 0, 1.f), o);
    row_stats("row stats top-k", 40, Q3, params(0.7f, 50, 0.9f), o);
    row_stats("row stats top-p", 40, Q3, params(0.7f, 0, 0.9f), o);
    row_stats("row stats greedy", 40, Q3, params(0.f, 0, 1.f), o);
    residual("residual with q", 40, Q3, params(0.7f, 0, 1.f), true, o);
    residual("residual top-k with q", 40, Q3, params(0.7f, 50, 0.9f), true, o);
    residual("residual top-k without q", 40, Q3, params(0.7f, 50, 0.9f), false, o);
    residual("residual top-p", 40, Q3, params(0.7f, 0, 0.8f), true, o);
  }

  // the fused head
  {
    const size_t need = spec_lm_head_workspace_bytes(512, Q3, 4096);
    HostWs ws(need);
    const int rc = spec_lm_head_row_stats(512, Q3, 4096, kDev, 4096, kDev, 4096, params(1.f, 0, 1.f), (int32_t*)kDev,
                                          (float*)kDev, (int32_t*)kDev, nullptr, nullptr, nullptr, (float*)kDev, ws.p,
                                          ws.n, nullptr);
    CHECK(rc == SPEC_OK, "lm head rc %d", rc);
    CHECK(hoststub::check_disjoint() == 0, "lm head: carved arrays overlap");
  }

  // invalid calls: refused with their documented code, nothing launched
  {
    HostWs ws(1 << 20);
    spec_pos_stats ps;
    memset(&ps, 0, sizeof(ps));
    const int before = hoststub::g_launches;
    spec_call_options bad = multi;
    bad.path = 9;
    CHECK(spec_verify_batch_ex(2, 100, 3, SPEC_BF16, kDev, 100, kDev, 100, (int32_t*)kDev, (int32_t*)kDev, 6,
                               params(1.f, 0, 1.f), 0, 0, (int32_t*)kDev, (int32_t*)kDev, ps, nullptr,
                               (int32_t*)kDev, ws.p, ws.n, nullptr, &bad) == SPEC_ERR_INVALID,
          "unknown path accepted");
    CHECK(spec_verify_batch(2, 100, 3, SPEC_BF16, kDev, 99, kDev, 100, (int32_t*)kDev, (int32_t*)kDev, 6,
                            params(1.f, 0, 1.f), 0, 0, (int32_t*)kDev, (int32_t*)kDev, ps, nullptr, (int32_t*)kDev,
                            ws.p, ws.n, nullptr) == SPEC_ERR_INVALID,
          "short row stride accepted");
    CHECK(spec_verify_batch(2, 100, 3, SPEC_BF16, kDev, 100, kDev, 100, (int32_t*)kDev, (int32_t*)kDev, 7,
                            params(1.f, 0, 1.f), 0, 0, (int32_t*)kDev, (int32_t*)kDev, ps, nullptr, (int32_t*)kDev,
                            ws.p, ws.n, nullptr) == SPEC_ERR_INVALID,
          "more draft rows than B gamma_max accepted");
    CHECK(spec_verify_batch(2, 100, 3, SPEC_BF16, kDev, 100, kDev, 100, (int32_t*)kDev, (int32_t*)kDev, 6,
                            params(NAN, 0, 1.f), 0, 0, (int32_t*)kDev, (int32_t*)kDev, ps, nullptr, (int32_t*)kDev,
                            ws.p, ws.n, nullptr) == SPEC_ERR_INVALID,
          "NaN temperature accepted");
    CHECK(spec_verify_batch(2, 100, 3, SPEC_BF16, kDev, 100, kDev, 100, (int32_t*)kDev, (int32_t*)kDev, 6,
                            params(1.f, 0, 1.f), 0, 0, (int32_t*)kDev, (int32_t*)kDev, ps, nullptr, (int32_t*)kDev,
                            (char*)ws.p + 16, ws.n - 16, nullptr) == SPEC_ERR_INVALID,
          "misaligned workspace accepted");
    CHECK(spec_row_stats(3, 100, SPEC_BF16, kDev, 100, params(1.f, 0, 0.f), nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr, ws.p, ws.n, nullptr) == SPEC_ERR_INVALID,
          "top_p 0 accepted");
    CHECK(spec_residual_sample(3, 100, SPEC_BF16, nullptr, 100, nullptr, 0, params(1.f, 0, 1.f), nullptr, 0, 0,
                               (int32_t*)kDev, nullptr, (int32_t*)kDev, ws.p, ws.n, nullptr) == SPEC_ERR_INVALID,
          "null p rows accepted");
    CHECK(hoststub::g_launches == before, "an invalid call launched");
  }

  CHECK(hoststub::g_errors == 0, "%d carved arrays outside the workspace or misaligned", hoststub::g_errors);
  printf("host layer: %d launches checked, %d failures\n", hoststub::g_launches, g_fail);
  return g_fail == 0 ? 0 : 1;
}

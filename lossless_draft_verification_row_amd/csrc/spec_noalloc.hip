// spec_noalloc.hip -- spec_verify_batch for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  The call's
// workspace is a static device array of the library, one copy per GPU, held until the process
// ends; the caller passes only inputs and outputs.
#include <mutex>

#include "spec_device.h"
#include "spec_internal.h"
#include "spec_verify.h"

// The scratch array.  In host code `scratch` is a stand-in for the device symbol, not a device
// address: host code uses only the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[SPEC_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // per device: the device address of its copy of `scratch`

// Clears one device's scratch (records tagged by earlier calls must not exist before the first).
__global__ __launch_bounds__(specv::kThreads) void k_zero_scratch(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * specv::kThreads + threadIdx.x; i < n16; i += (size_t)gridDim.x * specv::kThreads)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The current device's scratch address, set up on the first call on that device: the symbol's
// address for this device, then one clearing kernel on the caller's stream (stream-ordered
// before that call's own kernels).  Returns nullptr if the device or the symbol cannot be had.
void* scratch_for_current_device(hipStream_t st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    hipLaunchKernelGGL(k_zero_scratch, dim3(1024), dim3(specv::kThreads), 0, st, (uint4*)ptr,
                       (size_t)SPEC_NOALLOC_SCRATCH_BYTES / 16);
    if (hipGetLastError() != hipSuccess) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

int spec_verify_batch_noalloc(int B, int V, int gamma_max, spec_dtype dt, const void* target_logits,
                              int64_t target_ld, const void* draft_logits, int64_t draft_ld,
                              const int32_t* draft_tokens, const int32_t* cu_draft, int n_draft_rows,
                              spec_sampling_params sp, uint64_t seed, uint64_t step, int32_t* out_tokens,
                              int32_t* out_num_accepted, spec_pos_stats pos_stats, float* out_req_stats,
                              int32_t* out_status, void* hip_stream) {
  if (B < 0 || V <= 0 || gamma_max < 0) return SPEC_ERR_INVALID;
  if (B == 0) return SPEC_OK;
  if (spec_verify_workspace_bytes(B, V, gamma_max, dt, sp) > (size_t)SPEC_NOALLOC_SCRATCH_BYTES)
    return SPEC_ERR_SCRATCH_LIMIT;
  void* ws = scratch_for_current_device((hipStream_t)hip_stream);
  if (ws == nullptr) return SPEC_ERR_LAUNCH;
  return spec_verify_batch(B, V, gamma_max, dt, target_logits, target_ld, draft_logits, draft_ld, draft_tokens,
                           cu_draft, n_draft_rows, sp, seed, step, out_tokens, out_num_accepted, pos_stats,
                           out_req_stats, out_status, ws, (size_t)SPEC_NOALLOC_SCRATCH_BYTES, hip_stream);
}

}  // extern "C"

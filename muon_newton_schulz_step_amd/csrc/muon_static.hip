// muon_step_static: the Muon step for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Its scratch is `scratch` below, a fixed area of
// MUON_STATIC_SCRATCH_BYTES that every GPU the library runs on holds from
// module load until the process ends; the entry point itself allocates
// nothing and otherwise runs exactly muon_step (same checks, same kernels).
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per GPU, with that GPU current, and only
// that address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "muon.h"
#include "muon_kernels.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MUON_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device address of the current GPU's `scratch`, looked up on the first
// call on that GPU (with it current) and kept.
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MUON_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MUON_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MUON_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MUON_OK;
}

// Workspace source of the static entry point: refuses steps that need more
// than the fixed area, before anything is enqueued.
int static_workspace(const void*, size_t need, void** ws, size_t* bytes) {
  if (need > (size_t)MUON_STATIC_SCRATCH_BYTES) return MUON_ERR_WORKSPACE;
  if (int st = current_scratch(ws)) return st;
  *bytes = (size_t)MUON_STATIC_SCRATCH_BYTES;
  return MUON_OK;
}

}  // namespace

extern "C" int muon_step_static(int n, const int* rows, const int* cols, void* const* params,
                                int param_dtype, const void* const* grads, int grad_dtype,
                                float* const* momentum, float mu, float lr, const float* scale,
                                const muon_coeff* coeffs, int n_steps, float eps, int compute,
                                hipStream_t stream) {
  const muon::WorkspaceSource src{static_workspace, nullptr};
  return muon::step_with_source(n, rows, cols, params, param_dtype, grads, grad_dtype, momentum,
                                mu, lr, scale, coeffs, n_steps, eps, compute, src, stream);
}

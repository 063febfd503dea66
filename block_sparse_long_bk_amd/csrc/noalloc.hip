// noalloc.hip -- msa_forward_noalloc: the whole forward on a scratch area the
// library owns, for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array of MSA_NOALLOC_SCRATCH_BYTES.
// In host code its name only stands in for the symbol: the device address of
// each GPU's copy comes from hipGetSymbolAddress, looked up once per device
// (with that device current) and kept; only that address is handed on.  The
// forward needs no scratch contents to start at zero, so nothing is cleared.
#include <hip/hip_runtime.h>

#include <mutex>

#include "msa.h"
#include "msa_internal.h"

namespace {

static_assert(MSA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size in whole 256-byte lines");
static __device__ __align__(256) char scratch[MSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, or an error.
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" msa_status_t msa_forward_noalloc(const msa_problem_t* prob, const void* q, const void* k, const void* v,
                                            const void* idx_q, const void* idx_k, int32_t* block_ids, void* out,
                                            float* lse, void* stream) {
  // Everything that can be checked without the GPU is checked first.
  msa_status_t rc = msa_validate(prob);
  if (rc != MSA_OK) return rc;
  size_t full = 0, least = 0;
  rc = msa_workspace_size(prob, MSA_OP_FORWARD, &full, &least);
  if (rc != MSA_OK) return rc;
  if (least > (size_t)MSA_NOALLOC_SCRATCH_BYTES) return MSA_ERR_WORKSPACE;
  if (!q || !k || !v || !idx_q || !idx_k || !block_ids || !out) return MSA_ERR_INVALID_ARG;
  void* ws = nullptr;
  const hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) return static_cast<msa_status_t>(msa::record_hip_error(e));
  return msa_forward(prob, q, k, v, idx_q, idx_k, block_ids, out, lse, ws, (size_t)MSA_NOALLOC_SCRATCH_BYTES, stream);
}

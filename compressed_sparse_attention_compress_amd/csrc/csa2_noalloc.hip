// csa2_score_topk_noalloc: csa2_score_topk with its scratch in a fixed device
// array of this library instead of a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops).
//
// The array is a file-scope __device__ variable: every GPU the library runs on
// holds its own copy until the process ends.  Host code never passes the
// variable's name to a kernel (on the host it is only a stand-in); its device
// address is looked up once per device with hipGetSymbolAddress, with that device
// current, and that address is what the score kernels receive.  Calls on one GPU
// share the array, so calls that overlap on one GPU (different streams, or
// different host threads) race.  The score kernels write every scratch byte they
// read, so nothing has to be cleared between calls.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "csa2.h"
#include "csa2_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[CSA2_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

// The scratch array's device address on the current device (looked up once).
hipError_t scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" csa2_status csa2_score_topk_noalloc(csa2_runtime* rt, const csa2_score_topk_args* a, csa2_stream stream) {
  if (a == nullptr) return csa2::set_error(CSA2_ERR_INVALID_ARG, "csa2_score_topk_noalloc: args is NULL");
  if (a->workspace != nullptr || a->workspace_bytes != 0)
    return csa2::set_error(CSA2_ERR_INVALID_ARG,
                           "csa2_score_topk_noalloc: takes no workspace (workspace must be NULL and workspace_bytes 0)");
  size_t need = 0;
  csa2_status s = csa2::score_topk_plan(rt, a, &need);
  if (s != CSA2_OK) return s;
  if (need > (size_t)CSA2_NOALLOC_SCRATCH_BYTES) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "csa2_score_topk_noalloc: this call needs %zu bytes of scratch, more than the %zu the library holds "
             "(use csa2_score_topk with a workspace)",
             need, (size_t)CSA2_NOALLOC_SCRATCH_BYTES);
    return csa2::set_error(CSA2_ERR_WORKSPACE, msg);
  }
  void* ptr = nullptr;
  const hipError_t e = scratch_for_current_device(&ptr);
  if (e != hipSuccess) {
    char msg[256];
    snprintf(msg, sizeof(msg), "csa2_score_topk_noalloc: scratch address lookup failed: %s", hipGetErrorString(e));
    return csa2::set_error(CSA2_ERR_HIP, msg);
  }
  csa2_score_topk_args b = *a;
  b.workspace = ptr;
  b.workspace_bytes = CSA2_NOALLOC_SCRATCH_BYTES;
  return csa2_score_topk(rt, &b, stream);
}

// noalloc.hip -- the Markov draft for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that
// forbid hipMalloc): dspark_draft_markov_noalloc.
//
// Same kernels and results as dspark_draft_markov.  The draft's scratch (the
// status word, the per-chunk statistics, the grid-barrier flags and the
// per-slice records) lives in one file-scope device array of kScratchBytes,
// which every GPU the library runs on holds until the process ends.  Host
// code never passes the array's name to a kernel (on the host it is only a
// stand-in symbol): the array's device address is looked up once per device
// with hipGetSymbolAddress and kept, and only that address is used.
#include "dspark.h"

#include <cmath>
#include <mutex>

#include "launch.hpp"
#include "workspace.hpp"

namespace dspark {
namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;   // DSPARK_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == DSPARK_NOALLOC_SCRATCH_BYTES, "header and library agree");
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scr_mu;
void* g_scr_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up once per device).
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scr_mu);
  if (g_scr_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scr_ptr[dev] = p;
  }
  *out = g_scr_ptr[dev];
  return hipSuccess;
}

__global__ void k_word_set(uint32_t* p, uint32_t v) {
  if (threadIdx.x == 0) *p = v;
}
__global__ void k_word_copy(uint32_t* dst, const uint32_t* src) {
  if (threadIdx.x == 0) *dst = *src;
}

}  // namespace
}  // namespace dspark

using namespace dspark;

extern "C" dspark_status dspark_draft_markov_noalloc(int R, int gamma, int V, int r, float T,
                                                     uint64_t seed, uint64_t round, const void* U,
                                                     dspark_dtype U_dt, const void* W1,
                                                     const void* W2t, dspark_dtype W_dt,
                                                     const int32_t* x0, int32_t* x, float* logp_d,
                                                     float* lse_d, float* margin, uint32_t* flags,
                                                     hipStream_t stream) {
  DSPARK_ABI_RANGE();
  if (R < 0 || gamma < 1 || V < 1) return DSPARK_E_INVALID;
  if (gamma > 32) return DSPARK_E_UNSUPPORTED;
  if (r < 0) return DSPARK_E_INVALID;
  if (r > 512 || (r % 16) != 0) return DSPARK_E_UNSUPPORTED;
  if (!(T >= 0.f) || !std::isfinite(T)) return DSPARK_E_INVALID;
  if ((U_dt != DSPARK_F32 && U_dt != DSPARK_BF16) || (W_dt != DSPARK_F32 && W_dt != DSPARK_BF16))
    return DSPARK_E_INVALID;
  if (R == 0) return DSPARK_OK;
  if (!U || !x0 || !x || !logp_d || !lse_d) return DSPARK_E_INVALID;
  if (r > 0 && (!W1 || !W2t)) return DSPARK_E_INVALID;
  if (r > 0 && (((reinterpret_cast<uintptr_t>(W1) | reinterpret_cast<uintptr_t>(W2t)) & 15) != 0))
    return DSPARK_E_UNSUPPORTED;
  if (draft_ws_compact(nullptr, R, V, nullptr) > kScratchBytes) return DSPARK_E_WORKSPACE;
  void* base = nullptr;
  if (scratch_ptr(&base) != hipSuccess) return DSPARK_E_HIP;
  DraftWs ws;
  draft_ws_compact(reinterpret_cast<char*>(base), R, V, &ws);
  // the status word starts at zero for this call (a kernel, not a memset, so
  // that the call can be captured into a graph)
  hipLaunchKernelGGL(k_word_set, dim3(1), dim3(64), 0, stream, ws.status, 0u);
  if (hipGetLastError() != hipSuccess) return DSPARK_E_HIP;
  if (launch_draft(R, gamma, V, r, T, seed, round, U, U_dt == DSPARK_BF16, W1, W2t,
                   W_dt == DSPARK_BF16, x0, x, logp_d, lse_d, margin, ws, stream) != hipSuccess)
    return DSPARK_E_HIP;
  if (flags) {
    hipLaunchKernelGGL(k_word_copy, dim3(1), dim3(64), 0, stream, flags, ws.status);
    if (hipGetLastError() != hipSuccess) return DSPARK_E_HIP;
  }
  return DSPARK_OK;
}

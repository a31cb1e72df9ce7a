// kvsel_select_static: kvsel_select with its scratch memory in a static
// device array instead of a caller's workspace, for callers that cannot
// allocate (code under graph capture, tight serving loops).
//
// `scratch` is a file-scope __device__ array; every GPU the library runs
// on holds one copy of it until the process ends. In host code the name
// `scratch` is only a host-side stand-in, never a device address: the
// entry point looks up each device's copy once, with hipGetSymbolAddress
// while that device is current, and passes that address to the kernels.
// Every call on one GPU shares that GPU's copy, so calls that overlap on a
// GPU (other streams, other threads) race; the selection kernels clear
// what must start at zero at the start of each call.
#include <cmath>
#include <mutex>

#include "kvsel.h"
#include "kvsel_kernels.h"

namespace kvsel {

constexpr size_t kStaticScratchBytes = size_t(16) << 20;   // 16 MiB per GPU

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's copy of `scratch`.
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace kvsel

using namespace kvsel;

extern "C" {

size_t kvsel_static_scratch_bytes(void) { return kStaticScratchBytes; }

int32_t kvsel_select_static(const float* scores, const float* weight, int32_t L, int32_t H_kv,
                            int32_t n, int32_t W, int64_t budget, int32_t adaptive,
                            float score_norm, float eps, float alpha, int32_t* idx,
                            int32_t* head_offsets, uint8_t* stage, void* stream) {
  SelectPlan p;
  const int32_t rc = select_plan(weight != nullptr, L, H_kv, n, W, budget, adaptive, score_norm,
                                 eps, alpha, &p);
  if (rc != KVSEL_OK) return rc;
  if (select_ws_bytes(p) > kStaticScratchBytes) return KVSEL_ERR_SCRATCH;
  const int32_t rp = select_pointers_ok(p, scores, weight, idx, head_offsets);
  if (rp != KVSEL_OK) return rp;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return KVSEL_ERR_HIP;
  const hipError_t e = select_launch(p, scores, weight, idx, head_offsets, stage, ws,
                                     static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KVSEL_OK : KVSEL_ERR_HIP;
}

}  // extern "C"

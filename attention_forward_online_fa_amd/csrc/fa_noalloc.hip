// fa_fwd_noalloc: the forward pass of fa_fwd_ex without any device memory
// allocation, for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc). Declared in
// include/fa.h.
//
// The only scratch memory the forward pass needs is the key-split workspace
// (fp32 partial outputs and log-sum-exps that the merge kernel combines).
// Here it lives in one static device array per GPU, fixed at
// FA_NOALLOC_SCRATCH_BYTES and held until the process ends. Its device
// address is looked up once per device, with that device current, and only
// that address is handed to the kernels: in host code the array's own name is
// a host-side stand-in, not a device address.
//
// Nothing in the array needs to start at zero: every partial log-sum-exp of a
// launch is written by that launch, and the merge reads a partial output only
// where its log-sum-exp is finite, i.e. where the same launch wrote it. All
// calls on one GPU share its array, so calls that overlap on one GPU (on
// different streams, or from different threads) race; calls queued in order
// on one stream do not.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_kernels.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

std::mutex g_mu;
void* g_ptr[kMaxDevices];   // device address of `scratch` on each device (null = not looked up)

// The current device's address of `scratch`, looked up on the first call on
// that device.
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA_ERR_HIP;
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_fwd_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE,
                              int B, int H, int HKV, int Sq, int Sk, int D, float scale,
                              int causal, int window, int dtype, int num_splits, void* stream) {
  // scratch_address runs after the argument checks, so argument errors come
  // back before any HIP call, as from fa_fwd_ex
  return fa::forward_fixed_workspace(Q, K, V, O, LSE, B, H, HKV, Sq, Sk, D, scale, causal, window,
                                     dtype, num_splits, stream,
                                     fa::FixedWorkspace{scratch_address, FA_NOALLOC_SCRATCH_BYTES});
}

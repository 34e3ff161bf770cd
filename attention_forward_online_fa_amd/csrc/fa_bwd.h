// Internal interface between the backward C ABI (fa_bwd_api.cpp) and its
// kernels (fa_bwd.hip). Not installed; callers use include/fa.h.
#pragma once
#include <hip/hip_runtime.h>

namespace fa {

struct BwdParams {
  const void* Q;      // [B, H, Sq, D] input type
  const void* K;      // [B, HKV, Sk, D]
  const void* V;      // [B, HKV, Sk, D]
  const void* O;      // [B, H, Sq, D]   forward output
  const void* dO;     // [B, H, Sq, D]   gradient of the loss with respect to O
  const float* LSE;   // [B, H, Sq]      forward log-sum-exp (natural log)
  float* dQ;          // [B, H, Sq, D]   fp32 (written)
  float* dK;          // [B, HKV, Sk, D] fp32 (written)
  float* dV;          // [B, HKV, Sk, D] fp32 (written)
  float* Dws;         // [B, H, Sq]      workspace: D_i = dO_i . O_i
  int B, H, HKV, Sq, Sk;
  float scale;
  int causal, window;
  // MFMA dQ kernel (16-bit inputs): |scale| log2(e) (at least 1e-30, so a
  // masked score of -inf stays -inf) with Q negated when scale < 0, and the
  // number of 128-row query tiles
  float sl_abs;
  int neg_q;
  int n_qblk;
};

// Queue the dQ kernel (which also writes Dws) and then the dK/dV kernel.
hipError_t launch_backward(const BwdParams& p, int dtype, int D, hipStream_t stream);

}  // namespace fa

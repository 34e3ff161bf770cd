// C ABI of the backward pass: argument checks, the D_i workspace and the
// launch. Declared in include/fa.h (fa_bwd).
#include "fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "fa_bwd.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_bwd(int B, int H, int HKV, int Sq, int Sk, int D, int causal, int window, int dtype) {
  if (B < 1 || H < 1 || HKV < 1 || Sq < 1 || Sk < 1 || D < 1) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_DTYPE;
  if (D != 16 && D != 32 && D != 48 && D != 64 && D != 80 && D != 96 && D != 128 && D != 256)
    return FA_ERR_HEAD_DIM;
  if (H % HKV != 0) return FA_ERR_GQA;
  if (window < 0 || (causal != 0 && causal != 1)) return FA_ERR_WINDOW;
  // every row index (b H + h) Sq + i and element offset is formed in 64 bits;
  // keep the row counts inside int range as the forward does
  if ((double)B * H * Sq >= 2147483647.0 || (double)B * HKV * Sk >= 2147483647.0)
    return FA_ERR_SHAPE;
  if ((double)B * H * Sq * D * 4 > 4.0e18 || (double)B * HKV * Sk * D * 4 > 4.0e18)
    return FA_ERR_SHAPE;
  return FA_OK;
}

}  // namespace

extern "C" int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                      const float* LSE, float* dQ, float* dK, float* dV, int B, int H, int HKV,
                      int Sq, int Sk, int D, float scale, int causal, int window, int dtype,
                      void* stream_ptr) {
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return FA_ERR_NULLPTR;
  const int st = check_bwd(B, H, HKV, Sq, Sk, D, causal, window, dtype);
  if (st != FA_OK) return st;
  for (const void* p : {Q, K, V, O, dO, (const void*)LSE, (const void*)dQ, (const void*)dK,
                        (const void*)dV})
    if (!aligned16(p)) return FA_ERR_ALIGN;

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  fa::BwdParams p = {};
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.dO = dO;
  p.LSE = LSE;
  p.dQ = dQ;
  p.dK = dK;
  p.dV = dV;
  p.B = B;
  p.H = H;
  p.HKV = HKV;
  p.Sq = Sq;
  p.Sk = Sk;
  p.scale = scale;
  p.causal = causal;
  p.window = window;
  p.neg_q = scale < 0.f ? 1 : 0;
  const double mag = std::fabs((double)scale) * 1.4426950408889634;
  p.sl_abs = mag > 1e-30 ? (float)mag : 1e-30f;
  p.n_qblk = (Sq + 127) / 128;
  if ((double)B * H * p.n_qblk > 2147483647.0) return FA_ERR_SHAPE;
  // D_i workspace, stream-ordered from the device's default memory pool
  void* ws = nullptr;
  if (hipMallocAsync(&ws, (size_t)B * H * Sq * sizeof(float), stream) != hipSuccess)
    return FA_ERR_WORKSPACE;
  p.Dws = static_cast<float*>(ws);
  const hipError_t e = fa::launch_backward(p, dtype, D, stream);
  const hipError_t f = hipFreeAsync(ws, stream);
  return (e == hipSuccess && f == hipSuccess) ? FA_OK : FA_ERR_HIP;
}

// Backward pass of the fused attention (gradients of sum(O * dO) with
// respect to Q, K and V) for gfx950, in the per-row form of the forge
// flash_attention.metal backward kernels: nothing of size Sq x Sk is stored;
// each query row recomputes its probabilities from the saved log-sum-exp,
//   P_ij  = exp(scale q_i.k_j - LSE_i)            (visible keys only)
//   D_i   = dO_i . O_i                            (the FA2 identity)
//   dS_ij = P_ij (dO_i . v_j - D_i)
//   dQ_i  = scale sum_j dS_ij k_j                 (kernel bwd_dq_kernel)
//   dV_j  = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i
//                                                 (kernel bwd_dkdv_kernel)
// with dK and dV summed over the query heads of a kv head. As in forge, dK
// and dV accumulate privately per key row (no atomics, deterministic), and
// D_i is computed once per query row by the dQ kernel and handed to the dK/dV
// kernel through a workspace.
//
// Work decomposition: a group of 16 lanes owns one row (a query row in the
// dQ kernel, a key row in the dK/dV kernel) and holds D/16 consecutive
// elements of each row vector per lane; dot products reduce over the 16 lanes
// with four DPP row rotations. A wavefront serves four rows, a workgroup 16. This
// is the pages' thread-per-row design mapped to wavefronts, on the VALU (no
// MFMA): a baseline that is exact to fp32 rounding, not a tuned kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_bwd.h"

namespace fa {

constexpr int kBwdThreads = 256;   // 4 wavefronts x 4 rows
constexpr int kRowsPerBlock = 16;
constexpr float kLog2e = 1.4426950408889634f;

template <typename E>
__device__ __forceinline__ float to_f32(E x) { return (float)x; }

// Value of lane (l + n) mod 16 of the same 16-lane row (DPP row_ror:n).
template <int N>
__device__ __forceinline__ float row_ror(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), 0x120 + N, 0xf, 0xf, false));
}

// Sum over the 16 lanes of one row group (every lane gets the total):
// register-to-register rotations within the row, no LDS round trips.
__device__ __forceinline__ float group_sum(float x) {
  x += row_ror<8>(x);
  x += row_ror<4>(x);
  x += row_ror<2>(x);
  x += row_ror<1>(x);
  return x;
}

template <typename E, int NE>
__device__ __forceinline__ void load_part(const E* __restrict__ p, float (&x)[NE]) {
#pragma unroll
  for (int e = 0; e < NE; ++e) x[e] = to_f32(p[e]);
}

// Visible keys [lo, hi) of query row i (causal: j <= i; window: j >= i - w + 1).
__device__ __forceinline__ void row_keys(const BwdParams& p, int i, int& lo, int& hi) {
  lo = p.window > 0 ? max(0, i - p.window + 1) : 0;
  hi = p.causal ? min(p.Sk, i + 1) : p.Sk;
}

// Query rows [lo, hi) that see key j.
__device__ __forceinline__ void key_rows(const BwdParams& p, int j, int& lo, int& hi) {
  lo = p.causal ? j : 0;
  hi = p.window > 0 ? min(p.Sq, j + p.window) : p.Sq;
}

// One 16-lane group per query row (b, h, i): D_i, then dQ_i.
template <typename E, int D>
__global__ __launch_bounds__(kBwdThreads)
void bwd_dq_kernel(BwdParams p) {
  constexpr int NE = D / 16;
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const long row = (long)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  const long rows = (long)p.B * p.H * p.Sq;
  if (row >= rows) return;   // whole 16-lane groups leave together
  const int i = (int)(row % p.Sq);
  const long bh = row / p.Sq;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const int hk = h / (p.H / p.HKV);

  const E* Qr = (const E*)p.Q + row * D + l16 * NE;
  const E* Or = (const E*)p.O + row * D + l16 * NE;
  const E* dOr = (const E*)p.dO + row * D + l16 * NE;
  const E* Kh = (const E*)p.K + ((long)b * p.HKV + hk) * p.Sk * D + l16 * NE;
  const E* Vh = (const E*)p.V + ((long)b * p.HKV + hk) * p.Sk * D + l16 * NE;

  float q[NE], o[NE], go[NE], dq[NE];
  load_part<E, NE>(Qr, q);
  load_part<E, NE>(Or, o);
  load_part<E, NE>(dOr, go);
  float dd = 0.f;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    dd = fmaf(go[e], o[e], dd);
    dq[e] = 0.f;
  }
  const float Di = group_sum(dd);
  const float L2 = p.LSE[row] * kLog2e;   // base-2 log-sum-exp (-inf: no visible key)
  const float sl = p.scale * kLog2e;

  int lo, hi;
  row_keys(p, i, lo, hi);
  if (L2 == -INFINITY) hi = lo;            // empty row: P = 0 everywhere
  // key j + 1's rows are loaded while key j is computed
  float kn[NE], vn[NE];
  if (lo < hi) {
    load_part<E, NE>(Kh + (long)lo * D, kn);
    load_part<E, NE>(Vh + (long)lo * D, vn);
  }
  for (int j = lo; j < hi; ++j) {
    float k[NE], v[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      k[e] = kn[e];
      v[e] = vn[e];
    }
    if (j + 1 < hi) {
      load_part<E, NE>(Kh + (long)(j + 1) * D, kn);
      load_part<E, NE>(Vh + (long)(j + 1) * D, vn);
    }
    float s = 0.f, dp = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      s = fmaf(q[e], k[e], s);
      dp = fmaf(go[e], v[e], dp);
    }
    s = group_sum(s);
    dp = group_sum(dp);
    const float pr = __builtin_amdgcn_exp2f(fmaf(s, sl, -L2));
    const float ds = pr * (dp - Di);
#pragma unroll
    for (int e = 0; e < NE; ++e) dq[e] = fmaf(ds, k[e], dq[e]);
  }
  float* out = p.dQ + row * D + l16 * NE;
#pragma unroll
  for (int e = 0; e < NE; ++e) out[e] = p.scale * dq[e];
  if (l16 == 0) p.Dws[row] = Di;
}

// One 16-lane group per key row (b, hk, j): dK_j and dV_j over the query
// heads of kv head hk and the query rows that see key j.
template <typename E, int D>
__global__ __launch_bounds__(kBwdThreads)
void bwd_dkdv_kernel(BwdParams p) {
  constexpr int NE = D / 16;
  const int lane = threadIdx.x & 63, l16 = lane & 15;
  const long krow = (long)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 4);
  const long krows = (long)p.B * p.HKV * p.Sk;
  if (krow >= krows) return;
  const int j = (int)(krow % p.Sk);
  const long bhk = krow / p.Sk;
  const int hk = (int)(bhk % p.HKV), b = (int)(bhk / p.HKV);
  const int g = p.H / p.HKV;

  float k[NE], v[NE], dk[NE], dv[NE];
  load_part<E, NE>((const E*)p.K + krow * D + l16 * NE, k);
  load_part<E, NE>((const E*)p.V + krow * D + l16 * NE, v);
#pragma unroll
  for (int e = 0; e < NE; ++e) dk[e] = dv[e] = 0.f;
  const float sl = p.scale * kLog2e;

  int lo, hi;
  key_rows(p, j, lo, hi);
  for (int h = hk * g; h < hk * g + g; ++h) {
    const long base = ((long)b * p.H + h) * p.Sq;
    // query row i + 1 is loaded while row i is computed
    float qn[NE], gn[NE], ln = 0.f, dn = 0.f;
    if (lo < hi) {
      load_part<E, NE>((const E*)p.Q + (base + lo) * D + l16 * NE, qn);
      load_part<E, NE>((const E*)p.dO + (base + lo) * D + l16 * NE, gn);
      ln = p.LSE[base + lo];
      dn = p.Dws[base + lo];
    }
    for (int i = lo; i < hi; ++i) {
      const long row = base + i;
      float q[NE], go[NE];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        q[e] = qn[e];
        go[e] = gn[e];
      }
      const float Li = ln, Di = dn;
      if (i + 1 < hi) {
        load_part<E, NE>((const E*)p.Q + (row + 1) * D + l16 * NE, qn);
        load_part<E, NE>((const E*)p.dO + (row + 1) * D + l16 * NE, gn);
        ln = p.LSE[row + 1];
        dn = p.Dws[row + 1];
      }
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        s = fmaf(q[e], k[e], s);
        dp = fmaf(go[e], v[e], dp);
      }
      s = group_sum(s);
      dp = group_sum(dp);
      // row i sees key j, so it is not empty and its LSE is finite
      const float pr = __builtin_amdgcn_exp2f(fmaf(s, sl, -Li * kLog2e));
      const float ds = pr * (dp - Di);
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        dv[e] = fmaf(pr, go[e], dv[e]);
        dk[e] = fmaf(ds, q[e], dk[e]);
      }
    }
  }
  float* odk = p.dK + krow * D + l16 * NE;
  float* odv = p.dV + krow * D + l16 * NE;
#pragma unroll
  for (int e = 0; e < NE; ++e) {
    odk[e] = p.scale * dk[e];
    odv[e] = dv[e];
  }
}

template <typename E, int D>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  const long rows = (long)p.B * p.H * p.Sq, krows = (long)p.B * p.HKV * p.Sk;
  hipLaunchKernelGGL((bwd_dq_kernel<E, D>), dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(kBwdThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<E, D>), dim3((unsigned)((krows + kRowsPerBlock - 1) / kRowsPerBlock)),
                     dim3(kBwdThreads), 0, stream, p);
  return hipGetLastError();
}

template <typename E>
static hipError_t launch_bwd_e(const BwdParams& p, int D, hipStream_t stream) {
  switch (D) {
    case 64: return launch_bwd_t<E, 64>(p, stream);
    case 128: return launch_bwd_t<E, 128>(p, stream);
    case 256: return launch_bwd_t<E, 256>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_backward(const BwdParams& p, int dtype, int D, hipStream_t stream) {
  if (dtype == 0) return launch_bwd_e<float>(p, D, stream);
  if (dtype == 1) return launch_bwd_e<__bf16>(p, D, stream);
  if (dtype == 2) return launch_bwd_e<_Float16>(p, D, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

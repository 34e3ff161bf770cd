// Backward pass of the fused attention (gradients of sum(O * dO) with
// respect to Q, K and V) for gfx950, in the per-row form of the forge
// flash_attention.metal backward kernels: nothing of size Sq x Sk is stored;
// each query row recomputes its probabilities from the saved log-sum-exp,
//   P_ij  = exp(scale q_i.k_j - LSE_i)            (visible keys only)
//   D_i   = dO_i . O_i                            (the FA2 identity)
//   dS_ij = P_ij (dO_i . v_j - D_i)
//   dQ_i  = scale sum_j dS_ij k_j                 (the dQ kernels)
//   dV_j  = sum_i P_ij dO_i,  dK_j = scale sum_i dS_ij q_i
//                                                 (the dK/dV kernels)
// with dK and dV summed over the query heads of a kv head. Every dK/dV row
// has a single owner that sums its contributions in a fixed order, so no
// atomics are needed and the result is deterministic (the approach of the
// forge flash_attention.metal backward kernels). D_i is computed once per
// query row by the dQ kernel and handed to the dK/dV kernel through a
// workspace.
//
// Three kernel families:
// - 16-bit inputs: MFMA kernels (bwd_dq_mfma_kernel, bwd_dkdv_mfma_kernel) at
//   tile dims 64, 128 and 256; in their general form they read views with
//   strides and head dims below the tile dim (those dims read as zeros).
// - fp32 inputs at D = 32, 64, 96, 128, 256: MFMA kernels on
//   v_mfma_f32_32x32x2_f32 (bwd_dq_f32_mfma_kernel, bwd_dkdv_f32_mfma_kernel,
//   in fa_bwd_f32.hip; at 256 the head dims split over wavefront pairs).
// - fp32 inputs at D = 16, 48, 80 on small problems (larger ones are staged
//   into the MFMA kernels of the 32, 64, 96 tiles, the extra dims zero): the
//   per-row kernels below (bwd_dq_kernel, bwd_dkdv_kernel), the pages'
//   thread-per-row design mapped to wavefronts on the VALU: a group of G = 4,
//   8 or 16 lanes (the fewest that keep D / G <= 8; the kernels also take 32
//   for wider rows) owns R consecutive rows of one head (bwd_rows_per_group: 4
//   with 16 lanes, else 2), query rows in the dQ kernel, key rows in the dK/dV
//   kernel. A lane holds D / G consecutive elements of each row vector; dot
//   products reduce over the group with two to four DPP steps (and one lane
//   permute at G = 32).
// On small grids the per-row kernels run each group's range in chunks
// (blockIdx.y), and the MFMA dQ kernels the key axis in chunks, whose partial
// sums sum_parts_kernel adds in chunk order. Under a block mask (the block
// masks of the metal-flash-attention README, "Modifications to
// FlashAttention"; Msk instances of every kernel) each MFMA workgroup first
// lists the tiles its mask leaves visible (bwd_build_list) and copies and
// computes only those; the per-row kernels test the mask byte per pair.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_bwd.h"
#include "fa_bwd_device.h"
#include "fa_tile.h"

namespace fa {

// General-form copies: an offset past any buffer range (its chunk lands in LDS
// as zeros) and the largest range given to a copy (below that offset).
constexpr int kBwdOutOfRange = 0x7ffffff0;
constexpr long long kBwdMaxRange = 0x7fff0000LL;

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
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
      0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Sum over the G lanes of one group (G = 4, 8, 16 or 32, aligned): quad_perm
// swaps within each 4 lanes, then row_half_mirror (8); row rotations (16),
// plus the other 16-lane row through a lane permute (32).
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (G >= 16) {
    x += row_ror<8>(x);
    x += row_ror<4>(x);
    x += row_ror<2>(x);
    x += row_ror<1>(x);
    if constexpr (G == 32) x += __shfl_xor(x, 16);
  } else {
    x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]
    x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]
    if constexpr (G == 8) x += dpp<0x141>(x);   // row_half_mirror: the other quad of 8
  }
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

// Rows per lane group in the per-row kernels: R rows of one head share every
// K/V (dQ) or Q/dO (dK/dV) load and give the group R independent
// dot-product chains; four with 16-lane groups, two with 4, 8 or 32 lanes.
template <int D>
constexpr int rows_per_group() { return bwd_rows_per_group(D); }

// D_i, then dQ_i, for R consecutive query rows (b, h, i0 ..) per 16-lane group.
template <typename E, int D, bool Msk>
__global__ __launch_bounds__(kBwdThreads)
void bwd_dq_kernel(BwdParams p) {
  constexpr int G = bwd_lanes_per_row(D), NE = D / G, R = rows_per_group<D>();
  const int lg = threadIdx.x & (G - 1);    // lane within the group
  const long grp = (long)blockIdx.x * (kBwdThreads / G) + threadIdx.x / G;
  const long per_head = (p.Sq + R - 1) / R;
  if (grp >= (long)p.B * p.H * per_head) return;   // whole 16-lane groups leave together
  const long bh = grp / per_head;
  const int i0 = (int)(grp - bh * per_head) * R;
  const int h = (int)(bh % p.H), b = (int)(bh / p.H);
  const int hk = h / (p.H / p.HKV);
  const E* Kh = (const E*)p.K + ((long)b * p.HKV + hk) * p.Sk * D + lg * NE;
  const E* Vh = (const E*)p.V + ((long)b * p.HKV + hk) * p.Sk * D + lg * NE;
  const float sl = p.scale * kLog2e;

  float q[R][NE], go[R][NE], dq[R][NE], Di[R], L2[R];
  int rlo[R], rhi[R];
  const unsigned char* mrow[R];   // (block mask: each row's mask row)
  int lo = p.Sk, hi = 0;   // union of the rows' visible keys
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int i = i0 + r;
    if constexpr (Msk) mrow[r] = bwd_mask_row(p, b, h, hk, min(i, p.Sq - 1) / kBwdMaskQ);
    rlo[r] = 0;
    rhi[r] = 0;
    float dd = 0.f;
    L2[r] = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e) q[r][e] = go[r][e] = dq[r][e] = 0.f;
    if (i < p.Sq) {
      const long row = bh * p.Sq + i;
      float o[NE];
      load_part<E, NE>((const E*)p.Q + row * D + lg * NE, q[r]);
      load_part<E, NE>((const E*)p.O + row * D + lg * NE, o);
      load_part<E, NE>((const E*)p.dO + row * D + lg * NE, go[r]);
#pragma unroll
      for (int e = 0; e < NE; ++e) dd = fmaf(go[r][e], o[e], dd);
      L2[r] = p.LSE[row] * kLog2e;         // base-2 log-sum-exp (-inf: no visible key)
      row_keys(p, i, rlo[r], rhi[r]);
      if (L2[r] == -INFINITY) rhi[r] = rlo[r];   // empty row: P = 0 everywhere
      if (rlo[r] < rhi[r]) {
        lo = min(lo, rlo[r]);
        hi = max(hi, rhi[r]);
      }
    }
    Di[r] = group_sum<G>(dd);
  }
  if (p.nch > 1) {   // this launch's chunk of the union (empty past its end)
    const int c0 = lo + (int)blockIdx.y * p.chunk_q;
    hi = min(hi, c0 + p.chunk_q);
    lo = c0;
  }
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
    float s[R], dp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s[r] = dp[r] = 0.f;
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        s[r] = fmaf(q[r][e], k[e], s[r]);
        dp[r] = fmaf(go[r][e], v[e], dp[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s[r] = group_sum<G>(s[r]);
      dp[r] = group_sum<G>(dp[r]);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool in = j >= rlo[r] && j < rhi[r] && (!Msk || mrow[r][j / kBwdMaskK] != 0);
      const float pr = in ? __builtin_amdgcn_exp2f(fmaf(s[r], sl, -L2[r])) : 0.f;
      const float ds = pr * (dp[r] - Di[r]);
#pragma unroll
      for (int e = 0; e < NE; ++e) dq[r][e] = fmaf(ds, k[e], dq[r][e]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (i0 + r >= p.Sq) continue;
    const long row = bh * p.Sq + i0 + r;
    if (p.nch > 1) {
      float* out = p.part_q + ((long)blockIdx.y * p.B * p.H * p.Sq + row) * D + lg * NE;
#pragma unroll
      for (int e = 0; e < NE; ++e) out[e] = dq[r][e];
    } else {
      float* out = p.dQ + row * D + lg * NE;
#pragma unroll
      for (int e = 0; e < NE; ++e) out[e] = p.scale * dq[r][e];
    }
    if (lg == 0 && blockIdx.y == 0) p.Dws[row] = Di[r];
  }
}

// dK_j and dV_j for R consecutive key rows (b, hk, j0 ..) per 16-lane group,
// over the query heads of kv head hk and the query rows that see each key.
template <typename E, int D, bool Msk>
__global__ __launch_bounds__(kBwdThreads)
void bwd_dkdv_kernel(BwdParams p) {
  constexpr int G = bwd_lanes_per_row(D), NE = D / G, R = rows_per_group<D>();
  const int lg = threadIdx.x & (G - 1);    // lane within the group
  const long grp = (long)blockIdx.x * (kBwdThreads / G) + threadIdx.x / G;
  const long per_head = (p.Sk + R - 1) / R;
  if (grp >= (long)p.B * p.HKV * per_head) return;
  const long bhk = grp / per_head;
  const int j0 = (int)(grp - bhk * per_head) * R;
  const int hk = (int)(bhk % p.HKV), b = (int)(bhk / p.HKV);
  const int g = p.H / p.HKV;
  const float sl = p.scale * kLog2e;

  float k[R][NE], v[R][NE], dk[R][NE], dv[R][NE];
  int rlo[R], rhi[R];
  int lo = p.Sq, hi = 0;   // union of the query rows that see the keys
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int j = j0 + r;
#pragma unroll
    for (int e = 0; e < NE; ++e) k[r][e] = v[r][e] = dk[r][e] = dv[r][e] = 0.f;
    rlo[r] = rhi[r] = 0;
    if (j < p.Sk) {
      const long krow = bhk * p.Sk + j;
      load_part<E, NE>((const E*)p.K + krow * D + lg * NE, k[r]);
      load_part<E, NE>((const E*)p.V + krow * D + lg * NE, v[r]);
      key_rows(p, j, rlo[r], rhi[r]);
      if (rlo[r] < rhi[r]) {
        lo = min(lo, rlo[r]);
        hi = max(hi, rhi[r]);
      }
    }
  }
  if (p.nch > 1) {   // this launch's chunk of the union, in every query head
    const int c0 = lo + (int)blockIdx.y * p.chunk_k;
    hi = min(hi, c0 + p.chunk_k);
    lo = c0;
  }

  for (int h = hk * g; h < hk * g + g; ++h) {
    const long base = ((long)b * p.H + h) * p.Sq;
    // query row i + 1 is loaded while row i is computed
    float qn[NE], gn[NE], ln = 0.f, dn = 0.f;
    if (lo < hi) {
      load_part<E, NE>((const E*)p.Q + (base + lo) * D + lg * NE, qn);
      load_part<E, NE>((const E*)p.dO + (base + lo) * D + lg * NE, gn);
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
        load_part<E, NE>((const E*)p.Q + (row + 1) * D + lg * NE, qn);
        load_part<E, NE>((const E*)p.dO + (row + 1) * D + lg * NE, gn);
        ln = p.LSE[row + 1];
        dn = p.Dws[row + 1];
      }
      float s[R], dp[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        s[r] = dp[r] = 0.f;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          s[r] = fmaf(q[e], k[r][e], s[r]);
          dp[r] = fmaf(go[e], v[r][e], dp[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        s[r] = group_sum<G>(s[r]);
        dp[r] = group_sum<G>(dp[r]);
      }
      const unsigned char* mrow = Msk ? bwd_mask_row(p, b, h, hk, i / kBwdMaskQ) : nullptr;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        // a row that sees key j is not empty, so its LSE is finite
        const bool in = i >= rlo[r] && i < rhi[r] && (!Msk || mrow[(j0 + r) / kBwdMaskK] != 0);
        const float pr = in ? __builtin_amdgcn_exp2f(fmaf(s[r], sl, -Li * kLog2e)) : 0.f;
        const float ds = pr * (dp[r] - Di);
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          dv[r][e] = fmaf(pr, go[e], dv[r][e]);
          dk[r][e] = fmaf(ds, q[e], dk[r][e]);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (j0 + r >= p.Sk) continue;
    const long krow = bhk * p.Sk + j0 + r;
    const bool part = p.nch > 1;
    const long prow = (long)blockIdx.y * p.B * p.HKV * p.Sk + krow;
    float* odk = (part ? p.part_k + prow * D : p.dK + krow * D) + lg * NE;
    float* odv = (part ? p.part_v + prow * D : p.dV + krow * D) + lg * NE;
    const float ks = part ? 1.f : p.scale;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      odk[e] = ks * dk[r][e];
      odv[e] = dv[r][e];
    }
  }
}

// ------------------------------------------------------------------ MFMA dQ
// dQ for 16-bit inputs at D <= 128 on MFMA, in the forward kernel's layout:
// a workgroup is 4 wavefronts x 32 query rows, K and V tiles of 32 keys are
// double-buffered in LDS by the buffer unit, and a lane owns one query row.
//   S^T  = K Q^T          (A: K rows from LDS, B: Q rows in registers)
//   dP^T = V dO^T         (A: V rows from LDS, B: dO rows in registers)
//   P = exp2(S^T |scale| log2 e - LSE log2 e),  dS^T = P (dP^T - D_i)
//   dQ^T += K^T dS^T      (A: K^T by transposed reads of the K tile, B: dS^T
//                          packed to the input type as the forward packs P)
// The K tile is read both by rows (S^T) and transposed (K^T). With either the
// forward's K swizzle or its V swizzle alone, half the LDS cycles went to bank
// conflicts; the tiles take the swizzle that serves both patterns
// (Bf16Tile::swz_b), so K is copied once. V is read by rows only.
// D_i = dO_i . O_i is formed here and written for the dK/dV kernel.
template <typename E, int D, bool Gen, bool Msk>
__global__ __launch_bounds__(kBwdThreads, D <= 128 ? 2 : 1)
void bwd_dq_mfma_kernel(BwdParams p) {
  constexpr int BN = 32;
  using T = Bf16Tile<D, BN>;
  using X = Elt<E>;
  typedef typename X::x8 e16x8;
  // D = 256: one wavefront per SIMD (the dQ^T accumulators, 128 registers, in AGPRs)
  static_assert(D == 64 || D == 128 || D == 256, "MFMA tile dims");
  __shared__ __attribute__((aligned(1024))) char kbuf0[T::TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1[T::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0[T::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1[T::TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int units = p.B * p.H;
  const int qblk = p.n_qblk - 1 - (int)(blockIdx.x / units);   // heaviest query tiles first
  const int u = blockIdx.x % units;
  const int h = u % p.H, b = u / p.H;
  const int hkv = h / (p.H / p.HKV);
  const int q0 = qblk * 128, qw = q0 + wave * 32, i = qw + l32;
  const bool row_ok = i < p.Sq;
  const long row = ((long)b * p.H + h) * p.Sq + i;

  // row starts: contiguous tensors, or (general form) the views' strides
  const E *Qh, *Oh, *dOh, *Kp, *Vp;
  long long qr = D, orow = D, dor = D, kr = D, vr = D;   // element row strides
  if constexpr (Gen) {
    Qh = (const E*)p.Q + b * p.qs[0] + h * p.qs[1];
    Oh = (const E*)p.O + b * p.os[0] + h * p.os[1];
    dOh = (const E*)p.dO + b * p.dos[0] + h * p.dos[1];
    Kp = (const E*)p.K + b * p.ks[0] + hkv * p.ks[1];
    Vp = (const E*)p.V + b * p.vs[0] + hkv * p.vs[1];
    qr = p.qs[2];
    orow = p.os[2];
    dor = p.dos[2];
    kr = p.ks[2];
    vr = p.vs[2];
  } else {
    Qh = (const E*)p.Q + ((long)b * p.H + h) * p.Sq * D;
    Oh = (const E*)p.O + ((long)b * p.H + h) * p.Sq * D;
    dOh = (const E*)p.dO + ((long)b * p.H + h) * p.Sq * D;
    Kp = (const E*)p.K + ((long)b * p.HKV + hkv) * p.Sk * D;
    Vp = (const E*)p.V + ((long)b * p.HKV + hkv) * p.Sk * D;
  }

  // key range of the block; on small grids only key chunk blockIdx.y of it
  // (chunk_q is a multiple of BN, so the chunks split the key tiles exactly)
  int lo = 0, hi = p.Sk;
  if (p.causal) hi = min(hi, min(q0 + 128, p.Sq));
  if (p.window > 0) lo = max(0, q0 - p.window + 1);
  if (p.nch > 1) {
    lo = max(lo, (int)blockIdx.y * p.chunk_q);
    hi = min(hi, ((int)blockIdx.y + 1) * p.chunk_q);
  }
  const int t0 = (lo / BN) * BN;
  const int n_cand = hi > lo ? (hi - t0 + BN - 1) / BN : 0;   // key tiles of the range
  // block mask: only the tiles whose mask byte is nonzero are copied and
  // computed, listed in portions of up to kBwdMaxList tiles
  __shared__ unsigned tlist[Msk ? kBwdMaxList : 1];
  __shared__ int tsh[2];
  int n_tiles = n_cand, c_next = n_cand;
  const unsigned char* mrow = nullptr;
  if constexpr (Msk) {
    mrow = bwd_mask_row(p, b, h, hkv, qblk);
    n_tiles = bwd_build_list(
        0, n_cand, tlist, tsh, wave, lane,
        [&](int t) { return mrow[(t0 + t * BN) / kBwdMaskK] != 0 ? 1u : 0u; },
        [](int t, unsigned) { return (unsigned)t; },
        &c_next);
  }
  // first key of the t-th tile visited
  auto tile_kt = [&](int t) {
    if constexpr (Msk)
      return t0 + BN * (int)__builtin_amdgcn_readfirstlane(tlist[t]);
    else
      return t0 + t * BN;
  };

  const int voff = T::dma_off(64 * wave * T::NIW + lane, kSwzB);
  // general form: each copy instruction's lane offset in full (any row
  // stride), or past the buffer's range for a chunk at or beyond dim dv,
  // which then lands in LDS as zeros
  int pk_off[Gen ? T::NIW : 1], pv_off[Gen ? T::NIW : 1];
  if constexpr (Gen) {
#pragma unroll
    for (int k = 0; k < T::NIW; ++k) {
      const int P = 64 * (wave * T::NIW + k) + lane, r = P / T::CPR;
      const int ck = (P % T::CPR) ^ T::swz_b(r);
      pk_off[k] = 8 * ck < p.dv ? r * (int)(2 * kr) + 16 * ck : kBwdOutOfRange;
      pv_off[k] = 8 * ck < p.dv ? r * (int)(2 * vr) + 16 * ck : kBwdOutOfRange;
    }
  }
  auto issue = [&](int kt, char* kd, char* vd) {
    const E* kb = Kp + kt * kr;
    const E* vb = Vp + kt * vr;
    if constexpr (Gen) {
      // valid bytes from the tile's first row: up to the end of row Sk - 1
      const unsigned kbytes = (unsigned)min((long long)(p.Sk - kt - 1) * 2 * kr + 2 * p.dv, kBwdMaxRange);
      const unsigned vbytes = (unsigned)min((long long)(p.Sk - kt - 1) * 2 * vr + 2 * p.dv, kBwdMaxRange);
#pragma unroll
      for (int k = 0; k < T::NIW; ++k) {
        const int off = (wave * T::NIW + k) * 1024;
        dma16(kb, kbytes, pk_off[k], kd + off);
        dma16(vb, vbytes, pv_off[k], vd + off);
      }
    } else {
      const unsigned bytes = (unsigned)min((long)(p.Sk - kt) * T::ROW, 0x7fffffffL);
#pragma unroll
      for (int k = 0; k < T::NIW; ++k) {
        const int off = (wave * T::NIW + k) * 1024;
        dma16(kb, bytes, voff ^ T::dma_xor(k, kSwzB), kd + off);
        dma16(vb, bytes, voff ^ T::dma_xor(k, kSwzB), vd + off);
      }
    }
  };
  if (n_tiles > 0) issue(tile_kt(0), kbuf0, vbuf0);

  // Q and dO rows as B operands (k-slot (g, e) of step t is dim 16t + 8g + e);
  // D_i from the same dims of O, summed over the two lane halves.
  e16x8 qf[T::DC], dof[T::DC];
  float dd = 0.f;
#pragma unroll
  for (int t = 0; t < T::DC; ++t) {
    // (general form: the dims from dv on, a multiple of 16, are zeros)
    if (row_ok && (!Gen || 16 * t < p.dv)) {
      qf[t] = *(const e16x8*)(Qh + i * qr + 16 * t + 8 * g);
      dof[t] = *(const e16x8*)(dOh + i * dor + 16 * t + 8 * g);
      const e16x8 ov = *(const e16x8*)(Oh + i * orow + 16 * t + 8 * g);
#pragma unroll
      for (int e = 0; e < 8; ++e) dd = fmaf((float)dof[t][e], (float)ov[e], dd);
    } else {
      qf[t] = e16x8{};
      dof[t] = e16x8{};
    }
    if (p.neg_q) {   // negative scale: -Q and |scale| (exact sign flips)
      u32x4 bits = __builtin_bit_cast(u32x4, qf[t]) ^ 0x80008000u;
      qf[t] = __builtin_bit_cast(e16x8, bits);
    }
  }
  const float Di = dd + __shfl_xor(dd, 32);
  // base-2 LSE; +inf for rows past Sq or with no visible key, so that P = 0
  float L2 = row_ok ? p.LSE[row] * 1.4426950408889634f : INFINITY;
  if (L2 == -INFINITY) L2 = INFINITY;
  const float sl = p.sl_abs;

  // operand offsets (tile-relative): K/V rows for S^T and dP^T, K^T for dQ^T
  const int krow = perm_row(l32);
  int koff[T::DC];
#pragma unroll
  for (int t = 0; t < T::DC; ++t) koff[t] = krow * T::ROW + (((2 * t + g) ^ T::swz_b(krow)) << 4);
  // transposed reads, as the forward reads V^T: the second read is 4 rows on,
  // where the XOR differs in bit 0 (vrow % 8 < 4): byte-offset bit 4 flips
  const int blk = lane >> 4, li = lane & 15;
  const int vrow = 8 * g + (li >> 2);
  int ktoff[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) {
    const int chunk = 4 * db + 2 * (blk & 1) + ((li & 3) >> 1);
    ktoff[db] = vrow * T::ROW + ((chunk ^ T::swz_b(vrow)) << 4) + 8 * (li & 1);
  }

  f32x16 dq[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) dq[db] = f32x16{};

  auto step = [&](int t, const char* Kc, const char* Vc, char* Kn, char* Vn) __attribute__((always_inline)) {
    const int kt = tile_kt(t);
    wait_dma_and_sync();
    if (t + 1 < n_tiles) issue(tile_kt(t + 1), Kn, Vn);
    if (qw >= p.Sq || (p.causal && kt > qw + 31) ||
        (p.window > 0 && kt + BN - 1 < qw - p.window + 1))
      return;
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int t2 = 0; t2 < T::DC; ++t2) {
      const e16x8 ak = *(const e16x8*)(Kc + koff[t2]);
      const e16x8 av = *(const e16x8*)(Vc + koff[t2]);
      s = X::mfma(ak, qf[t2], s);
      dp = X::mfma(av, dof[t2], dp);
    }
    if constexpr (D == 256) {
      // one wavefront per SIMD: operand reads eight products ahead (at two
      // wavefronts per SIMD the other one hides the latency; measured equal)
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int k = 0; k < 2 * T::DC - 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    // element v holds key kt + 8g + c, c = 16 (v / 8) + v % 8
    const bool edge = (kt + BN > p.Sk) || (p.causal && kt + BN - 1 > qw) ||
                      (p.window > 0 && kt < qw + 31 - p.window + 1);
    typename X::x8 dsf[2];
    // the mask in one branch (a test per element inside the exponential
    // loop became a branch per element on every tile); the row index goes
    // through an empty asm so that the test stays behind the branch
    float xs[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) xs[v] = fmaf(s[v], sl, -L2);
    if (edge) {
      int ii = i;
      asm volatile("" : "+v"(ii));
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int j = kt + 8 * g + 16 * (v >> 3) + (v & 7);
        const bool vis = j < p.Sk && (!p.causal || j <= ii) && (p.window <= 0 || j > ii - p.window);
        xs[v] = vis ? xs[v] : -INFINITY;
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float pr = __builtin_amdgcn_exp2f(xs[v]);
      dsf[v >> 3][v & 7] = (E)(pr * (dp[v] - Di));
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      e16x8 a[T::DB];
#pragma unroll
      for (int db = 0; db < T::DB; ++db) {
        const int o = ktoff[db] + 16 * c * T::ROW;
        a[db] = read_v_pair<e16x8>(Kc, o, (o + 4 * T::ROW) ^ 16);
      }
#pragma unroll
      for (int db = 0; db < T::DB; ++db) dq[db] = X::mfma(a[db], dsf[c], dq[db]);
    }
  };

  for (;;) {
    for (int t = 0; t < n_tiles; t += 2) {
      step(t, kbuf0, vbuf0, kbuf1, vbuf1);
      if (t + 1 < n_tiles) step(t + 1, kbuf1, vbuf1, kbuf0, vbuf0);
    }
    if (c_next >= n_cand) break;
    if constexpr (Msk) {   // the next portion of the list
      n_tiles = bwd_build_list(
          c_next, n_cand, tlist, tsh, wave, lane,
          [&](int t) { return mrow[(t0 + t * BN) / kBwdMaskK] != 0 ? 1u : 0u; },
          [](int t, unsigned) { return (unsigned)t; }, &c_next);
      if (n_tiles > 0) issue(tile_kt(0), kbuf0, vbuf0);
    }
  }

  // lane holds dims 32 db + 8 a + 4 g + (0..3) of row i; a key chunk writes
  // its unscaled partial sums, added up in chunk order afterwards
  // (general form: dQ is a view with strides p.dqs, written in its first dv dims)
  if (row_ok) {
    const bool part = p.nch > 1;
    const float sc = part ? 1.f : p.scale;
    float* dst = part ? p.part_q + ((long)blockIdx.y * p.B * p.H * p.Sq + row) * D
                 : Gen ? p.dQ + b * p.dqs[0] + h * p.dqs[1] + i * p.dqs[2]
                       : p.dQ + row * D;
    const int dlim = Gen && !part ? p.dv : D;
#pragma unroll
    for (int db = 0; db < T::DB; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if (32 * db + 8 * a + 4 * g >= dlim) continue;
        const f32x4 v4 = {dq[db][4 * a] * sc, dq[db][4 * a + 1] * sc,
                          dq[db][4 * a + 2] * sc, dq[db][4 * a + 3] * sc};
        *(f32x4*)(dst + 32 * db + 8 * a + 4 * g) = v4;
      }
    if (g == 0 && blockIdx.y == 0) p.Dws[row] = Di;
  }
}

// ------------------------------------------------------------- MFMA dK, dV
// dK and dV for 16-bit inputs at D <= 128 on MFMA, the mirror of the dQ
// kernel: a workgroup owns 128 keys (4 wavefronts x 32, a lane owns one key)
// with K and V rows in registers, and walks 32-row tiles of Q and dO (and the
// tile rows' base-2 LSE and D_i) through LDS, over every query head of the kv
// head, double-buffered by the buffer unit.
//   S  = Q K^T, dP = dO V^T      (A: Q / dO rows from LDS, B: K / V rows)
//   P  = exp2(S |scale| log2 e - LSE log2 e),  dS = P (dP - D)
//   dV^T += dO^T P,  dK^T += Q^T dS   (A: transposed reads of the dO / Q
//                                      tiles, B: P / dS packed to the input type)
template <typename E, int D, bool Gen, bool Msk>
__global__ __launch_bounds__(kBwdThreads, 1)
void bwd_dkdv_mfma_kernel(BwdParams p) {
  // 64 query rows per copied tile, worked as two independent 32-row halves
  // between barriers, so one half's MFMAs can issue under the other's
  // exponentials (one wavefront per SIMD leaves no other wavefront to do it).
  // D = 256 is blocked along the output dims: a workgroup accumulates dK and
  // dV for DO = 128 of the 256 dims (blockIdx.x % 2 picks which) while its
  // score products S and dP take all 256; its Q/dO tiles are 32 rows (the
  // four copies of a 64-row tile would not fit in LDS).
  constexpr int DO = D <= 128 ? D : 128;         // output dims per workgroup
  constexpr int DBO = DO / 32;                   // output dim blocks per workgroup
  constexpr int BM = D <= 128 ? 64 : 32, HM = 32, NH = BM / HM;
  using T = Bf16Tile<D, BM>;
  using X = Elt<E>;
  typedef typename X::x8 e16x8;
  static_assert(D == 64 || D == 128 || D == 256, "MFMA tile dims");
  // Q and dO tiles are read by rows and transposed: one copy each, with the
  // swizzle that serves both (see the dQ kernel)
  __shared__ __attribute__((aligned(1024))) char qbuf0[T::TILE];
  __shared__ __attribute__((aligned(1024))) char qbuf1[T::TILE];
  __shared__ __attribute__((aligned(1024))) char obuf0[T::TILE];
  __shared__ __attribute__((aligned(1024))) char obuf1[T::TILE];
  __shared__ __attribute__((aligned(16))) float lbuf0[2 * BM];   // [0, BM): base-2 LSE, [BM, 2 BM): D
  __shared__ __attribute__((aligned(16))) float lbuf1[2 * BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int units = p.B * p.HKV;
  const int ob = blockIdx.x % (D / DO);               // output dim block: dims DO ob ..
  const int bid = blockIdx.x / (D / DO);
  const int kblk = bid / units;   // ascending: under a causal mask the first keys see most rows
  const int u = bid % units;
  const int hkv = u % p.HKV, b = u / p.HKV;
  const int gh = p.H / p.HKV;
  const int k0 = kblk * 128, kw = k0 + wave * 32, j = kw + l32;
  const bool key_ok = j < p.Sk;
  const long krow = ((long)b * p.HKV + hkv) * p.Sk + j;

  // query rows [r_lo, r_hi) that see some key of the block (small grids:
  // within the workgroup's row chunk rc, whose bounds are multiples of 128, so
  // that no row tile straddles two chunks)
  int r_lo = 0, r_hi = p.Sq;
  if (p.causal) r_lo = min(k0, p.Sq);
  if (p.window > 0) r_hi = min(p.Sq, k0 + 128 + p.window - 1);
  // (chunks in reverse, so that under a causal mask the latest rows, which
  // see the most key blocks, are dispatched first)
  const int rc = p.nrc - 1 - (int)blockIdx.y;
  if (p.nrc > 1) {
    r_lo = max(r_lo, rc * p.chunk_r);
    r_hi = min(r_hi, (rc + 1) * p.chunk_r);
  }
  const int rt0 = (r_lo / BM) * BM;
  const int n_rt = r_hi > r_lo ? (r_hi - rt0 + BM - 1) / BM : 0;
  const int n_cand = n_rt * gh;   // (query head, row tile) pairs
  // block mask: only the pairs whose mask byte is nonzero for one of the
  // block's two key columns are copied, listed in portions of up to
  // kBwdMaxList entries (query head << 22 | row tile << 2 | a flag per
  // column); a wavefront computes only where its own column's flag is set
  __shared__ unsigned tlist[Msk ? kBwdMaxList : 1];
  __shared__ int tsh[2];
  const int kb0 = k0 / kBwdMaskK;
  auto pair_flags = [&](int c) {
    const int hl = c / n_rt, r0 = rt0 + (c % n_rt) * BM;
    const unsigned char* m = bwd_mask_row(p, b, hkv * gh + hl, hkv, r0 / kBwdMaskQ);
    return (m[kb0] != 0 ? 1u : 0u) | (kb0 + 1 < p.bm_nkb && m[kb0 + 1] != 0 ? 2u : 0u);
  };
  auto list_portion = [&](int c0, int* next) {
    return bwd_build_list(
        c0, n_cand, tlist, tsh, wave, lane, pair_flags,
        [&](int c, unsigned f) { return (unsigned)(c / n_rt) << 22 | (unsigned)(c % n_rt) << 2 | f; },
        next);
  };
  int n_tiles = n_cand, c_next = n_cand;
  if constexpr (Msk) n_tiles = list_portion(0, &c_next);

  const int voff = T::dma_off(64 * wave * T::NIW + lane, kSwzB);
  // general form (views with strides, head dim dv): each copy instruction's
  // lane offset in full, or past the buffer's range for a chunk at or beyond
  // dim dv (zeros in LDS)
  const long long qr = Gen ? p.qs[2] : D, dor = Gen ? p.dos[2] : D;   // element row strides
  int pq_off[Gen ? T::NIW : 1], po_off[Gen ? T::NIW : 1];
  if constexpr (Gen) {
#pragma unroll
    for (int k = 0; k < T::NIW; ++k) {
      const int P = 64 * (wave * T::NIW + k) + lane, r = P / T::CPR;
      const int ck = (P % T::CPR) ^ T::swz_b(r);
      pq_off[k] = 8 * ck < p.dv ? r * (int)(2 * qr) + 16 * ck : kBwdOutOfRange;
      po_off[k] = 8 * ck < p.dv ? r * (int)(2 * dor) + 16 * ck : kBwdOutOfRange;
    }
  }
  // the tile rows' LSE (wave 0) and D (wave 1): loaded into xl with the
  // tile's copies and written to LDS by store_l at the start of the step that
  // works the tile, after the wait for those copies (converted there too, so
  // that no instruction waits for the load while the previous tile is worked)
  float xl = 0.f;
  auto store_l = [&](float* ld) __attribute__((always_inline)) {
    if (wave < 2 && lane < BM) {
      float x = xl;
      if (wave == 0) {
        x *= 1.4426950408889634f;             // base 2
        if (x == -INFINITY) x = INFINITY;     // a row with no visible key: P = 0
      }
      ld[wave * BM + lane] = x;
    }
  };
  auto issue = [&](int h, int r0, char* qd, char* od) {
    const long base = ((long)b * p.H + h) * p.Sq;
    const int r = r0 + lane;
    if (wave == 0) xl = r < p.Sq ? p.LSE[base + r] : INFINITY;
    else if (wave == 1) xl = r < p.Sq ? p.Dws[base + r] : 0.f;
    if constexpr (Gen) {
      const E* qb = (const E*)p.Q + b * p.qs[0] + h * p.qs[1] + r0 * qr;
      const E* ob = (const E*)p.dO + b * p.dos[0] + h * p.dos[1] + r0 * dor;
      // valid bytes from the tile's first row: up to the end of row Sq - 1
      const unsigned qbytes = (unsigned)min((long long)(p.Sq - r0 - 1) * 2 * qr + 2 * p.dv, kBwdMaxRange);
      const unsigned obytes = (unsigned)min((long long)(p.Sq - r0 - 1) * 2 * dor + 2 * p.dv, kBwdMaxRange);
#pragma unroll
      for (int k = 0; k < T::NIW; ++k) {
        const int off = (wave * T::NIW + k) * 1024;
        dma16(qb, qbytes, pq_off[k], qd + off);
        dma16(ob, obytes, po_off[k], od + off);
      }
    } else {
      const unsigned bytes = (unsigned)min((long)(p.Sq - r0) * T::ROW, 0x7fffffffL);
      const E* qb = (const E*)p.Q + (base + r0) * D;
      const E* ob = (const E*)p.dO + (base + r0) * D;
#pragma unroll
      for (int k = 0; k < T::NIW; ++k) {
        const int off = (wave * T::NIW + k) * 1024;
        dma16(qb, bytes, voff ^ T::dma_xor(k, kSwzB), qd + off);
        dma16(ob, bytes, voff ^ T::dma_xor(k, kSwzB), od + off);
      }
    }
  };
  // tiles in (query head, row tile) order, followed by a cursor: the head
  // and rows of the tile last issued, and the rows of the tile being worked
  // (no divisions per tile)
  int ih = hkv * gh, ir = rt0, cur_r0 = rt0;
  unsigned cur_fl = 3;   // (block mask: the current pair's column flags)
  const int rt_end = rt0 + n_rt * BM;
  auto from_list = [&](int t) {   // the cursor at list entry t
    const unsigned e = __builtin_amdgcn_readfirstlane(tlist[t]);
    ih = hkv * gh + (int)(e >> 22);
    ir = rt0 + (int)((e >> 2) & 0xfffffu) * BM;
    return e & 3u;
  };
  if constexpr (Msk)
    if (n_tiles > 0) cur_fl = from_list(0);
  cur_r0 = ir;
  if (n_tiles > 0) issue(ih, ir, qbuf0, obuf0);

  // K and V rows as B operands (k-slot (g, e) of step t is dim 16t + 8g + e)
  e16x8 kf[T::DC], vf[T::DC];
  const E* krp = Gen ? (const E*)p.K + b * p.ks[0] + hkv * p.ks[1] + j * p.ks[2]
                     : (const E*)p.K + krow * D;
  const E* vrp = Gen ? (const E*)p.V + b * p.vs[0] + hkv * p.vs[1] + j * p.vs[2]
                     : (const E*)p.V + krow * D;
#pragma unroll
  for (int t = 0; t < T::DC; ++t) {
    // (general form: the dims from dv on, a multiple of 16, are zeros)
    const bool ok = key_ok && (!Gen || 16 * t < p.dv);
    kf[t] = ok ? *(const e16x8*)(krp + 16 * t + 8 * g) : e16x8{};
    vf[t] = ok ? *(const e16x8*)(vrp + 16 * t + 8 * g) : e16x8{};
    if (p.neg_q) {   // negative scale: -K and |scale| (exact sign flips)
      u32x4 bits = __builtin_bit_cast(u32x4, kf[t]) ^ 0x80008000u;
      kf[t] = __builtin_bit_cast(e16x8, bits);
    }
  }
  const float sl = p.sl_abs;

  // operand offsets (tile-relative, first half; the second half is 32 rows on,
  // where both swizzles repeat): Q / dO rows, and their transposes
  const int qrow = perm_row(l32);
  int roff[T::DC];
#pragma unroll
  for (int t = 0; t < T::DC; ++t) roff[t] = qrow * T::ROW + (((2 * t + g) ^ T::swz_b(qrow)) << 4);
  const int blk = lane >> 4, li = lane & 15;
  const int vrow = 8 * g + (li >> 2);
  int troff[DBO];   // the output dim blocks DBO ob + db
#pragma unroll
  for (int db = 0; db < DBO; ++db) {
    const int chunk = 4 * (DBO * ob + db) + 2 * (blk & 1) + ((li & 3) >> 1);
    troff[db] = vrow * T::ROW + ((chunk ^ T::swz_b(vrow)) << 4) + 8 * (li & 1);
  }

  f32x16 dk[DBO], dv[DBO];
#pragma unroll
  for (int db = 0; db < DBO; ++db) dk[db] = dv[db] = f32x16{};

  auto step = [&](int t, const char* Qc, const char* Oc, float* Lc, char* Qn, char* On)
      __attribute__((always_inline)) {
    const int r0 = cur_r0;
    const unsigned fl = cur_fl;
    // (Lc was last read two steps back, before the previous step's barrier)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    store_l(Lc);
    __syncthreads();
    if (t + 1 < n_tiles) {
      if constexpr (Msk) {
        cur_fl = from_list(t + 1);
      } else {
        ir += BM;
        if (ir >= rt_end) {
          ir = rt0;
          ++ih;
        }
      }
      issue(ih, ir, Qn, On);
      cur_r0 = ir;
    }
    if (kw >= p.Sk || (p.causal && r0 + BM - 1 < kw) ||
        (p.window > 0 && r0 > kw + 31 + p.window - 1) || (Msk && !((fl >> (wave >> 1)) & 1u)))
      return;
    f32x16 sc[NH], dp[NH];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      sc[hh] = f32x16{};
      dp[hh] = f32x16{};
#pragma unroll
      for (int t2 = 0; t2 < T::DC; ++t2) {
        const e16x8 aq = *(const e16x8*)(Qc + roff[t2] + hh * HM * T::ROW);
        const e16x8 ao = *(const e16x8*)(Oc + roff[t2] + hh * HM * T::ROW);
        sc[hh] = X::mfma(aq, kf[t2], sc[hh]);
        dp[hh] = X::mfma(ao, vf[t2], dp[hh]);
      }
    }
    // operand reads four products ahead of their MFMAs (the scheduler's own
    // order read one or two ahead, and one wavefront per SIMD left the LDS
    // latency exposed)
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int k = 0; k < 2 * NH * T::DC - 4; ++k) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    const bool edge = (kw + 31 >= p.Sk) || (p.causal && r0 < kw + 31) ||
                      (p.window > 0 && r0 + BM - 1 > kw + p.window - 1);
    typename X::x8 pp[NH][2], ds[NH][2];
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      // element v holds query row r0 + 32 hh + 8g + c, c = 16 (v / 8) + v % 8
      f32x4 lq[4], dq4[4];
#pragma unroll
      for (int h4 = 0; h4 < 4; ++h4) {
        const int rr = HM * hh + 16 * (h4 >> 1) + 8 * g + 4 * (h4 & 1);
        lq[h4] = *(const f32x4*)(Lc + rr);
        dq4[h4] = *(const f32x4*)(Lc + BM + rr);
      }
      // the mask in one branch per half, as in the dQ kernel
      float xs[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) xs[v] = fmaf(sc[hh][v], sl, -lq[v >> 2][v & 3]);
      if (edge) {
        int jj = j;
        asm volatile("" : "+v"(jj));
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = r0 + HM * hh + 8 * g + 16 * (v >> 3) + (v & 7);
          const bool vis = jj < p.Sk && (!p.causal || jj <= r) && (p.window <= 0 || jj > r - p.window);
          xs[v] = vis ? xs[v] : -INFINITY;
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pr = __builtin_amdgcn_exp2f(xs[v]);
        pp[hh][v >> 3][v & 7] = (E)pr;
        ds[hh][v >> 3][v & 7] = (E)(pr * (dp[hh][v] - dq4[v >> 2][v & 3]));
      }
    }
#pragma unroll
    for (int hh = 0; hh < NH; ++hh)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        e16x8 ao[DBO], aq[DBO];
#pragma unroll
        for (int db = 0; db < DBO; ++db) {
          // (the second read is 4 rows on, where the XOR differs in bit 0)
          const int o = troff[db] + (HM * hh + 16 * c) * T::ROW;
          ao[db] = read_v_pair<e16x8>(Oc, o, (o + 4 * T::ROW) ^ 16);
          aq[db] = read_v_pair<e16x8>(Qc, o, (o + 4 * T::ROW) ^ 16);
        }
#pragma unroll
        for (int db = 0; db < DBO; ++db) {
          dv[db] = X::mfma(ao[db], pp[hh][c], dv[db]);
          dk[db] = X::mfma(aq[db], ds[hh][c], dk[db]);
        }
      }
  };

  for (;;) {
    for (int t = 0; t < n_tiles; t += 2) {
      step(t, qbuf0, obuf0, lbuf0, qbuf1, obuf1);
      if (t + 1 < n_tiles) step(t + 1, qbuf1, obuf1, lbuf1, qbuf0, obuf0);
    }
    if (c_next >= n_cand) break;
    if constexpr (Msk) {   // the next portion of the list
      n_tiles = list_portion(c_next, &c_next);
      if (n_tiles > 0) {
        cur_fl = from_list(0);
        cur_r0 = ir;
        issue(ih, ir, qbuf0, obuf0);
      }
    }
  }

  // lane holds dims DO ob + 32 db + 8 a + 4 g + (0..3) of key j (general
  // form: views with strides p.dks / p.dvs, written in their first dv dims;
  // row chunks: the unscaled partial sums of chunk rc)
  if (key_ok) {
    const bool part = p.nrc > 1;   // (contiguous rows of D dims, general form too)
    const long po = (long)rc * p.B * p.HKV * p.Sk * D;
    float* odk = (part  ? p.part_k + po + krow * D
                  : Gen ? p.dK + b * p.dks[0] + hkv * p.dks[1] + j * p.dks[2]
                        : p.dK + krow * D) + DO * ob;
    float* odv = (part  ? p.part_v + po + krow * D
                  : Gen ? p.dV + b * p.dvs[0] + hkv * p.dvs[1] + j * p.dvs[2]
                        : p.dV + krow * D) + DO * ob;
    const int dlim = (Gen && !part ? p.dv : D) - DO * ob;
    const float ks = part ? 1.f : p.scale;
#pragma unroll
    for (int db = 0; db < DBO; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        if (32 * db + 8 * a + 4 * g >= dlim) continue;
        const f32x4 k4 = {dk[db][4 * a] * ks, dk[db][4 * a + 1] * ks,
                          dk[db][4 * a + 2] * ks, dk[db][4 * a + 3] * ks};
        const f32x4 v4 = {dv[db][4 * a], dv[db][4 * a + 1], dv[db][4 * a + 2], dv[db][4 * a + 3]};
        *(f32x4*)(odk + 32 * db + 8 * a + 4 * g) = k4;
        *(f32x4*)(odv + 32 * db + 8 * a + 4 * g) = v4;
      }
  }
}

// Chunk sums: out = scale * sum over c < nch of part[c] (n4 float4 per part),
// in chunk order, for up to three tensors (dQ, dK, dV) in one launch, one per
// blockIdx.y.
struct SumJob {
  const float4* part;
  float4* out;
  float scale;
  long n4;
  int nch;
};
struct SumJobs {
  SumJob j[3];
};

__global__ __launch_bounds__(256) void sum_parts_kernel(SumJobs jobs) {
  const SumJob& jb = jobs.j[blockIdx.y];
  const float4* __restrict__ part = jb.part;
  float4* __restrict__ out = jb.out;
  const float scale = jb.scale;
  const long n4 = jb.n4;
  const int nch = jb.nch;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= n4) return;
  float4 acc = part[idx];
  for (int c = 1; c < nch; ++c) {
    const float4 x = part[c * n4 + idx];
    acc.x += x.x;
    acc.y += x.y;
    acc.z += x.z;
    acc.w += x.w;
  }
  out[idx] = make_float4(acc.x * scale, acc.y * scale, acc.z * scale, acc.w * scale);
}

// The jobs' reductions (n floats each, nch > 1) in one launch; none: nothing.
static hipError_t sum_parts(const SumJobs& jobs, int njobs, hipStream_t stream) {
  if (njobs == 0) return hipSuccess;
  long n4 = 0;
  for (int t = 0; t < njobs; ++t) n4 = n4 > jobs.j[t].n4 ? n4 : jobs.j[t].n4;
  const dim3 grid((unsigned)((n4 + 255) / 256), (unsigned)njobs);
  hipLaunchKernelGGL(sum_parts_kernel, grid, dim3(256), 0, stream, jobs);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  constexpr bool f32_mfma = sizeof(E) == 4 && bwd_f32_mfma(D);
  constexpr bool b16_mfma = sizeof(E) == 2 && (D == 64 || D == 128 || D == 256);
  // (MFMA dQ kernels: blockIdx.y = key chunk when p.nch > 1)
  if constexpr (b16_mfma) {
    const dim3 grid((unsigned)((long)p.B * p.H * p.n_qblk), (unsigned)p.nch);
    if (p.bmask)
      hipLaunchKernelGGL((bwd_dq_mfma_kernel<E, D, false, true>), grid, dim3(kBwdThreads), 0, stream, p);
    else if (p.gen)
      hipLaunchKernelGGL((bwd_dq_mfma_kernel<E, D, true, false>), grid, dim3(kBwdThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dq_mfma_kernel<E, D, false, false>), grid, dim3(kBwdThreads), 0, stream, p);
  } else if constexpr (f32_mfma) {
    const hipError_t e0 = launch_bwd_f32_mfma_dq(p, D, stream);
    if (e0 != hipSuccess) return e0;
  } else {
    constexpr int R = rows_per_group<D>(), GPB = kBwdThreads / bwd_lanes_per_row(D);
    const long groups = (long)p.B * p.H * ((p.Sq + R - 1) / R);
    const dim3 grid((unsigned)((groups + GPB - 1) / GPB), (unsigned)p.nch);
    if (p.bmask)
      hipLaunchKernelGGL((bwd_dq_kernel<E, D, true>), grid, dim3(kBwdThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<E, D, false>), grid, dim3(kBwdThreads), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (b16_mfma) {
    // (D = 256: two workgroups per key block, one per half of the output dims;
    // blockIdx.y: row chunk nrc - 1 - y when p.nrc > 1)
    const long kblocks = (long)p.B * p.HKV * ((p.Sk + 127) / 128) * (D == 256 ? 2 : 1);
    const dim3 grid((unsigned)kblocks, (unsigned)p.nrc);
    if (p.bmask)
      hipLaunchKernelGGL((bwd_dkdv_mfma_kernel<E, D, false, true>), grid, dim3(kBwdThreads), 0,
                         stream, p);
    else if (p.gen)
      hipLaunchKernelGGL((bwd_dkdv_mfma_kernel<E, D, true, false>), grid, dim3(kBwdThreads), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((bwd_dkdv_mfma_kernel<E, D, false, false>), grid, dim3(kBwdThreads), 0,
                         stream, p);
  } else if constexpr (f32_mfma) {
    const hipError_t e0 = launch_bwd_f32_mfma_dkdv(p, D, stream);
    if (e0 != hipSuccess) return e0;
  } else {
    constexpr int R = rows_per_group<D>(), GPB = kBwdThreads / bwd_lanes_per_row(D);
    const long groups = (long)p.B * p.HKV * ((p.Sk + R - 1) / R);
    const dim3 grid((unsigned)((groups + GPB - 1) / GPB), (unsigned)p.nch);
    if (p.bmask)
      hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, true>), grid, dim3(kBwdThreads), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<E, D, false>), grid, dim3(kBwdThreads), 0, stream, p);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the chunk sums, after both kernels, in one launch: dQ over its key chunks
  // (p.nch), dK and dV over the per-row kernels' key chunks (p.nch) or the
  // MFMA kernels' row chunks (p.nrc)
  SumJobs jobs = {};
  int njobs = 0;
  if (p.nch > 1)
    jobs.j[njobs++] = {(const float4*)p.part_q, (float4*)p.dQ, p.scale, (long)p.B * p.H * p.Sq * D / 4,
                       p.nch};
  const int nparts = b16_mfma || f32_mfma ? p.nrc : p.nch;
  if (nparts > 1) {
    const long nk4 = (long)p.B * p.HKV * p.Sk * D / 4;
    jobs.j[njobs++] = {(const float4*)p.part_k, (float4*)p.dK, p.scale, nk4, nparts};
    jobs.j[njobs++] = {(const float4*)p.part_v, (float4*)p.dV, 1.f, nk4, nparts};
  }
  return sum_parts(jobs, njobs, stream);
}

template <typename E>
static hipError_t launch_bwd_e(const BwdParams& p, int D, hipStream_t stream) {
  // (16-bit inputs reach here at their tile dims 64, 128, 256 only: other head
  // dims run those tiles in the general form or staged)
  if constexpr (sizeof(E) == 2) {
    switch (D) {
      case 64: return launch_bwd_t<E, 64>(p, stream);
      case 128: return launch_bwd_t<E, 128>(p, stream);
      case 256: return launch_bwd_t<E, 256>(p, stream);
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (D) {
      case 16: return launch_bwd_t<E, 16>(p, stream);
      case 32: return launch_bwd_t<E, 32>(p, stream);
      case 48: return launch_bwd_t<E, 48>(p, stream);
      case 64: return launch_bwd_t<E, 64>(p, stream);
      case 80: return launch_bwd_t<E, 80>(p, stream);
      case 96: return launch_bwd_t<E, 96>(p, stream);
      case 128: return launch_bwd_t<E, 128>(p, stream);
      case 256: return launch_bwd_t<E, 256>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
}

// Row copies around the staged backward (head dims padded to a kernel tile,
// or strided tensors). Rows are r = (b heads + h) S + i; row r of a strided
// view starts at base + b sb + h sh + i sr (byte strides, multiples of 16).
__device__ __forceinline__ long long view_row_offset(long r, int heads, int S, long long sb,
                                                     long long sh, long long sr) {
  const long bh = r / S;
  const long b = bh / heads;
  return b * sb + (bh - b * heads) * sh + (r - bh * S) * sr;
}

// One 16-byte chunk per thread: source row r of the view (its first cs
// chunks) -> contiguous row r of ct chunks, zeros past cs.
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* __restrict__ src,
                                                          uint4* __restrict__ dst, long rows,
                                                          int heads, int S, long long sb,
                                                          long long sh, long long sr, int cs,
                                                          int ct) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * ct) return;
  const long r = idx / ct;
  const int c = (int)(idx - r * ct);
  dst[idx] = c < cs ? *(const uint4*)(src + view_row_offset(r, heads, S, sb, sh, sr) + 16L * c)
                    : make_uint4(0u, 0u, 0u, 0u);
}

// One float4 per thread: the first cs float4 of contiguous row r (ct float4
// long) -> row r of the fp32 view.
__global__ __launch_bounds__(256) void scatter_rows_kernel(const float4* __restrict__ src,
                                                           char* __restrict__ dst, long rows,
                                                           int heads, int S, long long sb,
                                                           long long sh, long long sr, int ct,
                                                           int cs) {
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * cs) return;
  const long r = idx / cs;
  const int c = (int)(idx - r * cs);
  *(float4*)(dst + view_row_offset(r, heads, S, sb, sh, sr) + 16L * c) = src[r * ct + c];
}

hipError_t launch_gather_rows(const void* src, void* dst, int B, int heads, int S,
                              const long long st[3], int src_bytes, int dst_bytes,
                              hipStream_t stream) {
  const long rows = (long)B * heads * S;
  const long n = rows * (dst_bytes / 16);
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     (const char*)src, (uint4*)dst, rows, heads, S, st[0], st[1], st[2],
                     src_bytes / 16, dst_bytes / 16);
  return hipGetLastError();
}

hipError_t launch_scatter_rows(const float* src, void* dst, int B, int heads, int S,
                               const long long st[3], int dt, int dv, hipStream_t stream) {
  const long rows = (long)B * heads * S;
  const long n = rows * (dv / 4);
  hipLaunchKernelGGL(scatter_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     (const float4*)src, (char*)dst, rows, heads, S, st[0], st[1], st[2], dt / 4,
                     dv / 4);
  return hipGetLastError();
}

hipError_t launch_backward(const BwdParams& p, int dtype, int D, hipStream_t stream) {
  if (dtype == 0) return launch_bwd_e<float>(p, D, stream);
  if (dtype == 1) return launch_bwd_e<__bf16>(p, D, stream);
  if (dtype == 2) return launch_bwd_e<_Float16>(p, D, stream);
  return hipErrorInvalidValue;
}

}  // namespace fa

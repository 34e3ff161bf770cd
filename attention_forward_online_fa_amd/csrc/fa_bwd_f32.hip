// Backward kernels for fp32 inputs on MFMA (v_mfma_f32_32x32x2_f32) at head
// dims 32, 64, 96 and 128: the dQ / dK-dV split of the 16-bit MFMA kernels
// in fa_bwd.hip with the fp32 forward kernel's operand layouts. This file is
// compiled with the VGPR form of the MFMA instructions (-amdgpu-mfma-vgpr-form,
// set in build.py): at D = 128, one wavefront per SIMD, the compiler's default
// AGPR form moved every score and dP accumulator into VGPRs for the softmax,
// and the fp32 sliding-window backward ran 4.7 % slower with it; the 16-bit
// kernels, which keep the default, ran 2-5 % slower with the VGPR form.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_bwd.h"
#include "fa_bwd_device.h"
#include "fa_tile.h"

namespace fa {

// ------------------------------------------------------ fp32 inputs on MFMA
// The dQ and dK/dV products of fp32 inputs on v_mfma_f32_32x32x2_f32 (true
// fp32 products), with the operand layouts of the fp32 forward kernel: in a
// score product the k-slot g of step t is dim t + (D/2) g, so one 16-byte LDS
// read of a K (or Q) row feeds four steps; in an output product step u takes,
// in lane half g, the key (or query row) 8(u/4) + 4g + u%4 whose score element
// u the lane holds, and output row m of d-block db is dim (D/32) m + db, so
// one LDS read of a tile row feeds D/32 d-blocks. Tiles are 32 rows of fp32
// with rows padded to D + 4 floats (conflict-free reads in both patterns),
// staged through registers and double-buffered. A 32x32x2 fp32 MFMA takes
// 64 shader cycles, so the products dominate every step and one wavefront
// per SIMD keeps the pipe busy (D = 128: the accumulators live in AGPRs).
template <int D>
struct F32BwdTile {
  static constexpr int BN = 32;          // keys (dQ kernel) or query rows (dK/dV kernel) per tile
  static constexpr int DH = D / 2;       // k-steps of the score products
  static constexpr int DB = D / 32;      // 32-dim blocks of an output accumulator
  static constexpr int LD = D + 4;       // LDS row stride (floats)
  static constexpr int TILE_F = BN * LD;
  static constexpr int C4 = D / 4;       // float4 per row
  static constexpr int IT = BN * C4 / kBwdThreads;
  static_assert(BN * C4 % kBwdThreads == 0, "a tile splits evenly over the workgroup");
};

// DB consecutive floats at p (the output-product operands of one tile row).
template <int DB>
__device__ __forceinline__ void read_db(const float* p, float (&a)[DB]) {
  if constexpr (DB % 4 == 0) {
#pragma unroll
    for (int c4 = 0; c4 < DB / 4; ++c4) {
      const f32x4 x = *(const f32x4*)(p + 4 * c4);
      a[4 * c4] = x[0];
      a[4 * c4 + 1] = x[1];
      a[4 * c4 + 2] = x[2];
      a[4 * c4 + 3] = x[3];
    }
  } else {
#pragma unroll
    for (int e = 0; e < DB; ++e) a[e] = p[e];
  }
}

// At D = 256 the head dims are split over a pair of wavefronts (Q and dO rows
// of 128 dims per lane and the output accumulators of all 256 dims would not
// fit one wavefront's registers): wavefront w takes rows 32 (w / 2) of its
// workgroup and dims 128 (w % 2) .. +127 of every product. Each wavefront
// forms the scores and dP over its own dims; the pair adds its two partial
// tiles through LDS (the idle stage of the tile buffer), lower dims first, so
// that both hold the same sums, and each then accumulates the output products
// of its own dims. One workgroup covers 64 rows (dQ) or 64 keys (dK/dV).
template <int D>
struct F32BwdSplit {
  static constexpr bool SP = D == 256;
  static constexpr int HD = SP ? D / 2 : D;   // dims of one wavefront's products
  static constexpr int DHw = HD / 2;          // score k-steps per wavefront
  static constexpr int DBw = HD / 32;         // output d-blocks per wavefront
  static constexpr int RW = SP ? 64 : 128;    // query rows (dQ) or keys (dK/dV) per workgroup
  // block-mask list entries held in LDS at once (D = 256: what fits beside
  // the 130 KiB of tile buffers)
  static constexpr int LIST = SP ? 4096 : kBwdMaxList;
};

// Adds the pair's partial score and dP tiles (SP only): element v of s and dp
// goes to xb[(32 wave + v) 64 + lane] and [(32 wave + 16 + v) 64 + lane]; the
// second barrier keeps xb's stage from being refilled before the partner read it.
__device__ __forceinline__ void f32_pair_sum(float* xb, int wave, int lane, int hf, f32x16& s,
                                             f32x16& dp) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    xb[(32 * wave + v) * 64 + lane] = s[v];
    xb[(32 * wave + 16 + v) * 64 + lane] = dp[v];
  }
  __syncthreads();
  const int pw = wave ^ 1;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const float so = xb[(32 * pw + v) * 64 + lane];
    const float po = xb[(32 * pw + 16 + v) * 64 + lane];
    s[v] = hf ? so + s[v] : s[v] + so;
    dp[v] = hf ? po + dp[v] : dp[v] + po;
  }
  __syncthreads();
}

// dQ (and D_i) for fp32 inputs: 128 query rows per workgroup (64 at D = 256),
// K/V tiles of 32 keys; S^T = K Q^T, dP^T = V dO^T, dS = P (dP - D_i),
// dQ^T += K^T dS^T.
template <int D, bool Msk>
__global__ __launch_bounds__(kBwdThreads, D <= 64 ? 2 : 1)
void bwd_dq_f32_mfma_kernel(BwdParams p) {
  using T = F32BwdTile<D>;
  using W = F32BwdSplit<D>;
  static_assert(!W::SP || 4 * 32 * 64 <= T::TILE_F, "the pair sums fit one tile buffer");
  constexpr int BN = T::BN;
  __shared__ __attribute__((aligned(16))) float smem[2][2][T::TILE_F];   // [stage][K, V]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int rg = W::SP ? wave >> 1 : wave, hf = W::SP ? wave & 1 : 0;
  const int doff = hf * W::HD;   // first dim of the wavefront's products
  const int units = p.B * p.H;
  const int nqb = W::SP ? (p.Sq + W::RW - 1) / W::RW : p.n_qblk;
  const int qblk = nqb - 1 - (int)(blockIdx.x / units);   // heaviest query tiles first
  const int u = blockIdx.x % units;
  const int h = u % p.H, b = u / p.H;
  const int hkv = h / (p.H / p.HKV);
  const int q0 = qblk * W::RW, qw = q0 + rg * 32, i = qw + l32;
  const bool row_ok = i < p.Sq;
  const long row = ((long)b * p.H + h) * p.Sq + i;
  const float* Qh = (const float*)p.Q + ((long)b * p.H + h) * p.Sq * D;
  const float* Oh = (const float*)p.O + ((long)b * p.H + h) * p.Sq * D;
  const float* dOh = (const float*)p.dO + ((long)b * p.H + h) * p.Sq * D;
  const float* Kp = (const float*)p.K + ((long)b * p.HKV + hkv) * p.Sk * D;
  const float* Vp = (const float*)p.V + ((long)b * p.HKV + hkv) * p.Sk * D;

  int lo = 0, hi = p.Sk;
  if (p.causal) hi = min(hi, min(q0 + W::RW, p.Sq));
  if (p.window > 0) lo = max(0, q0 - p.window + 1);
  if (p.nch > 1) {   // key chunk blockIdx.y (chunk_q: a multiple of BN)
    lo = max(lo, (int)blockIdx.y * p.chunk_q);
    hi = min(hi, ((int)blockIdx.y + 1) * p.chunk_q);
  }
  const int t0 = (lo / BN) * BN;
  const int n_cand = hi > lo ? (hi - t0 + BN - 1) / BN : 0;   // key tiles of the range
  // block mask: only the tiles whose mask byte is nonzero, listed in portions
  __shared__ unsigned tlist[Msk ? W::LIST : 1];
  __shared__ int tsh[2];
  int n_tiles = n_cand, c_next = n_cand;
  const unsigned char* mrow = nullptr;
  auto list_portion = [&](int c0) {
    return bwd_build_list<W::LIST>(
        c0, n_cand, tlist, tsh, wave, lane,
        [&](int t) { return mrow[(t0 + t * BN) / kBwdMaskK] != 0 ? 1u : 0u; },
        [](int t, unsigned) { return (unsigned)t; },
        &c_next);
  };
  if constexpr (Msk) {
    mrow = bwd_mask_row(p, b, h, hkv, q0 / kBwdMaskQ);
    n_tiles = list_portion(0);
  }
  auto tile_kt = [&](int t) {   // first key of the t-th tile visited
    if constexpr (Msk)
      return t0 + BN * (int)__builtin_amdgcn_readfirstlane(tlist[t]);
    else
      return t0 + t * BN;
  };

  // Q and dO rows (dims doff + t + (HD/2) g), D_i over the lane's dims and its
  // partner's (at D = 256 over dims 128 g .. +127 of the whole row, so that
  // both wavefronts of a pair form the same D_i)
  float qf[W::DHw], dof[W::DHw];
  float dd = 0.f;
#pragma unroll
  for (int t4 = 0; t4 < W::DHw / 4; ++t4) {
    const long off = (long)i * D + doff + W::DHw * g + 4 * t4;
    const f32x4 qv = row_ok ? *(const f32x4*)(Qh + off) : f32x4{};
    const f32x4 dv = row_ok ? *(const f32x4*)(dOh + off) : f32x4{};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[4 * t4 + e] = qv[e];
      dof[4 * t4 + e] = dv[e];
    }
    if constexpr (!W::SP) {
      const f32x4 ov = row_ok ? *(const f32x4*)(Oh + off) : f32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) dd = fmaf(dv[e], ov[e], dd);
    }
  }
  if constexpr (W::SP) {
#pragma unroll 4
    for (int t4 = 0; t4 < D / 8; ++t4) {
      const long off = (long)i * D + (D / 2) * g + 4 * t4;
      const f32x4 dv = row_ok ? *(const f32x4*)(dOh + off) : f32x4{};
      const f32x4 ov = row_ok ? *(const f32x4*)(Oh + off) : f32x4{};
#pragma unroll
      for (int e = 0; e < 4; ++e) dd = fmaf(dv[e], ov[e], dd);
    }
  }
  const float Di = dd + __shfl_xor(dd, 32);
  // base-2 LSE; +inf for rows past Sq or with no visible key, so that P = 0
  float L2 = row_ok ? p.LSE[row] * kLog2e : INFINITY;
  if (L2 == -INFINITY) L2 = INFINITY;
  const float sl = p.scale * kLog2e;

  f32x4 kreg[T::IT], vreg[T::IT];
  auto load_tile = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < T::IT; ++it) {
      const int c = tid + it * kBwdThreads, r = c / T::C4, c4 = c % T::C4;
      const bool ok = kt + r < p.Sk;
      kreg[it] = ok ? *(const f32x4*)(Kp + (long)(kt + r) * D + 4 * c4) : f32x4{};
      vreg[it] = ok ? *(const f32x4*)(Vp + (long)(kt + r) * D + 4 * c4) : f32x4{};
    }
  };
  auto store_tile = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < T::IT; ++it) {
      const int c = tid + it * kBwdThreads, r = c / T::C4, c4 = c % T::C4;
      *(f32x4*)(&smem[st][0][r * T::LD + 4 * c4]) = kreg[it];
      *(f32x4*)(&smem[st][1][r * T::LD + 4 * c4]) = vreg[it];
    }
  };
  if (n_tiles > 0) {
    load_tile(tile_kt(0));
    store_tile(0);
  }
  __syncthreads();

  f32x16 dq[W::DBw];
#pragma unroll
  for (int db = 0; db < W::DBw; ++db) dq[db] = f32x16{};

  for (;;) {
  for (int it = 0; it < n_tiles; ++it) {
    const int kt = tile_kt(it);
    const float* Ks = smem[it & 1][0];
    const float* Vs = smem[it & 1][1];
    if (it + 1 < n_tiles) load_tile(tile_kt(it + 1));
    const bool skip = qw >= p.Sq || (p.causal && kt > qw + 31) ||
                      (p.window > 0 && kt + BN - 1 < qw - p.window + 1);
    f32x16 s = f32x16{}, dp = f32x16{};
    if (!skip) {
      const float* krow = Ks + l32 * T::LD + doff + W::DHw * g;
      const float* vrow = Vs + l32 * T::LD + doff + W::DHw * g;
#pragma unroll
      for (int t4 = 0; t4 < W::DHw / 4; ++t4) {
        const f32x4 a = *(const f32x4*)(krow + 4 * t4);
        const f32x4 c = *(const f32x4*)(vrow + 4 * t4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[4 * t4 + e], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x2f32(c[e], dof[4 * t4 + e], dp, 0, 0, 0);
        }
      }
    }
    // (every wavefront reaches the pair sum's barriers; a skipped pair adds zeros)
    if constexpr (W::SP) f32_pair_sum(smem[(it + 1) & 1][0], wave, lane, hf, s, dp);
    if (!skip) {
      // element v holds key kt + 8 (v / 4) + 4 g + v % 4 of row i
      const bool edge = (kt + BN > p.Sk) || (p.causal && kt + BN - 1 > qw) ||
                        (p.window > 0 && kt < qw + 31 - p.window + 1);
      float ds[16];
      if constexpr (D <= 64) {
        // the mask in one branch, as in the 16-bit kernels (at D = 128, one
        // wavefront per SIMD, the test inside the loop measured faster)
        float xs[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) xs[v] = fmaf(s[v], sl, -L2);
        if (edge) {
          int ii = i;
          asm volatile("" : "+v"(ii));
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int j = kt + 8 * (v >> 2) + 4 * g + (v & 3);
            const bool vis = j < p.Sk && (!p.causal || j <= ii) && (p.window <= 0 || j > ii - p.window);
            xs[v] = vis ? xs[v] : -INFINITY;
          }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) ds[v] = __builtin_amdgcn_exp2f(xs[v]) * (dp[v] - Di);
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = fmaf(s[v], sl, -L2);
          if (edge) {
            const int j = kt + 8 * (v >> 2) + 4 * g + (v & 3);
            const bool vis = j < p.Sk && (!p.causal || j <= i) && (p.window <= 0 || j > i - p.window);
            x = vis ? x : -INFINITY;
          }
          ds[v] = __builtin_amdgcn_exp2f(x) * (dp[v] - Di);
        }
      }
      // dQ^T += K^T dS^T: step u takes key 8 (u / 4) + 4 g + u % 4
#pragma unroll
      for (int u2 = 0; u2 < 16; ++u2) {
        float ka[W::DBw];
        read_db<W::DBw>(Ks + (8 * (u2 >> 2) + 4 * g + (u2 & 3)) * T::LD + doff + W::DBw * l32, ka);
#pragma unroll
        for (int db = 0; db < W::DBw; ++db)
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[db], ds[u2], dq[db], 0, 0, 0);
      }
    }
    if (it + 1 < n_tiles) store_tile((it + 1) & 1);
    __syncthreads();
  }
    if (c_next >= n_cand) break;
    if constexpr (Msk) {   // the next portion of the list
      n_tiles = list_portion(c_next);
      if (n_tiles > 0) {
        load_tile(tile_kt(0));
        store_tile(0);
      }
      __syncthreads();
    }
  }

  // element v of block db: dim doff + (HD/32)(8 (v / 4) + 4 g + v % 4) + db of
  // row i; a key chunk writes its unscaled partial sums
  if (row_ok) {
    const bool part = p.nch > 1;
    const float sc = part ? 1.f : p.scale;
    float* dst = part ? p.part_q + ((long)blockIdx.y * p.B * p.H * p.Sq + row) * D
                      : p.dQ + row * D;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float* d0 = dst + doff + W::DBw * (8 * (v >> 2) + 4 * g + (v & 3));
      if constexpr (W::DBw % 4 == 0) {
#pragma unroll
        for (int c4 = 0; c4 < W::DBw / 4; ++c4) {
          const f32x4 x = {dq[4 * c4][v] * sc, dq[4 * c4 + 1][v] * sc,
                           dq[4 * c4 + 2][v] * sc, dq[4 * c4 + 3][v] * sc};
          *(f32x4*)(d0 + 4 * c4) = x;
        }
      } else {
#pragma unroll
        for (int db = 0; db < W::DBw; ++db) d0[db] = dq[db][v] * sc;
      }
    }
    if (g == 0 && hf == 0 && blockIdx.y == 0) p.Dws[row] = Di;
  }
}

// dK and dV for fp32 inputs: a workgroup owns 128 keys (4 wavefronts x 32, a
// lane owns one key; at D = 256 64 keys, each on a wavefront pair) with K and
// V rows in registers, and walks 32-row tiles of Q and dO (with the rows'
// base-2 LSE and D_i) over every query head of the kv head: S = Q K^T,
// dP = dO V^T, dS = P (dP - D), dV^T += dO^T P, dK^T += Q^T dS.
template <int D, bool Msk>
__global__ __launch_bounds__(kBwdThreads, D <= 64 && !Msk ? 2 : 1)   // (masked: the list state spills at two)
void bwd_dkdv_f32_mfma_kernel(BwdParams p) {
  using T = F32BwdTile<D>;
  using W = F32BwdSplit<D>;
  constexpr int BM = T::BN;   // query rows per tile
  __shared__ __attribute__((aligned(16))) float smem[2][2][T::TILE_F];   // [stage][Q, dO]
  __shared__ __attribute__((aligned(16))) float lds_l[2][2][BM];         // [stage][L2, D]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int units = p.B * p.HKV;
  const int rg = W::SP ? wave >> 1 : wave, hf = W::SP ? wave & 1 : 0;
  const int doff = hf * W::HD;   // first dim of the wavefront's products
  const int kblk = blockIdx.x / units;   // ascending: under a causal mask the first keys see most rows
  const int u = blockIdx.x % units;
  const int hkv = u % p.HKV, b = u / p.HKV;
  const int gh = p.H / p.HKV;
  const int k0 = kblk * W::RW, kw = k0 + rg * 32, j = kw + l32;
  const bool key_ok = j < p.Sk;
  const long krow = ((long)b * p.HKV + hkv) * p.Sk + j;

  // query rows [r_lo, r_hi) that see some key of the block (small grids:
  // within the workgroup's row chunk rc, bounds multiples of 128)
  int r_lo = 0, r_hi = p.Sq;
  if (p.causal) r_lo = min(k0, p.Sq);
  if (p.window > 0) r_hi = min(p.Sq, k0 + W::RW + p.window - 1);
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
  // block's two key columns (D = 256: its one column, flagged for both row
  // groups), listed in portions (query head << 22 | row tile << 2 | a flag per
  // column); a wavefront computes only under its column's flag
  __shared__ unsigned tlist[Msk ? W::LIST : 1];
  __shared__ int tsh[2];
  const int kb0 = k0 / kBwdMaskK;
  auto pair_flags = [&](int c) {
    const int hl = c / n_rt, r0 = rt0 + (c % n_rt) * BM;
    const unsigned char* m = bwd_mask_row(p, b, hkv * gh + hl, hkv, r0 / kBwdMaskQ);
    if constexpr (W::SP) return m[kb0] != 0 ? 3u : 0u;
    return (m[kb0] != 0 ? 1u : 0u) | (kb0 + 1 < p.bm_nkb && m[kb0 + 1] != 0 ? 2u : 0u);
  };
  int n_tiles = n_cand, c_next = n_cand;
  auto list_portion = [&](int c0) {
    return bwd_build_list<W::LIST>(
        c0, n_cand, tlist, tsh, wave, lane, pair_flags,
        [&](int c, unsigned f) { return (unsigned)(c / n_rt) << 22 | (unsigned)(c % n_rt) << 2 | f; },
        &c_next);
  };
  if constexpr (Msk) n_tiles = list_portion(0);
  // query head, first row and column flags of the t-th pair visited
  auto tile_at = [&](int t, int& hq, int& r0) {
    if constexpr (Msk) {
      const unsigned e = __builtin_amdgcn_readfirstlane(tlist[t]);
      hq = hkv * gh + (int)(e >> 22);
      r0 = rt0 + (int)((e >> 2) & 0xfffffu) * BM;
      return e & 3u;
    } else {
      hq = hkv * gh + t / n_rt;
      r0 = rt0 + (t % n_rt) * BM;
      return 3u;
    }
  };

  // K and V rows of key j (dims doff + t + (HD/2) g)
  float kf[W::DHw], vf[W::DHw];
#pragma unroll
  for (int t4 = 0; t4 < W::DHw / 4; ++t4) {
    const long off = krow * D + doff + W::DHw * g + 4 * t4;
    const f32x4 kv = key_ok ? *(const f32x4*)((const float*)p.K + off) : f32x4{};
    const f32x4 vv = key_ok ? *(const f32x4*)((const float*)p.V + off) : f32x4{};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kf[4 * t4 + e] = kv[e];
      vf[4 * t4 + e] = vv[e];
    }
  }
  const float sl = p.scale * kLog2e;
  // vmcnt(0): the K/V loads land here. Left to the compiler, the wait for them
  // sat before the loop's first MFMA, where it also waited for the next tile's
  // register loads issued just before (the compiler's count merges the
  // loop-entry and back-edge paths).
  __builtin_amdgcn_s_waitcnt(0x0F70);

  f32x4 qreg[T::IT], oreg[T::IT];
  float lreg = 0.f;
  auto load_tile = [&](int t) __attribute__((always_inline)) {
    int hq, r0;
    tile_at(t, hq, r0);
    const long base = ((long)b * p.H + hq) * p.Sq;
#pragma unroll
    for (int it = 0; it < T::IT; ++it) {
      const int c = tid + it * kBwdThreads, r = c / T::C4, c4 = c % T::C4;
      const bool ok = r0 + r < p.Sq;
      const long off = (base + r0 + r) * D + 4 * c4;
      qreg[it] = ok ? *(const f32x4*)((const float*)p.Q + off) : f32x4{};
      oreg[it] = ok ? *(const f32x4*)((const float*)p.dO + off) : f32x4{};
    }
    // the tile rows' LSE (threads 0 .. 31) and D (threads 32 .. 63), taken
    // to base 2 by store_tile (converting here would wait for the load, and
    // with it for every copy of the tile, before the current tile is worked)
    if (tid < 2 * BM) {
      const int r = r0 + (tid & (BM - 1));
      if (tid < BM) lreg = r < p.Sq ? p.LSE[base + r] : INFINITY;
      else lreg = r < p.Sq ? p.Dws[base + r] : 0.f;
    }
  };
  auto store_tile = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < T::IT; ++it) {
      const int c = tid + it * kBwdThreads, r = c / T::C4, c4 = c % T::C4;
      *(f32x4*)(&smem[st][0][r * T::LD + 4 * c4]) = qreg[it];
      *(f32x4*)(&smem[st][1][r * T::LD + 4 * c4]) = oreg[it];
    }
    if (tid < 2 * BM) {
      float x = lreg;
      if (tid < BM) {
        x *= kLog2e;
        if (x == -INFINITY) x = INFINITY;   // a row with no visible key: P = 0
      }
      lds_l[st][tid / BM][tid & (BM - 1)] = x;
    }
  };
  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  f32x16 dk[W::DBw], dv[W::DBw];
#pragma unroll
  for (int db = 0; db < W::DBw; ++db) dk[db] = dv[db] = f32x16{};

  for (;;) {
  for (int t = 0; t < n_tiles; ++t) {
    int hq_unused, r0;
    const unsigned fl = tile_at(t, hq_unused, r0);
    const float* Qs = smem[t & 1][0];
    const float* Os = smem[t & 1][1];
    const float* Ls = lds_l[t & 1][0];
    const float* Dl = lds_l[t & 1][1];
    if (t + 1 < n_tiles) load_tile(t + 1);
    const bool skip = kw >= p.Sk || (p.causal && r0 + BM - 1 < kw) ||
                      (p.window > 0 && r0 > kw + 31 + p.window - 1) ||
                      (Msk && !((fl >> (wave >> 1)) & 1u));
    f32x16 s = f32x16{}, dp = f32x16{};
    if (!skip) {
      const float* qrow = Qs + l32 * T::LD + doff + W::DHw * g;
      const float* orow = Os + l32 * T::LD + doff + W::DHw * g;
#pragma unroll
      for (int t4 = 0; t4 < W::DHw / 4; ++t4) {
        const f32x4 a = *(const f32x4*)(qrow + 4 * t4);
        const f32x4 c = *(const f32x4*)(orow + 4 * t4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], kf[4 * t4 + e], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x2f32(c[e], vf[4 * t4 + e], dp, 0, 0, 0);
        }
      }
    }
    // (every wavefront reaches the pair sum's barriers; a skipped pair adds zeros)
    if constexpr (W::SP) f32_pair_sum(smem[(t + 1) & 1][0], wave, lane, hf, s, dp);
    if (!skip) {
      // element v holds query row r0 + 8 (v / 4) + 4 g + v % 4 of key j
      const bool edge = (kw + 31 >= p.Sk) || (p.causal && r0 < kw + 31) ||
                        (p.window > 0 && r0 + BM - 1 > kw + p.window - 1);
      float pr[16], ds[16];
      if constexpr (D <= 64) {   // the mask in one branch, as in the dQ kernel
        float xs[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) xs[v] = fmaf(s[v], sl, -Ls[8 * (v >> 2) + 4 * g + (v & 3)]);
        if (edge) {
          int jj = j;
          asm volatile("" : "+v"(jj));
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = r0 + 8 * (v >> 2) + 4 * g + (v & 3);
            const bool vis = jj < p.Sk && (!p.causal || jj <= r) && (p.window <= 0 || jj > r - p.window);
            xs[v] = vis ? xs[v] : -INFINITY;
          }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          pr[v] = __builtin_amdgcn_exp2f(xs[v]);
          ds[v] = pr[v] * (dp[v] - Dl[8 * (v >> 2) + 4 * g + (v & 3)]);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rr = 8 * (v >> 2) + 4 * g + (v & 3);
          float x = fmaf(s[v], sl, -Ls[rr]);
          if (edge) {
            const int r = r0 + rr;
            const bool vis = j < p.Sk && (!p.causal || j <= r) && (p.window <= 0 || j > r - p.window);
            x = vis ? x : -INFINITY;
          }
          pr[v] = __builtin_amdgcn_exp2f(x);
          ds[v] = pr[v] * (dp[v] - Dl[rr]);
        }
      }
      // dV^T += dO^T P, dK^T += Q^T dS: step u takes row 8 (u / 4) + 4 g + u % 4
#pragma unroll
      for (int u2 = 0; u2 < 16; ++u2) {
        const int rr = 8 * (u2 >> 2) + 4 * g + (u2 & 3);
        float oa[W::DBw], qa[W::DBw];
        read_db<W::DBw>(Os + rr * T::LD + doff + W::DBw * l32, oa);
        read_db<W::DBw>(Qs + rr * T::LD + doff + W::DBw * l32, qa);
#pragma unroll
        for (int db = 0; db < W::DBw; ++db) {
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(oa[db], pr[u2], dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[db], ds[u2], dk[db], 0, 0, 0);
        }
      }
    }
    if (t + 1 < n_tiles) store_tile((t + 1) & 1);
    __syncthreads();
  }
    if (c_next >= n_cand) break;
    if constexpr (Msk) {   // the next portion of the list
      n_tiles = list_portion(c_next);
      if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
      }
      __syncthreads();
    }
  }

  // element v of block db: dim doff + (HD/32)(8 (v / 4) + 4 g + v % 4) + db of
  // key j (row chunks: the unscaled partial sums of chunk rc)
  if (key_ok) {
    const bool part = p.nrc > 1;
    const long po = (long)rc * p.B * p.HKV * p.Sk * D;
    float* odk = (part ? p.part_k + po : p.dK) + krow * D;
    float* odv = (part ? p.part_v + po : p.dV) + krow * D;
    const float ks = part ? 1.f : p.scale;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = doff + W::DBw * (8 * (v >> 2) + 4 * g + (v & 3));
      if constexpr (W::DBw % 4 == 0) {
#pragma unroll
        for (int c4 = 0; c4 < W::DBw / 4; ++c4) {
          const f32x4 k4 = {dk[4 * c4][v] * ks, dk[4 * c4 + 1][v] * ks,
                            dk[4 * c4 + 2][v] * ks, dk[4 * c4 + 3][v] * ks};
          const f32x4 v4 = {dv[4 * c4][v], dv[4 * c4 + 1][v], dv[4 * c4 + 2][v], dv[4 * c4 + 3][v]};
          *(f32x4*)(odk + m + 4 * c4) = k4;
          *(f32x4*)(odv + m + 4 * c4) = v4;
        }
      } else {
#pragma unroll
        for (int db = 0; db < W::DBw; ++db) {
          odk[m + db] = dk[db][v] * ks;
          odv[m + db] = dv[db][v];
        }
      }
    }
  }
}

template <int D>
static hipError_t launch_dq_t(const BwdParams& p, hipStream_t stream) {
  using W = F32BwdSplit<D>;
  const long nqb = W::SP ? (p.Sq + W::RW - 1) / W::RW : p.n_qblk;
  const dim3 grid((unsigned)((long)p.B * p.H * nqb), (unsigned)p.nch);
  if (p.bmask)
    hipLaunchKernelGGL((bwd_dq_f32_mfma_kernel<D, true>), grid, dim3(kBwdThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((bwd_dq_f32_mfma_kernel<D, false>), grid, dim3(kBwdThreads), 0, stream, p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dkdv_t(const BwdParams& p, hipStream_t stream) {
  // (blockIdx.y: row chunk nrc - 1 - y when p.nrc > 1)
  using W = F32BwdSplit<D>;
  const dim3 grid((unsigned)((long)p.B * p.HKV * ((p.Sk + W::RW - 1) / W::RW)), (unsigned)p.nrc);
  if (p.bmask)
    hipLaunchKernelGGL((bwd_dkdv_f32_mfma_kernel<D, true>), grid, dim3(kBwdThreads), 0, stream, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_f32_mfma_kernel<D, false>), grid, dim3(kBwdThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_bwd_f32_mfma_dq(const BwdParams& p, int D, hipStream_t stream) {
  switch (D) {
    case 32: return launch_dq_t<32>(p, stream);
    case 64: return launch_dq_t<64>(p, stream);
    case 96: return launch_dq_t<96>(p, stream);
    case 128: return launch_dq_t<128>(p, stream);
    case 256: return launch_dq_t<256>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_f32_mfma_dkdv(const BwdParams& p, int D, hipStream_t stream) {
  switch (D) {
    case 32: return launch_dkdv_t<32>(p, stream);
    case 64: return launch_dkdv_t<64>(p, stream);
    case 96: return launch_dkdv_t<96>(p, stream);
    case 128: return launch_dkdv_t<128>(p, stream);
    case 256: return launch_dkdv_t<256>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa

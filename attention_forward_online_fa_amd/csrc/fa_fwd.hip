// Fused attention forward pass for gfx950 (MI355X): tiled QK^T and PV on
// MFMA with an online softmax between them, one query tile per workgroup.
//
// Method (the online-softmax recurrence of the forge flash_attention.metal
// header comment, applied per key tile instead of per key): for each K/V tile
//   S     = scale * Q K^T                (MFMA, fp32 accumulate)
//   m_new = max(m, rowmax(S))
//   P     = exp(S - m_new),  corr = exp(m - m_new)
//   l     = l * corr + rowsum(P),  O = O * corr + P V   (MFMA)
// and at the end O /= l, LSE = m + log(l) (the log-sum-exp output of the
// rustytorch flash_attention_forward.metal kernel). Scores are carried in
// base-2 units (scale * log2 e folded into one multiply) so every exponential
// is a single v_exp_f32. m starts at -inf; a row whose keys so far are all
// masked uses 0 as the shift so that exp(-inf - (-inf)) never appears (the
// NaN hazard named in the forge header comment). Rows that never see a key
// end with l = 0 and are written as O = 0, LSE = -inf.
//
// Whole K/V tiles above the causal diagonal or before the sliding window are
// never visited; only tiles that straddle a mask edge (or the end of the key
// axis) pay the per-element test, as the forge forward kernel does with its
// kb_lim / jb_begin bounds.
//
// Work decomposition (gfx950): a workgroup is 4 wavefronts x 32 query rows.
// The 16-bit kernel packs the query heads that share one K/V head into a
// workgroup (hp = 4 or 2 heads, each with 128 / hp rows; one head and 128 rows
// when the group size is odd, and under a block mask), so all of its
// wavefronts see the same key range; the fp32 kernel takes 128 rows of one
// (batch, head). Each wavefront keeps its 32 query rows in
// registers as the MFMA B operand and computes S^T = K Q^T, so a lane owns one
// query row (column of S^T) and half of the tile's keys: row max and row sum
// are in-lane plus one exchange with lane ^ 32. The P tile then feeds the
// second MFMA (O^T = V^T P^T) straight from registers; V stays row-major in
// LDS and the 16-bit kernel reads it transposed (ds_read_b64_tr_b16), the fp32
// kernel with its dims spread over the accumulator blocks. K/V tiles are
// double-buffered in LDS: the next tile's copy is in flight while the current
// tile is computed.
//
// Workgroup order: heaviest query tiles (latest rows under a causal mask)
// first; when the number of (batch, head, split) units is a multiple of 8 the
// blocks are remapped so that the query heads sharing one K/V head land on the
// same XCD (MI355X dispatches workgroups round-robin over its 8 XCDs, each
// with its own L2). The fp32 kernel can also run persistently: a fixed number
// of workgroups, each over a host-computed list of (query tile, key split)
// items (Params::sched).
#include "fa_fwd_common.h"
#include "fa_kernels.h"
#include "fa_tile.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// ============================================================ block masks
// Block-sparse form: the key tiles t in [0, n) of a workgroup's range (tile t
// holds keys t0 + t bn ..) whose mask byte is nonzero, in order, go to
// list[]; returns how many (uniform). Wave 0 compacts 64 candidate tiles per
// round with a ballot; the others wait at the barrier. The workgroup then
// visits only these tiles: their copies and their compute.
__device__ __forceinline__ int build_tile_list(const unsigned char* mrow, int t0, int n, int bn,
                                               unsigned short* list, int* count, int wave,
                                               int lane) {
  if (wave == 0) {
    int cnt = 0;
    for (int base = 0; base < n; base += 64) {
      const int t = base + lane;
      const bool vis = t < n && mrow[(t0 + t * bn) / kMaskBlockK] != 0;
      const unsigned long long bal = __ballot(vis);
      if (vis) list[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = (unsigned short)t;
      cnt += __popcll(bal);
    }
    if (lane == 0) *count = cnt;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*count);
}

__device__ __forceinline__ const unsigned char* mask_row(const Params& p, int b, int h, int hkv,
                                                         int qblk) {
  return p.bmask + b * p.bm_sb + (p.bm_by_kv ? hkv : h) * p.bm_sh + (long long)qblk * p.bm_nkb;
}

// ================================================= 16-bit inputs (bf16, fp16)
// (operand layouts, tile geometry and copies: fa_tile.h)
constexpr float kRowSumLimit = 1.8446744e19f;   // 2^64: row-sum bound that triggers a rescale

// E = __bf16 or _Float16 (inputs, O and the rounded P); fp32 accumulation,
// softmax and LSE either way. Form kFormStrided: Q, K, V and O are addressed
// through p.qs .. p.os (batch, head, row strides); otherwise they are
// contiguous. Form kFormBlockSparse: only the key tiles whose block-mask
// byte is nonzero are copied and computed. Form kFormPadded: strided tensors
// with rows of DV < D elements (DV = p.dv, a multiple of 16). The K/V tiles
// keep the D-dim layout with zeros from dim DV on (chunks whose copy offsets
// are sent out of the buffer's range); Q^T takes only the DV / 16 k-steps of
// real dims and O^T only the ceil(DV / 32) dim blocks that hold real dims.
template <typename E, int D, int BN, int Form, int DV = D>
__global__ __launch_bounds__(kThreads, (D == 128 ? 3 : 2))
void fwd_16b_kernel(Params p) {
  constexpr bool Pad = Form == kFormPadded;
  static_assert(Pad ? (DV % 16 == 0 && DV < D) : DV == D, "padded head dims only");
  constexpr int DC = DV / 16;             // k-steps of the S MFMA over real dims
  constexpr int DB = (DV + 31) / 32;      // O^T dim blocks holding real dims
  constexpr bool Strided = Form == kFormStrided || Pad, Sparse = Form == kFormBlockSparse;
  static_assert(kMaskBlockK % BN == 0, "a key tile lies inside one mask block");
  using T = Bf16Tile<D, BN>;
  using X = Elt<E>;
  typedef typename X::x8 e16x8;
  // K and V tiles double-buffered; four separate objects let the compiler see
  // that the copy filling one buffer never aliases the reads of another (it
  // would otherwise wait for the in-flight copy before reading).
  __shared__ __attribute__((aligned(1024))) char kbuf0[T::TILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1[T::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0[T::TILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1[T::TILE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wavefront
  const int l32 = lane & 31, g = lane >> 5;
  const Tile w = map_tile(p);
  // wavefront -> (head w.h + wave % hp, rows q0 + 32 (wave / hp) ..)
  const int bm = p.bm;                      // query rows per workgroup: kBlockM / hp
  const int h = w.h + wave % p.hp;
  const int q0 = w.qblk * bm;
  const int qw = q0 + (wave / p.hp) * 32;
  const int i = qw + l32;

  const E* Qp;
  const E* Kp;
  const E* Vp;
  long long qr = D;   // element row strides
  int krb = T::ROW, vrb = T::ROW;   // K / V row strides in bytes (strided: multiples of ROW)
  if constexpr (Strided) {
    Qp = (const E*)p.Q + w.b * p.qs[0] + h * p.qs[1];
    Kp = (const E*)p.K + w.b * p.ks[0] + w.hkv * p.ks[1];
    Vp = (const E*)p.V + w.b * p.vs[0] + w.hkv * p.vs[1];
    qr = p.qs[2];
    krb = (int)(p.ks[2] * 2);
    vrb = (int)(p.vs[2] * 2);
  } else {
    Qp = (const E*)p.Q + (size_t)(w.b * p.H + h) * p.Sq * D;
    Kp = (const E*)p.K + (size_t)(w.b * p.HKV + w.hkv) * p.Sk * D;
    Vp = (const E*)p.V + (size_t)(w.b * p.HKV + w.hkv) * p.Sk * D;
  }

  int lo, hi;
  key_range(p, q0, bm, w.split, lo, hi);
  const int t0 = (lo / BN) * BN;
  int n_tiles = hi > lo ? (hi - t0 + BN - 1) / BN : 0;
  __shared__ unsigned short tlist[Sparse ? kMaxListTiles : 1];
  __shared__ int tcount;
  if constexpr (Sparse)   // (block masks: hp = 1, the mask's 128-row blocks)
    n_tiles = build_tile_list(mask_row(p, w.b, w.h, w.hkv, w.qblk), t0, n_tiles, BN, tlist,
                              &tcount, wave, lane);
  // first key of the t-th tile visited
  auto tile_kt = [&](int t) {
    if constexpr (Sparse)
      return t0 + BN * __builtin_amdgcn_readfirstlane((int)tlist[t]);
    else
      return t0 + t * BN;
  };

  // DMA: LDS chunk P = 64 (wave NIW + k) + lane of a tile holds logical chunk
  // (P % CPR) ^ swz(row) of row P / CPR.
  const int P0 = 64 * wave * T::NIW + lane;
  const int voff_k = Strided ? (P0 / T::CPR) * krb + T::chunk_off(P0, false) : T::dma_off(P0, false);
  const int voff_v = Strided ? (P0 / T::CPR) * vrb + T::chunk_off(P0, true) : T::dma_off(P0, true);
  // Padded rows: each copy instruction's lane offset in full (a row stride
  // need not be a multiple of the tile row), or one past the buffer's range
  // for a chunk at or beyond dim DV, which then lands in LDS as zeros.
  // (a copy's range is capped below kOutOfRange, so such a chunk is entirely
  // out of range however long the key axis)
  constexpr int kOutOfRange = 0x7ffffff0;
  constexpr long long kMaxRange = 0x7fff0000LL;
  int pk_off[Pad ? T::NIW : 1], pv_off[Pad ? T::NIW : 1];
  if constexpr (Pad) {
#pragma unroll
    for (int k = 0; k < T::NIW; ++k) {
      const int P = P0 + 64 * k, row = P / T::CPR;
      const int ck = (P % T::CPR) ^ T::swz_k(row), cv = (P % T::CPR) ^ T::swz_v(row);
      pk_off[k] = 8 * ck < DV ? row * krb + 16 * ck : kOutOfRange;
      pv_off[k] = 8 * cv < DV ? row * vrb + 16 * cv : kOutOfRange;
    }
  }
  auto issue = [&](int kt, char* kdst, char* vdst, bool full = false) {
    if constexpr (Pad) {
      // valid bytes from the tile's first row: up to the end of row Sk - 1
      constexpr int rb = 2 * DV;
      const unsigned kbytes = full ? (unsigned)((BN - 1) * krb + rb)
                                   : (unsigned)min((long long)(p.Sk - kt - 1) * krb + rb, kMaxRange);
      const unsigned vbytes = full ? (unsigned)((BN - 1) * vrb + rb)
                                   : (unsigned)min((long long)(p.Sk - kt - 1) * vrb + rb, kMaxRange);
      const E* kb = Kp + (long long)kt * p.ks[2];
      const E* vb = Vp + (long long)kt * p.vs[2];
#pragma unroll
      for (int k = 0; k < T::NIW; ++k) {
        const int off = (wave * T::NIW + k) * 1024;
        dma16(kb, kbytes, pk_off[k], kdst + off);
        dma16(vb, vbytes, pv_off[k], vdst + off);
      }
    } else if constexpr (Strided) {
      // valid bytes from the tile's first row: up to the end of row Sk - 1
      const unsigned kbytes = full ? (unsigned)((BN - 1) * krb + T::ROW)
                                   : (unsigned)min((long long)(p.Sk - kt - 1) * krb + T::ROW, kMaxRange);
      const unsigned vbytes = full ? (unsigned)((BN - 1) * vrb + T::ROW)
                                   : (unsigned)min((long long)(p.Sk - kt - 1) * vrb + T::ROW, kMaxRange);
      const E* kb = Kp + (long long)kt * p.ks[2];
      const E* vb = Vp + (long long)kt * p.vs[2];
#pragma unroll
      for (int k = 0; k < T::NIW; ++k) {
        const int off = (wave * T::NIW + k) * 1024;
        dma16(kb, kbytes, (voff_k ^ T::chunk_xor(k, false)) + k * T::RPI * krb, kdst + off);
        dma16(vb, vbytes, (voff_v ^ T::chunk_xor(k, true)) + k * T::RPI * vrb, vdst + off);
      }
    } else {
      // a full tile needs no bound: BN rows are in range
      const unsigned bytes = full ? (unsigned)(BN * T::ROW) : (unsigned)min((long)(p.Sk - kt) * T::ROW, 0x7fffffffL);
      const E* kb = Kp + (size_t)kt * D;
      const E* vb = Vp + (size_t)kt * D;
#pragma unroll
      for (int k = 0; k < T::NIW; ++k) {
        const int off = (wave * T::NIW + k) * 1024;
        dma16(kb, bytes, voff_k ^ T::dma_xor(k, false), kdst + off);
        dma16(vb, bytes, voff_v ^ T::dma_xor(k, true), vdst + off);
      }
    }
  };

  // The first K/V copy goes out before the query rows are loaded, so the two
  // latencies overlap.
  if (n_tiles > 0) issue(tile_kt(0), kbuf0, vbuf0);

  // Query rows as the B operand: k-slot (g, e) of step t is dim 16t + 8g + e.
  e16x8 qf[DC];
#pragma unroll
  for (int t = 0; t < DC; ++t) {
    if (i < p.Sq)
      qf[t] = *(const e16x8*)(Qp + (long long)i * qr + 16 * t + 8 * g);
    else
      qf[t] = e16x8{};
    if (p.neg_q) {   // negative scale: use -Q and |scale| (exact sign flips)
      u32x4 bits = __builtin_bit_cast(u32x4, qf[t]) ^ 0x80008000u;
      qf[t] = __builtin_bit_cast(e16x8, bits);
    }
  }

  // Per-lane LDS read offsets (tile-relative). The swizzles only touch the low
  // four chunk-index bits, so chunks 16..31 of a row (D = 256) sit a fixed 256
  // bytes from chunks 0..15, and within those the offsets of K step t and of V
  // block db are the step-0 / block-0 offsets XOR 32 t and XOR 64 db in every
  // lane. D <= 128 keeps them in registers; D = 256, short of registers at two
  // wavefronts per SIMD, forms them with one XOR each.
  const int krow = perm_row(l32);
  constexpr int KO = DC < 8 ? DC : 8;
  constexpr int KR = D == 256 ? 1 : KO;
  int koff[KR];
#pragma unroll
  for (int t = 0; t < KR; ++t) koff[t] = krow * T::ROW + (((2 * t + g) ^ T::swz_k(krow)) << 4);
  auto k_off = [&](int t) { return (KR == 1 ? koff[0] ^ (32 * (t % KO)) : koff[t % KO]) + (t / KO) * 256; };
  const int blk = lane >> 4, li = lane & 15;
  const int vrow = 8 * g + (li >> 2);                       // + 16 C + 4 h
  constexpr int VO = DB < 4 ? DB : 4;
  constexpr int VR = D == 256 ? 1 : VO;
  int voff[VR];
#pragma unroll
  for (int db = 0; db < VR; ++db) {
    const int chunk = 4 * db + 2 * (blk & 1) + ((li & 3) >> 1);
    voff[db] = vrow * T::ROW + ((chunk ^ T::swz_v(vrow)) << 4) + 8 * (li & 1);
  }
  auto v_off = [&](int db) { return (VR == 1 ? voff[0] ^ (64 * (db % VO)) : voff[db % VO]) + (db / VO) * 256; };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_ref = -INFINITY, l = 0.f;
  const float sl = p.sl;
  f32x16 s[T::KB];
  e16x8 pf[T::KC];

  // ---- S^T = K Q^T for one tile
  auto qk = [&](const char* Ks) {
    // keep the XOR-derived offsets inside the loop (not hoisted into registers)
    if constexpr (KR == 1) asm volatile("" : "+v"(koff[0]));
#pragma unroll
    for (int kb = 0; kb < T::KB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int t = 0; t < DC; ++t) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb) {
        const e16x8 a = *(const e16x8*)(Ks + k_off(t) + kb * 32 * T::ROW);
        s[kb] = X::mfma(a, qf[t], s[kb]);
      }
    }
  };

  // ---- mask the keys of an edge tile this row cannot see
  auto mask = [&](int kt) {
    const bool edge = (kt + BN > p.Sk) || (p.causal && kt + BN - 1 > qw) ||
                      (p.window > 0 && kt < qw + 31 - p.window + 1);
    if (edge) {
      // Element v of block kb holds key kt + 8g + c with c = 32kb + 16(v/8) + v%8,
      // a compile-time constant: compare it with this row's visible range.
      const int base = kt + 8 * g;
      const int hi_c = (p.causal ? min(i, p.Sk - 1) : p.Sk - 1) - base;   // c <= hi_c
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (32 * kb + 16 * (v >> 3) + (v & 7) > hi_c) s[kb][v] = -INFINITY;
      if (p.window > 0) {
        const int lo_c = i - p.window + 1 - base;                           // c >= lo_c
#pragma unroll
        for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            if (32 * kb + 16 * (v >> 3) + (v & 7) < lo_c) s[kb][v] = -INFINITY;
      }
    }
  };

  // ---- P = exp2(S - m_sub) packed to the input type; returns this lane's
  // row sum of P. D <= 128 sums the fp32 values with VALU adds (the dot2
  // instructions issue to the matrix pipe, where they wait behind the other
  // wavefronts' MFMAs); D = 256, at two wavefronts per SIMD and short of
  // registers, sums the rounded 16-bit values with dot2.
  auto exp_pack_sum = [&](float m_sub) {
    if constexpr (D == 256) {
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pf[2 * kb + c2][e] = (E)fast_exp2(fmaf(s[kb][8 * c2 + e], sl, -m_sub));
      const typename X::x2 ones = {(E)1.f, (E)1.f};
      float rs = 0.f;
#pragma unroll
      for (int c = 0; c < T::KC; ++c)
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const typename X::x2 two = {pf[c][e], pf[c][e + 1]};
          rs = X::dot2(two, ones, rs);
        }
      return rs;
    } else {
      f32x4 ps;   // four partial sums (the first chunk initialises them: adding to
                  // a zero vector would cost four adds, as 0 + x is not x for x = -0)
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          f32x4 lo, hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo[e] = fast_exp2(fmaf(s[kb][8 * c2 + e], sl, -m_sub));
            hi[e] = fast_exp2(fmaf(s[kb][8 * c2 + 4 + e], sl, -m_sub));
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pf[2 * kb + c2][e] = (E)lo[e];
            pf[2 * kb + c2][4 + e] = (E)hi[e];
          }
          if (kb == 0 && c2 == 0) {
            ps = lo + hi;
          } else {
            ps += lo;
            ps += hi;
          }
        }
      return (ps[0] + ps[1]) + (ps[2] + ps[3]);
    }
  };

  // ---- softmax of one tile against the running reference max m_ref. The
  // exact tile max is only needed when the reference is too stale (or still
  // -inf): then some lane's row sum exceeds 2^64 (or is +inf), and the wave
  // takes the slow path: true row max, rescale O and l, recompute P. Exact in
  // every case, since O and l always share one reference; between rescales
  // every P stays below 2^64, far inside the float32 and bfloat16 range.
  float m_sub = -1e30f;   // m_ref, or -1e30 while m_ref is -inf
  auto softmax = [&]() {
    float rs = exp_pack_sum(m_sub);
    if (__any(!(rs <= X::kRowSumLimit))) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < T::KB; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
      mx = half_max(mx);
      const float mt = mx * sl;   // tile max in base-2 units (sl > 0)
      const float m_new = fmaxf(m_ref, mt);
      const float corr = fast_exp2(m_ref - (m_new == -INFINITY ? 0.f : m_new));
      m_ref = m_new;
      l *= corr;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= corr;
      rs = exp_pack_sum(m_ref == -INFINITY ? 0.f : m_ref);
      m_sub = m_ref == -INFINITY ? -1e30f : m_ref;
    }
    l += rs;
  };

  // ---- O^T += V^T P^T
  auto pv = [&](const char* Vs) {
    if constexpr (VR == 1) asm volatile("" : "+v"(voff[0]));
#pragma unroll
    for (int c = 0; c < T::KC; ++c) {
      if constexpr (D <= 128) {
        // all V operands of this 16-key chunk first, then its MFMAs
        e16x8 a[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int vo = v_off(db) + 16 * c * T::ROW;
          a[db] = read_v_pair<e16x8>(Vs, vo, vo + 4 * T::ROW);
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = X::mfma(a[db], pf[c], o[db]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, DB, 0);
      } else {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int base = 16 * c * T::ROW;
          const int vo = v_off(db) + base;
          const e16x8 a = read_v_pair<e16x8>(Vs, vo, vo + 4 * T::ROW);
          o[db] = X::mfma(a, pf[c], o[db]);
        }
      }
    }
  };

  auto wave_skips = [&](int kt) {
    return qw >= p.Sq || (p.causal && kt > qw + 31) ||
           (p.window > 0 && kt + BN - 1 < qw - p.window + 1);
  };

  // One tile: K(t), V(t) in (Kc, Vc); the copy of tile t+1 goes to (Kn, Vn).
  auto step = [&](int t, const char* Kc, const char* Vc, char* Kn, char* Vn) __attribute__((always_inline)) {
    const int kt = tile_kt(t);
    wait_dma_and_sync();
    if (t + 1 < n_tiles) issue(tile_kt(t + 1), Kn, Vn);
    if (wave_skips(kt)) return;
    qk(Kc);
    mask(kt);
    softmax();
    pv(Vc);
  };

  // Interior tiles: every row of the block sees every key of the tile and the
  // next tile exists with BN keys below Sk, so the step needs no skip, mask or
  // bounds decisions.
  auto step_in = [&](int t, const char* Kc, const char* Vc, char* Kn, char* Vn) __attribute__((always_inline)) {
    wait_dma_and_sync();
    issue(tile_kt(t + 1), Kn, Vn, true);
    qk(Kc);
    softmax();
    pv(Vc);
  };
  // Visited tiles [0, full_hi) hold BN keys below Sk; tiles [u_lo, u_hi) are
  // also fully visible to every row of the block. (Block masks: the visited
  // tiles are ascending, so only the last can be partial; without a causal
  // or window mask every visited tile is fully visible.)
  int full_hi = min(n_tiles, (p.Sk - t0) / BN);
  if constexpr (Sparse)
    full_hi = (n_tiles > 0 && tile_kt(n_tiles - 1) + BN > p.Sk) ? n_tiles - 1 : n_tiles;
  int u_lo = 0, u_hi = 0;
  if (q0 + bm <= p.Sq) {
    if constexpr (Sparse) {
      if (!p.causal && p.window <= 0) u_hi = full_hi;
    } else {
      u_hi = full_hi;
      if (p.causal) u_hi = min(u_hi, max(0, (q0 - t0 + 1) / BN));
      if (p.window > 0) {
        const int need = q0 + bm - p.window - t0;       // kt - t0 >= need
        u_lo = need > 0 ? (need + BN - 1) / BN : 0;
      }
    }
  }
  // steps t and t+1 both interior, and the tiles they copy (t+1, t+2) full
  auto in2 = [&](int t) __attribute__((always_inline)) {
    return t >= u_lo && t + 1 < u_hi && t + 2 < full_hi;
  };
  auto gen2 = [&](int t) __attribute__((always_inline)) {   // generic steps t, t+1; true when the loop is over
    step(t, kbuf0, vbuf0, kbuf1, vbuf1);
    if (t + 1 >= n_tiles) return true;
    step(t + 1, kbuf1, vbuf1, kbuf0, vbuf0);
    return t + 2 >= n_tiles;
  };

  int t = 0;
  bool done = n_tiles == 0;
  for (; !done && !in2(t); t += 2) done = gen2(t);
  for (; !done && in2(t); t += 2) {
    step_in(t, kbuf0, vbuf0, kbuf1, vbuf1);
    step_in(t + 1, kbuf1, vbuf1, kbuf0, vbuf0);
  }
  for (; !done; t += 2) done = gen2(t);

  // ---- epilogue: lane holds dims 32 db + 8 a + 4 g + (0..3) of row i.
  finish_row(p, w.b, h, w.split, i, g, m_ref, l,
             [&](bool partial, size_t row, int split, float inv) {
               if (partial) {
                 const size_t rows = (size_t)p.B * p.H * p.Sq;
                 float* dst = p.Opart + ((size_t)split * rows + row) * D;
#pragma unroll
                 for (int db = 0; db < DB; ++db)
#pragma unroll
                   for (int a = 0; a < 4; ++a) {
                     if (32 * db + 8 * a >= DV) continue;   // (DV: a multiple of 16)
                     f32x4 v4 = {o[db][4 * a] * inv, o[db][4 * a + 1] * inv,
                                 o[db][4 * a + 2] * inv, o[db][4 * a + 3] * inv};
                     *(f32x4*)(dst + 32 * db + 8 * a + 4 * g) = v4;
                   }
               } else {
                 E* dst = Strided ? (E*)p.O + w.b * p.os[0] + h * p.os[1] + (long long)i * p.os[2]
                                  : (E*)p.O + row * D;
#pragma unroll
                 for (int db = 0; db < DB; ++db)
#pragma unroll
                   for (int a = 0; a < 4; ++a) {
                     if (32 * db + 8 * a >= DV) continue;
                     typename X::x4 v4 = {(E)(o[db][4 * a] * inv), (E)(o[db][4 * a + 1] * inv),
                                          (E)(o[db][4 * a + 2] * inv), (E)(o[db][4 * a + 3] * inv)};
                     *(typename X::x4*)(dst + 32 * db + 8 * a + 4 * g) = v4;
                   }
               }
             });
}

// ====================================================================== fp32
// S^T tile = K Q^T with v_mfma_f32_32x32x2_f32 (true fp32 products). Step t
// pairs k-slot g with dim t + (D/2) g, so a lane reads four consecutive steps
// of its K row with one 16-byte LDS load. The PV MFMA step u takes, in lane
// half g, the key 8(u/4) + 4g + u%4 that the S accumulator element u holds,
// and O^T row m of d-block db is dim (D/32) m + db, so one 16-byte LDS load of
// a V row feeds four d-blocks and the epilogue stores 16-byte runs.
template <int D>
struct F32Tile {
  static constexpr int BN = 32;
  static constexpr int DH = D / 2;        // k-steps of the S MFMA
  static constexpr int DB = D / 32;       // d-blocks of the O^T accumulator
  static constexpr int LD = D + 4;        // LDS row stride (floats): conflict-free K reads
  static constexpr int TILE_F = BN * LD;  // floats per K or V tile
  static constexpr int STAGE_F = 2 * TILE_F;
  static constexpr int C4 = D / 4;        // float4 chunks per row
  static constexpr int IT = BN * C4 / kThreads;
  static_assert(BN * C4 % kThreads == 0, "tile must split evenly over the workgroup");
};

// Forms as for the 16-bit kernel; kFormPadded loads zeros for Q, K and V
// dims from p.dv on and stores O's first p.dv dims.
template <int D, int Form>
__global__ __launch_bounds__(kThreads, (D <= 128 ? 2 : 1))
void fwd_f32_kernel(Params p) {
  constexpr bool Pad = Form == kFormPadded;
  constexpr bool Strided = Form == kFormStrided || Pad, Sparse = Form == kFormBlockSparse;
  using T = F32Tile<D>;
  constexpr int BN = T::BN;
  __shared__ __attribute__((aligned(16))) float smem[2 * T::STAGE_F];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  // One item per workgroup, or (persistent launch) this slot's item list.
  const int k_end = p.sched ? p.sched[blockIdx.x + 1] : 1;
  for (int kk = p.sched ? p.sched[blockIdx.x] : 0; kk < k_end; ++kk) {
  const Tile w = p.sched ? item_tile(p, p.sched[p.nslot + 1 + kk]) : map_tile(p);
  const int q0 = w.qblk * kBlockM;
  const int qw = q0 + wave * 32;
  const int i = qw + l32;

  const float* Qp;
  const float* Kp;
  const float* Vp;
  long long qr = D, kr = D, vr = D;   // element row strides
  if constexpr (Strided) {
    Qp = (const float*)p.Q + w.b * p.qs[0] + w.h * p.qs[1];
    Kp = (const float*)p.K + w.b * p.ks[0] + w.hkv * p.ks[1];
    Vp = (const float*)p.V + w.b * p.vs[0] + w.hkv * p.vs[1];
    qr = p.qs[2];
    kr = p.ks[2];
    vr = p.vs[2];
  } else {
    Qp = (const float*)p.Q + (size_t)(w.b * p.H + w.h) * p.Sq * D;
    Kp = (const float*)p.K + (size_t)(w.b * p.HKV + w.hkv) * p.Sk * D;
    Vp = (const float*)p.V + (size_t)(w.b * p.HKV + w.hkv) * p.Sk * D;
  }

  int lo, hi;
  key_range(p, q0, kBlockM, w.split, lo, hi);
  const int t0 = (lo / BN) * BN;
  int n_tiles = hi > lo ? (hi - t0 + BN - 1) / BN : 0;
  __shared__ unsigned short tlist[Sparse ? kMaxListTiles : 1];
  __shared__ int tcount;
  if constexpr (Sparse)
    n_tiles = build_tile_list(mask_row(p, w.b, w.h, w.hkv, w.qblk), t0, n_tiles, BN, tlist,
                              &tcount, wave, lane);
  auto tile_kt = [&](int t) {
    if constexpr (Sparse)
      return t0 + BN * __builtin_amdgcn_readfirstlane((int)tlist[t]);
    else
      return t0 + t * BN;
  };

  float qf[T::DH];
#pragma unroll
  for (int t4 = 0; t4 < T::DH / 4; ++t4) {
    const bool ok = i < p.Sq && (!Pad || T::DH * g + 4 * t4 < p.dv);
    f32x4 v = ok ? *(const f32x4*)(Qp + (long long)i * qr + T::DH * g + 4 * t4) : f32x4{};
    qf[4 * t4 + 0] = v[0];
    qf[4 * t4 + 1] = v[1];
    qf[4 * t4 + 2] = v[2];
    qf[4 * t4 + 3] = v[3];
  }

  f32x16 o[T::DB];
#pragma unroll
  for (int db = 0; db < T::DB; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  f32x4 kreg[T::IT], vreg[T::IT];
  auto load_tile = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < T::IT; ++it) {
      const int c = tid + it * kThreads;
      const int row = c / T::C4, c4 = c % T::C4;
      const int key = kt + row;
      const bool ok = key < p.Sk && (!Pad || 4 * c4 < p.dv);
      kreg[it] = ok ? *(const f32x4*)(Kp + (long long)key * kr + 4 * c4) : f32x4{};
      vreg[it] = ok ? *(const f32x4*)(Vp + (long long)key * vr + 4 * c4) : f32x4{};
    }
  };
  auto store_tile = [&](float* st) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < T::IT; ++it) {
      const int c = tid + it * kThreads;
      const int row = c / T::C4, c4 = c % T::C4;
      *(f32x4*)(st + row * T::LD + 4 * c4) = kreg[it];
      *(f32x4*)(st + T::TILE_F + row * T::LD + 4 * c4) = vreg[it];
    }
  };

  if (n_tiles > 0) {
    load_tile(tile_kt(0));
    store_tile(smem);
  }
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int kt = tile_kt(it);
    const float* Ks = smem + (it & 1) * T::STAGE_F;
    const float* Vs = Ks + T::TILE_F;
    if (it + 1 < n_tiles) load_tile(tile_kt(it + 1));

    const bool skip = qw >= p.Sq || (p.causal && kt > qw + 31) ||
                      (p.window > 0 && kt + BN - 1 < qw - p.window + 1);
    if (!skip) {
      f32x16 s = f32x16{};
      const float* krow = Ks + l32 * T::LD + T::DH * g;
#pragma unroll
      for (int t4 = 0; t4 < T::DH / 4; ++t4) {
        const f32x4 a = *(const f32x4*)(krow + 4 * t4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[4 * t4 + e], s, 0, 0, 0);
      }
      const bool edge = (kt + BN > p.Sk) || (p.causal && kt + BN - 1 > qw) ||
                        (p.window > 0 && kt < qw + 31 - p.window + 1);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = s[v] * p.sl;
        if (edge) {
          const int j = kt + 8 * (v >> 2) + 4 * g + (v & 3);
          x = visible(p, i, j) ? x : -INFINITY;
        }
        s[v] = x;
      }
      // P against the running reference max m (base-2 units); the exact tile
      // max is needed only when some lane's row sum exceeds 2^64 (which
      // includes the first tile, m = -inf): then O and l are rescaled and P
      // recomputed. O and l always share the reference: the same softmax.
      f32x16 e;
      auto exps = [&](float m_sub) __attribute__((always_inline)) {
        float part[4];   // the first four exponentials initialise the partial sums
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          e[v] = fast_exp2(s[v] - m_sub);
          part[v & 3] = v < 4 ? e[v] : part[v & 3] + e[v];
        }
        return (part[0] + part[1]) + (part[2] + part[3]);
      };
      float rs = exps(m == -INFINITY ? -1e30f : m);
      if (__any(!(rs <= kRowSumLimit))) {
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx);
        const float corr = fast_exp2(m - (m_new == -INFINITY ? 0.f : m_new));
        m = m_new;
        l *= corr;
#pragma unroll
        for (int db = 0; db < T::DB; ++db) o[db] *= corr;
        rs = exps(m == -INFINITY ? 0.f : m);
      }
      l += rs;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int key = 8 * (u >> 2) + 4 * g + (u & 3);
        const float* vrow = Vs + key * T::LD + T::DB * l32;
        float va[T::DB];
        if constexpr (T::DB >= 4) {
#pragma unroll
          for (int c4 = 0; c4 < T::DB / 4; ++c4) {
            const f32x4 x = *(const f32x4*)(vrow + 4 * c4);
            va[4 * c4 + 0] = x[0];
            va[4 * c4 + 1] = x[1];
            va[4 * c4 + 2] = x[2];
            va[4 * c4 + 3] = x[3];
          }
        } else {
#pragma unroll
          for (int e = 0; e < T::DB; ++e) va[e] = vrow[e];
        }
#pragma unroll
        for (int db = 0; db < T::DB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(va[db], e[u], o[db], 0, 0, 0);
      }
    }

    if (it + 1 < n_tiles) store_tile(smem + ((it + 1) & 1) * T::STAGE_F);
    __syncthreads();
  }

  // ---- epilogue: element v of block db is dim (D/32)(8(v/4) + 4g + v%4) + db.
  finish_row(p, w.b, w.h, w.split, i, g, m, l,
             [&](bool partial, size_t row, int split, float inv) __attribute__((always_inline)) {
               float* dst;
               if (partial) {
                 const size_t rows = (size_t)p.B * p.H * p.Sq;
                 dst = p.Opart + ((size_t)split * rows + row) * D;
               } else if constexpr (Strided) {
                 dst = (float*)p.O + w.b * p.os[0] + w.h * p.os[1] + (long long)i * p.os[2];
               } else {
                 dst = (float*)p.O + row * D;
               }
#pragma unroll
               for (int v = 0; v < 16; ++v) {
                 const int mrow = 8 * (v >> 2) + 4 * g + (v & 3);
                 float* d0 = dst + T::DB * mrow;
                 if (T::DB % 4 == 0) {
#pragma unroll
                   for (int c4 = 0; c4 < T::DB / 4; ++c4) {
                     if (Pad && T::DB * mrow + 4 * c4 >= p.dv) continue;
                     f32x4 x = {o[4 * c4][v] * inv, o[4 * c4 + 1][v] * inv,
                                o[4 * c4 + 2][v] * inv, o[4 * c4 + 3][v] * inv};
                     *(f32x4*)(d0 + 4 * c4) = x;
                   }
                 } else {
#pragma unroll
                   for (int db = 0; db < T::DB; ++db)
                     if (!Pad || T::DB * mrow + db < p.dv) d0[db] = o[db][v] * inv;
                 }
               }
             });
  __syncthreads();   // LDS is reused by the next item
  }
}

// ============================================================ split merge
// O = sum_s exp(LSE_s - LSE) O_s and LSE = log sum_s exp(LSE_s): the block
// form of the online-softmax rescale. A split that saw no key has
// LSE_s = -inf and weight 0; a row with no key in any split gets O = 0 and
// LSE = -inf. Strided: O row (b, h, i) of the flat row index (b H + h) Sq + i
// sits at O + b os[0] + h os[1] + i os[2]. Partial rows hold D floats of
// which the first dv (a multiple of 4) are O's dims.
template <typename OutT, int D, bool Strided>
__global__ __launch_bounds__(kThreads)
void merge_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart,
                  OutT* __restrict__ O, float* __restrict__ LSE, long rows, int nsplit,
                  int H, int Sq, long long os0, long long os1, long long os2, int dv) {
  constexpr int TPR = D / 4;               // threads per row, 4 dims each
  constexpr int RPB = kThreads / TPR;
  if (threadIdx.x >= RPB * TPR) return;    // (D = 96: 16 threads left over)
  const long row = (long)blockIdx.x * RPB + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  if (row >= rows) return;
  const bool on = 4 * c < dv;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, Lpart[(size_t)s * rows + row]);
  f32x4 acc = f32x4{};
  float den = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < nsplit; ++s) {
      const float ls = Lpart[(size_t)s * rows + row];
      if (ls == -INFINITY) continue;   // no key in this split (its O part is not written)
      const float wgt = __expf(ls - M);
      den += wgt;
      if (on) acc += wgt * *(const f32x4*)(Opart + ((size_t)s * rows + row) * D + 4 * c);
    }
    acc *= 1.f / den;
  }
  OutT* dst;
  if constexpr (Strided) {
    const long bh = row / Sq;
    dst = O + (bh / H) * os0 + (bh % H) * os1 + (row % Sq) * os2 + 4 * c;
  } else {
    dst = O + (size_t)row * D + 4 * c;
  }
  if (!on) {
  } else if constexpr (sizeof(OutT) == 2) {
    typedef typename Elt<OutT>::x4 o4;
    *(o4*)dst = o4{(OutT)acc[0], (OutT)acc[1], (OutT)acc[2], (OutT)acc[3]};
  } else {
    *(f32x4*)dst = acc;
  }
  if (c == 0) LSE[row] = M == -INFINITY ? -INFINITY : M + __logf(den);
}

// ================================================================ launch
int key_tile(int dtype, int D) {
  if (dtype != 0) return D >= 128 ? 32 : 64;   // 16-bit inputs
  return F32Tile<64>::BN;
}

int block_m(int dtype, int D) { return kBlockM; }

template <int D>
static int f32_occupancy(int form) {
  int n = 0;
  hipError_t e = hipErrorInvalidValue;
  if (form == kFormContiguous)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_f32_kernel<D, kFormContiguous>, kThreads, 0);
  if (form == kFormStrided)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_f32_kernel<D, kFormStrided>, kThreads, 0);
  if (form == kFormBlockSparse)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_f32_kernel<D, kFormBlockSparse>, kThreads, 0);
  if constexpr (D <= 128)
    if (form == kFormPadded)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fwd_f32_kernel<D, kFormPadded>, kThreads, 0);
  return e == hipSuccess ? n : 0;
}

int f32_blocks_per_cu(int D, int form) {
  if (D == 32) return f32_occupancy<32>(form);
  if (D == 64) return f32_occupancy<64>(form);
  if (D == 96) return f32_occupancy<96>(form);
  if (D == 128) return f32_occupancy<128>(form);
  if (D == 256) return f32_occupancy<256>(form);
  return 0;
}

template <typename OutT, int D, bool Strided>
static hipError_t launch_merge(const Params& p, hipStream_t stream) {
  const long rows = (long)p.B * p.H * p.Sq;
  constexpr int RPB = kThreads / (D / 4);
  const long blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((merge_kernel<OutT, D, Strided>), dim3((unsigned)blocks), dim3(kThreads), 0,
                     stream, p.Opart, p.Lpart, (OutT*)p.O, p.LSE, rows, p.nsplit, p.H, p.Sq,
                     p.os[0], p.os[1], p.os[2], p.dv);
  return hipGetLastError();
}

template <typename E, int D, int BN, int Form, int DV = D>
static hipError_t launch_16b_e(const Params& p, long blocks, hipStream_t stream) {
  hipLaunchKernelGGL((fwd_16b_kernel<E, D, BN, Form, DV>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
  return hipSuccess;
}

// The 16-bit kernel at tile dim D; the padded form is instantiated per head dim.
template <int D, int BN, int Form>
static hipError_t launch_16b(const Params& p, bool bf16, long blocks, hipStream_t stream) {
  if constexpr (Form == kFormPadded) {
    switch (p.dv) {
#define FA_PADDED_DV(X)                                                                   \
      case X:                                                                             \
        if constexpr (tile_dim(X, 1) == D)                                                \
          return bf16 ? launch_16b_e<__bf16, D, BN, Form, X>(p, blocks, stream)            \
                      : launch_16b_e<_Float16, D, BN, Form, X>(p, blocks, stream);        \
        return hipErrorInvalidValue;
      FA_PADDED_DV(16)
      FA_PADDED_DV(32)
      FA_PADDED_DV(48)
      FA_PADDED_DV(80)
      FA_PADDED_DV(96)
#undef FA_PADDED_DV
      default: return hipErrorInvalidValue;
    }
  } else {
    return bf16 ? launch_16b_e<__bf16, D, BN, Form>(p, blocks, stream)
                : launch_16b_e<_Float16, D, BN, Form>(p, blocks, stream);
  }
}

template <int D, int Form>
static hipError_t launch_d(const Params& p, int dtype, hipStream_t stream) {
  constexpr bool Strided = Form == kFormStrided || Form == kFormPadded;
  const long blocks = (long)p.units * p.n_qblk;
  constexpr int BN = D >= 128 ? 32 : 64;
  // (the 16-bit kernel has no persistent form; sched is ignored)
  if (dtype == 1 || dtype == 2) {
    if constexpr (D == 32 || D == 96) return hipErrorInvalidValue;   // fp32-only tile dims
    else {
      const hipError_t e = launch_16b<D, BN, Form>(p, dtype == 1, blocks, stream);
      if (e != hipSuccess) return e;
    }
  } else {
    const long grid = p.sched ? (long)p.nslot : blocks;
    hipLaunchKernelGGL((fwd_f32_kernel<D, Form>), dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  if constexpr (D != 32 && D != 96) {
    if (dtype == 1) return launch_merge<__bf16, D, Strided>(p, stream);
    if (dtype == 2) return launch_merge<_Float16, D, Strided>(p, stream);
  }
  return launch_merge<float, D, Strided>(p, stream);
}

template <int D>
static hipError_t launch_form(const Params& p, int dtype, int form, hipStream_t stream) {
  if (form == kFormStrided) return launch_d<D, kFormStrided>(p, dtype, stream);
  if (form == kFormBlockSparse) return launch_d<D, kFormBlockSparse>(p, dtype, stream);
  if (form == kFormPadded) {
    if constexpr (D <= 128) return launch_d<D, kFormPadded>(p, dtype, stream);
    return hipErrorInvalidValue;   // padded head dims run on the 64 and 128 tiles
  }
  return launch_d<D, kFormContiguous>(p, dtype, stream);
}

hipError_t launch_forward(const Params& p, int dtype, int D, int form, hipStream_t stream) {
  switch (D) {
    case 32: return launch_form<32>(p, dtype, form, stream);
    case 64: return launch_form<64>(p, dtype, form, stream);
    case 96: return launch_form<96>(p, dtype, form, stream);
    case 128: return launch_form<128>(p, dtype, form, stream);
    case 256: return launch_form<256>(p, dtype, form, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fa

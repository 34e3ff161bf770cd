// C ABI of the backward pass: argument checks, the D_i workspace, the staged
// copies (padded head dims, strided tensors) and the launch. Declared in
// include/fa.h (fa_bwd, fa_bwd_strided, fa_bwd_block_sparse).
#include "fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "fa_bwd.h"

namespace {

// Visible (query row, key) pairs of one head, counted up to `cap`: rows i <
// Sq see keys j < Sk with j <= i under a causal mask and j > i - window under
// a window.
double visible_pairs(int Sq, int Sk, int causal, int window, double cap) {
  double n = 0;
  for (long i = 0; i < Sq && n < cap; ++i) {
    const long hi = causal ? std::min<long>(i + 1, Sk) : Sk;
    const long lo = window > 0 ? std::max<long>(0, i - window + 1) : 0;
    if (hi > lo) n += (double)(hi - lo);
  }
  return n;
}

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

// Element strides (batch, head, row) of one view: the caller's, or those of a
// contiguous [B, heads, S, D] tensor when `given` is NULL.
void view_strides(const long long* given, int heads, int S, int D, long long out[3]) {
  if (given) {
    out[0] = given[0];
    out[1] = given[1];
    out[2] = given[2];
  } else {
    out[2] = D;
    out[1] = (long long)S * D;
    out[0] = (long long)heads * S * D;
  }
}

// Stride rules of the backward's views: non-negative, every row start 16-byte
// aligned, rows of D elements not overlapping along the row axis, and every
// element offset far inside int64 (the gradients must also have disjoint
// rows, checked by the caller).
int check_view(const long long st[3], int B, int heads, int S, int D, int esz) {
  for (int a = 0; a < 3; ++a)
    if (st[a] < 0 || (st[a] * esz) % 16 != 0) return FA_ERR_STRIDE;
  if (st[2] < D) return FA_ERR_STRIDE;
  const double last = (double)(B - 1) * st[0] + (double)(heads - 1) * st[1] +
                      (double)(S - 1) * st[2] + D;
  if (last * esz > 4.0e18) return FA_ERR_SHAPE;
  return FA_OK;
}

// Block mask of fa_bwd_block_sparse (NULL for the other entry points).
struct BwdMask {
  const unsigned char* mask;
  int batch, heads;
};

// The backward's plan for one call (host computation only): the tile dim
// the kernels run at, how the inputs reach them, and the small-grid chunks.
struct BwdPlan {
  int DT = 0;
  bool gen = false, padded = false, staged = false, per_row = false;
  int nch = 1, chunk_q = 0, chunk_k = 0;   // key chunks (dQ; the per-row kernels: both)
  int nrc = 1, chunk_r = 0;                // row chunks of the MFMA dK/dV kernels
};

// contiguous: every tensor in its contiguous [B, heads, S, D] layout;
// max_row_stride: the largest row stride (elements) of Q, K, V, O, dO;
// cus: compute units of the device.
BwdPlan plan_backward(int B, int H, int HKV, int Sq, int Sk, int D, int causal, int window,
                      int dtype, bool contiguous, long long max_row_stride, int cus) {
  BwdPlan pl;
  const long n_qblk = (Sq + 127) / 128;
  // fp32 at D = 256: MFMA kernels with 64 query rows (keys) per workgroup
  const bool f32_256 = dtype == FA_F32 && D == 256;
  const size_t nq = (size_t)B * H * Sq, nk = (size_t)B * HKV * Sk;
  // 16-bit inputs at head dims 16 .. 96 other than 64 run the MFMA kernels of
  // the 64 or 128 tile with the dims from D on held as zeros (they add exact
  // zeros to every dot product, and the gradients' extra dims are not
  // written). The 16-bit MFMA kernels read such head dims, and strided views,
  // directly (their general form: per-view strides, copy offsets formed in
  // full, chunks at or beyond D read as zeros), as long as every row stride
  // keeps a tile's copy offsets far inside 32 bits. Otherwise, and for fp32
  // views, the inputs are staged: copied to contiguous zero-padded rows, and
  // the gradients copied back into the caller's views.
  const int DT16 = D <= 64 ? 64 : D <= 128 ? 128 : 256;
  bool gen = false;
  if (dtype != FA_F32 && (!contiguous || D != DT16))
    gen = max_row_stride <= (1LL << 22);   // 64 rows x 2 bytes x 2^22 = 2^29 bytes per tile
  // fp32 head dims below an fp32 MFMA tile (16, 48, 80) are staged into it
  // when the work is large enough to pay for the staging copies (B H visible
  // pairs at least 2^23; smaller problems run faster on the per-row kernels,
  // whose launch has no copies around it); D = 256 keeps the per-row kernels
  const int DTF = D <= 32 ? 32 : D <= 64 ? 64 : D <= 96 ? 96 : D <= 128 ? 128 : D;
  const double pad_work = 8388608.0;
  const bool f32_pad = dtype == FA_F32 && D != DTF &&
                       (double)B * H * visible_pairs(Sq, Sk, causal, window, pad_work / ((double)B * H)) >=
                           pad_work;
  const bool padded = dtype != FA_F32 ? D != DT16 : f32_pad;
  const bool staged = !gen && (padded || !contiguous);
  const int DT = padded ? (dtype != FA_F32 ? DT16 : DTF) : D;
  // The per-row kernels (fp32 inputs at D = 16, 48, 80 unstaged) on grids too
  // small to fill the GPU: each row group's range is cut into nch chunks that run side by side
  // (a causal grid is otherwise bound by its longest rows), their partial
  // sums added up afterwards in chunk order (deterministic). A group's range
  // spans at most `span` + R - 1 keys (query rows): the ranges of its R
  // adjacent rows.
  const bool per_row = dtype == FA_F32 && !fa::bwd_f32_mfma(DT);
  if (per_row) {
    const int R = fa::bwd_rows_per_group(DT);
    const long groups = (long)B * H * ((Sq + R - 1) / R);
    const long target = 1L << 18;   // row groups that fill the GPU several times over
    // keys per query row and query rows per key: at most `window` only under
    // causal + window (a window alone bounds one side)
    const bool band = causal && window > 0;
    const long span_q = (band ? std::min(Sk, window) : Sk) + R - 1;
    const long span_k = (band ? std::min(Sq, window) : Sq) + R - 1;
    if (groups < target) {
      long n = std::min({(target + groups - 1) / groups, (std::max(span_q, span_k) + 127) / 128, 8L});
      const double per_chunk = (double)(nq + 2 * nk) * DT * 4;
      while (n > 1 && n * per_chunk > 512.0 * (1 << 20)) --n;   // workspace at most 512 MiB
      pl.nch = (int)std::max(1L, n);
    }
    pl.chunk_q = (int)((span_q + pl.nch - 1) / pl.nch);
    pl.chunk_k = (int)((span_k + pl.nch - 1) / pl.nch);
  } else {
    // MFMA kernels: when the dQ kernel has fewer query tiles than two per
    // CU, cut the key axis into chunks of whole 32-key tiles (at least 16
    // tiles each, at most 16 chunks, workspace at most 512 MiB)
    const long qwg = (long)B * H * (f32_256 ? (Sq + 63) / 64 : n_qblk);
    const long tiles = (Sk + 31) / 32;
    if (qwg < 2L * cus) {
      long n = std::min({(2L * cus + qwg - 1) / qwg, tiles / 16, 16L});
      while (n > 1 && (double)n * nq * DT * 4 > 512.0 * (1 << 20)) --n;
      if (n > 1) {
        pl.chunk_q = (int)((tiles + n - 1) / n) * 32;
        pl.nch = (int)((Sk + pl.chunk_q - 1) / pl.chunk_q);
      }
    }
  }
  // MFMA dK/dV kernels: when their workgroups (two per 128 keys at D = 256)
  // fill less than the GPU's slots (one per CU; two for fp32 at D <= 64; fp32
  // counts the slots twice) and a
  // workgroup's walk is long (Sq rows of each of its H / HKV query heads: at
  // least 2048, fp32 1024; shorter walks gain less than the partial sums
  // cost), cut the query rows into chunks of whole 128-row blocks (a causal
  // grid is otherwise as long as its first key blocks, which see every row):
  // as many as fill the (doubled) slots, at most 8, workspace at most 512 MiB.
  // The partial sums are contiguous rows; views (the general form) get the
  // summed dK and dV from contiguous rows too. A block mask's 128-row blocks
  // never straddle two chunks, so the same chunks serve it (and an all-ones
  // mask keeps the dense sums bit for bit).
  pl.chunk_r = Sq;
  if (!per_row) {
    const long wgs = (long)B * HKV * ((Sk + 127) / 128) * (DT == 256 ? 2 : 1);
    const bool f32 = dtype == FA_F32;
    const long target = (long)cus * (f32 && DT <= 64 ? 2 : 1) * (f32 ? 2 : 1);
    const long blocks = (Sq + 127) / 128;
    const long walk = (long)Sq * (H / HKV);
    if (wgs < target && walk >= (f32 ? 1024 : 2048)) {
      long n = std::min({(target + wgs - 1) / wgs, blocks, 8L});
      while (n > 1 && 2.0 * n * nk * DT * 4 > 512.0 * (1 << 20)) --n;
      if (n > 1) {
        pl.chunk_r = (int)((blocks + n - 1) / n) * 128;
        pl.nrc = (int)((Sq + pl.chunk_r - 1) / pl.chunk_r);
      }
    }
  }
  pl.DT = DT;
  pl.gen = gen;
  pl.padded = padded;
  pl.staged = staged;
  pl.per_row = per_row;
  return pl;
}

// The backward pass for views with the given element strides (NULL =
// contiguous): q, k, v, o, dO in the input type, then dQ, dK, dV (fp32).
int backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* LSE, float* dQ, float* dK, float* dV, int B, int H, int HKV, int Sq,
             int Sk, int D, const long long* const given[8], float scale, int causal,
             int window, int dtype, void* stream_ptr, const BwdMask* bm = nullptr) {
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV || (bm && !bm->mask))
    return FA_ERR_NULLPTR;
  int st = check_bwd(B, H, HKV, Sq, Sk, D, causal, window, dtype);
  if (st != FA_OK) return st;
  if (bm) {
    // block masks: contiguous tensors at the forward's block-mask head dims
    if ((bm->batch != 1 && bm->batch != B) ||
        (bm->heads != 1 && bm->heads != HKV && bm->heads != H))
      return FA_ERR_MASK;
    if (D != 64 && D != 128 && D != 256) return FA_ERR_HEAD_DIM;
    // the dK/dV kernels' list entries hold a query head of the group in 10 bits
    if (H / HKV >= 1024) return FA_ERR_SHAPE;
  }
  for (const void* p : {Q, K, V, O, dO, (const void*)LSE, (const void*)dQ, (const void*)dK,
                        (const void*)dV})
    if (!aligned16(p)) return FA_ERR_ALIGN;
  // views: 0 Q, 1 K, 2 V, 3 O, 4 dO (input type), 5 dQ, 6 dK, 7 dV (fp32)
  const int esz = dtype == FA_F32 ? 4 : 2;
  long long vs[8][3];
  bool contiguous = true;
  for (int t = 0; t < 8; ++t) {
    const bool kv = t == 1 || t == 2 || t == 6 || t == 7;
    const int heads = kv ? HKV : H, S = kv ? Sk : Sq;
    view_strides(given ? given[t] : nullptr, heads, S, D, vs[t]);
    if ((st = check_view(vs[t], B, heads, S, D, t < 5 ? esz : 4)) != FA_OK) return st;
    long long c[3];
    view_strides(nullptr, heads, S, D, c);
    contiguous = contiguous && std::equal(vs[t], vs[t] + 3, c);
  }
  if (!fa::output_rows_disjoint(vs[5], B, H, Sq, D) ||
      !fa::output_rows_disjoint(vs[6], B, HKV, Sk, D) ||
      !fa::output_rows_disjoint(vs[7], B, HKV, Sk, D))
    return FA_ERR_STRIDE;

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
  if (bm) {
    p.bmask = bm->mask;
    p.bm_nqb = (Sq + fa::kBwdMaskQ - 1) / fa::kBwdMaskQ;
    p.bm_nkb = (Sk + fa::kBwdMaskK - 1) / fa::kBwdMaskK;
    const long long slab = (long long)p.bm_nqb * p.bm_nkb;
    p.bm_sh = bm->heads == 1 ? 0 : slab;
    p.bm_sb = bm->batch == 1 ? 0 : bm->heads * slab;
    p.bm_by_q = bm->heads == H ? 1 : 0;
  }
  long long mx = 0;   // the largest row stride of the inputs
  for (int t = 0; t < 5; ++t) mx = std::max(mx, vs[t][2]);
  const int cus = fa::device_cus();
  if (cus <= 0) return FA_ERR_HIP;
  const BwdPlan pl = plan_backward(B, H, HKV, Sq, Sk, D, causal, window, dtype, contiguous, mx, cus);
  const bool gen = pl.gen, staged = pl.staged, per_row = pl.per_row;
  const int DT = pl.DT;
  p.nch = pl.nch;
  p.chunk_q = pl.chunk_q;
  p.chunk_k = pl.chunk_k;
  p.nrc = pl.nrc;
  p.chunk_r = pl.chunk_r;
  const size_t nq = (size_t)B * H * Sq, nk = (size_t)B * HKV * Sk;
  auto up = [](size_t bytes) { return (bytes + 255) / 256 * 256; };
  // workspace, stream-ordered from the library's memory pool: D_i, and when
  // padded Q, O, dO, K, V (input type) and dQ, dK, dV (fp32) at DT
  const size_t b_d = up(nq * sizeof(float));
  const size_t b_q = staged ? up(nq * DT * esz) : 0, b_k = staged ? up(nk * DT * esz) : 0;
  size_t b_gk = staged ? up(nk * DT * 4) : 0;   // (and the general form's row chunks)
  size_t b_gq = staged ? up(nq * DT * 4) : 0;   // (the general form's key chunks also use it)
  if (gen && p.nch > 1) b_gq = up(nq * DT * 4);   // summed dQ before it goes to the view
  if (gen && p.nrc > 1) b_gk = up(nk * DT * 4);   // summed dK, dV before they go to the views
  const size_t b_pq = p.nch > 1 ? up((size_t)p.nch * nq * DT * 4) : 0;
  const size_t b_pk = p.nch > 1 && per_row ? up((size_t)p.nch * nk * DT * 4)
                      : p.nrc > 1          ? up((size_t)p.nrc * nk * DT * 4)
                                           : 0;
  void* ws = nullptr;
  const int wst = fa::library_workspace(b_d + 3 * b_q + 2 * b_k + b_gq + 2 * b_gk + b_pq + 2 * b_pk,
                                        stream, &ws);
  if (wst != FA_OK) return wst;
  char* w = static_cast<char*>(ws);
  p.Dws = reinterpret_cast<float*>(w);
  if (p.nch > 1 || p.nrc > 1) {
    char* pp = w + b_d + 3 * b_q + 2 * b_k + b_gq + 2 * b_gk;
    p.part_q = p.nch > 1 ? reinterpret_cast<float*>(pp) : nullptr;
    p.part_k = b_pk ? reinterpret_cast<float*>(pp + b_pq) : nullptr;
    p.part_v = b_pk ? reinterpret_cast<float*>(pp + b_pq + b_pk) : nullptr;
  }
  hipError_t e = hipSuccess;
  if (staged) {
    char* q = w + b_d;
    char* o = q + b_q;
    char* go = o + b_q;
    char* k = go + b_q;
    char* v = k + b_k;
    float* gq = reinterpret_cast<float*>(v + b_k);
    float* gk = reinterpret_cast<float*>(reinterpret_cast<char*>(gq) + b_gq);
    float* gv = reinterpret_cast<float*>(reinterpret_cast<char*>(gk) + b_gk);
    long long bs[8][3];   // byte strides
    for (int t = 0; t < 8; ++t)
      for (int a = 0; a < 3; ++a) bs[t][a] = vs[t][a] * (t < 5 ? esz : 4);
    const struct { const void* src; void* dst; int heads, S, view; } stage[5] = {
        {Q, q, H, Sq, 0}, {O, o, H, Sq, 3}, {dO, go, H, Sq, 4}, {K, k, HKV, Sk, 1},
        {V, v, HKV, Sk, 2}};
    for (const auto& t : stage)
      if (e == hipSuccess)
        e = fa::launch_gather_rows(t.src, t.dst, B, t.heads, t.S, bs[t.view], esz * D, esz * DT,
                                   stream);
    p.Q = q;
    p.O = o;
    p.dO = go;
    p.K = k;
    p.V = v;
    p.dQ = gq;
    p.dK = gk;
    p.dV = gv;
    if (e == hipSuccess) e = fa::launch_backward(p, dtype, DT, stream);
    if (e == hipSuccess) e = fa::launch_scatter_rows(gq, dQ, B, H, Sq, bs[5], DT, D, stream);
    if (e == hipSuccess) e = fa::launch_scatter_rows(gk, dK, B, HKV, Sk, bs[6], DT, D, stream);
    if (e == hipSuccess) e = fa::launch_scatter_rows(gv, dV, B, HKV, Sk, bs[7], DT, D, stream);
  } else if (gen) {
    p.gen = 1;
    p.dv = D;
    std::copy(vs[0], vs[0] + 3, p.qs);
    std::copy(vs[1], vs[1] + 3, p.ks);
    std::copy(vs[2], vs[2] + 3, p.vs);
    std::copy(vs[3], vs[3] + 3, p.os);
    std::copy(vs[4], vs[4] + 3, p.dos);
    std::copy(vs[5], vs[5] + 3, p.dqs);
    std::copy(vs[6], vs[6] + 3, p.dks);
    std::copy(vs[7], vs[7] + 3, p.dvs);
    // with key chunks (dQ) or row chunks (dK, dV) the chunk sums land in
    // contiguous rows first
    char* g0 = w + b_d + 3 * b_q + 2 * b_k;
    float* gq = p.nch > 1 ? reinterpret_cast<float*>(g0) : nullptr;
    float* gk = p.nrc > 1 ? reinterpret_cast<float*>(g0 + b_gq) : nullptr;
    float* gv = p.nrc > 1 ? reinterpret_cast<float*>(g0 + b_gq + b_gk) : nullptr;
    if (gq) p.dQ = gq;
    if (gk) {
      p.dK = gk;
      p.dV = gv;
    }
    e = fa::launch_backward(p, dtype, DT, stream);
    long long bs[3][3];   // byte strides of the dQ, dK, dV views
    for (int t = 0; t < 3; ++t)
      for (int a = 0; a < 3; ++a) bs[t][a] = vs[5 + t][a] * 4;
    if (e == hipSuccess && gq) e = fa::launch_scatter_rows(gq, dQ, B, H, Sq, bs[0], DT, D, stream);
    if (e == hipSuccess && gk) e = fa::launch_scatter_rows(gk, dK, B, HKV, Sk, bs[1], DT, D, stream);
    if (e == hipSuccess && gv) e = fa::launch_scatter_rows(gv, dV, B, HKV, Sk, bs[2], DT, D, stream);
  } else {
    e = fa::launch_backward(p, dtype, D, stream);
  }
  const hipError_t f = hipFreeAsync(ws, stream);
  return (e == hipSuccess && f == hipSuccess) ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                      const float* LSE, float* dQ, float* dK, float* dV, int B, int H, int HKV,
                      int Sq, int Sk, int D, float scale, int causal, int window, int dtype,
                      void* stream) {
  return backward(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, HKV, Sq, Sk, D, nullptr, scale, causal,
                  window, dtype, stream);
}

extern "C" int fa_bwd_block_sparse(const void* Q, const void* K, const void* V, const void* O,
                                   const void* dO, const float* LSE, float* dQ, float* dK,
                                   float* dV, int B, int H, int HKV, int Sq, int Sk, int D,
                                   const unsigned char* block_mask, int mask_batch,
                                   int mask_heads, float scale, int causal, int window, int dtype,
                                   void* stream) {
  const BwdMask bm = {block_mask, mask_batch, mask_heads};
  return backward(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, HKV, Sq, Sk, D, nullptr, scale, causal,
                  window, dtype, stream, &bm);
}

extern "C" int fa_bwd_strided(const void* Q, const void* K, const void* V, const void* O,
                              const void* dO, const float* LSE, float* dQ, float* dK, float* dV,
                              int B, int H, int HKV, int Sq, int Sk, int D,
                              const long long* q_strides, const long long* k_strides,
                              const long long* v_strides, const long long* o_strides,
                              const long long* do_strides, const long long* dq_strides,
                              const long long* dk_strides, const long long* dv_strides,
                              float scale, int causal, int window, int dtype, void* stream) {
  const long long* const given[8] = {q_strides, k_strides, v_strides, o_strides,
                                     do_strides, dq_strides, dk_strides, dv_strides};
  return backward(Q, K, V, O, dO, LSE, dQ, dK, dV, B, H, HKV, Sq, Sk, D, given, scale, causal,
                  window, dtype, stream);
}

extern "C" int fa_bwd_plan(int B, int H, int HKV, int Sq, int Sk, int D, int causal, int window,
                           int dtype, int num_cus, int* plan) {
  if (!plan) return FA_ERR_NULLPTR;
  const int st = check_bwd(B, H, HKV, Sq, Sk, D, causal, window, dtype);
  if (st != FA_OK) return st;
  if (num_cus < 1) return FA_ERR_SHAPE;
  const BwdPlan pl = plan_backward(B, H, HKV, Sq, Sk, D, causal, window, dtype, true, D, num_cus);
  const int out[8] = {pl.DT, pl.gen, pl.staged, pl.per_row, pl.nch, pl.chunk_q, pl.nrc, pl.chunk_r};
  for (int t = 0; t < 8; ++t) plan[t] = out[t];
  return FA_OK;
}

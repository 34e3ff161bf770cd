// Internal interface between the backward C ABI (fa_bwd_api.cpp) and its
// kernels (fa_bwd.hip). Not installed; callers use include/fa.h.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>

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
  // Small grids: the key range is cut into nch chunks, one per blockIdx.y,
  // whose unscaled partial sums are added up in chunk order afterwards (nch =
  // 1: gradients written directly). Per-row kernels: each row group's range
  // in chunks of chunk_q keys (dQ) or chunk_k query rows (dK/dV), partial sums
  // to part_q [nch][B H Sq][D] and part_k, part_v [nch][B HKV Sk][D]. MFMA
  // dQ kernels: key chunk c = [c chunk_q, (c + 1) chunk_q) (chunk_q a
  // multiple of the 32-key tile), partial sums to part_q.
  int nch, chunk_q, chunk_k;
  float* part_q;
  float* part_k;
  float* part_v;
  // MFMA dK/dV kernels on small grids: the query rows are cut into nrc
  // chunks [c chunk_r, (c + 1) chunk_r) (chunk_r a multiple of 128; chunk c =
  // nrc - 1 - blockIdx.y, the last rows first), each writing unscaled dK and
  // dV partial sums to contiguous rows part_k / part_v [nrc][B HKV Sk][D]
  // (the general form too), added up in chunk order afterwards (nrc = 1: dK
  // and dV written directly).
  int nrc, chunk_r;
  // General form of the 16-bit MFMA kernels (gen = 1): the tensors are views
  // with these element strides (batch, head, row; the head dim contiguous),
  // Q, K, V, O, dO in the input type and dQ, dK, dV in fp32, with head dim
  // dv (a multiple of 16, at most the kernel's tile dim D): the kernels read
  // the dims from dv on as zeros and write only the first dv. gen = 0:
  // contiguous [B, heads, S, D] tensors, strides unused.
  int gen, dv;
  long long qs[3], ks[3], vs[3], os[3], dos[3], dqs[3], dks[3], dvs[3];
  // Block mask (fa_bwd_block_sparse; NULL otherwise): one byte per
  // (kBwdMaskQ query rows, kBwdMaskK keys) block, contiguous
  // [mask batch][mask heads][bm_nqb][bm_nkb]; bm_sb / bm_sh are the batch and
  // head strides in bytes (0 for an axis of extent 1) and bm_by_q says
  // whether the head axis is indexed by the query head (else the kv head).
  const unsigned char* bmask;
  long long bm_sb, bm_sh;
  int bm_nqb, bm_nkb, bm_by_q;
};

// Block-mask granularity (the forward's: FA_MASK_BLOCK_Q x FA_MASK_BLOCK_K).
constexpr int kBwdMaskQ = 128, kBwdMaskK = 64;
// Longest visible-tile list a masked backward workgroup keeps in LDS: key
// tiles of a dQ workgroup (chunks of the key axis beyond that), and
// (query head, 128-row block) pairs of a dK/dV workgroup.
constexpr int kBwdMaxList = 8192;

// Group shape of the per-row kernels (fp32 inputs, D = 256): lanes per row
// (a group holds D / lanes elements of each row vector per lane: the fewest
// lanes, 4, 8, 16 or 32, that keep it at most 8) and rows of one head per
// group (4 with 16 lanes, 2 otherwise; each measured best).
constexpr int bwd_lanes_per_row(int D) { return D <= 32 ? 4 : D <= 64 ? 8 : D <= 128 ? 16 : 32; }
constexpr int bwd_rows_per_group(int D) { return bwd_lanes_per_row(D) == 16 ? 4 : 2; }

// fp32 inputs at these head dims run the MFMA backward kernels (16, 48 and 80
// staged into the 32, 64, 96 tiles when the work is large, else the per-row
// kernels; 256 with its dims split over wavefront pairs); 16-bit inputs
// always run MFMA kernels.
constexpr bool bwd_f32_mfma(int D) { return D == 32 || D == 64 || D == 96 || D == 128 || D == 256; }

constexpr int kBwdThreads = 256;   // threads per backward workgroup (4 wavefronts)
constexpr float kLog2e = 1.4426950408889634f;

// Queue the dQ kernel (which also writes Dws) and then the dK/dV kernel.
hipError_t launch_backward(const BwdParams& p, int dtype, int D, hipStream_t stream);

// The fp32 MFMA kernels (fa_bwd_f32.hip; D one of bwd_f32_mfma's dims): the
// dQ kernel (key chunks on blockIdx.y when p.nch > 1) and the dK/dV kernel
// (row chunks on blockIdx.y when p.nrc > 1); at D = 256 64 query rows (keys)
// per workgroup instead of 128.
hipError_t launch_bwd_f32_mfma_dq(const BwdParams& p, int D, hipStream_t stream);
hipError_t launch_bwd_f32_mfma_dkdv(const BwdParams& p, int D, hipStream_t stream);

// Row copies of the staged backward (fp32 views, and 16-bit views whose row
// strides exceed what the general form's copy offsets allow): inputs copied
// to contiguous zero-padded rows first, gradients copied back. gather: the B heads S rows of a view with byte strides st (batch,
// head, row; multiples of 16), src_bytes each, -> contiguous rows of
// dst_bytes with zeros after src_bytes. scatter: contiguous fp32 rows of dt
// floats -> the first dv floats of each row of an fp32 view (byte strides st).
hipError_t launch_gather_rows(const void* src, void* dst, int B, int heads, int S,
                              const long long st[3], int src_bytes, int dst_bytes,
                              hipStream_t stream);
hipError_t launch_scatter_rows(const float* src, void* dst, int B, int heads, int S,
                               const long long st[3], int dt, int dv, hipStream_t stream);

// True when the rows of a [B, heads, S, D] view with element strides st
// (batch, head, row) are pairwise disjoint (fa_api.cpp).
bool output_rows_disjoint(const long long st[3], int B, int heads, int S, int D);

// Compute units of the current device (cached; fa_api.cpp), 0 on error.
int device_cus();

// Stream-ordered workspace of `bytes` from the library's memory pool on the
// current device (fa_api.cpp); release with hipFreeAsync. Returns an fa_status.
int library_workspace(size_t bytes, hipStream_t stream, void** out);

}  // namespace fa

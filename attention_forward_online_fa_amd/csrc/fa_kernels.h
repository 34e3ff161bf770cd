// Internal interface between the C ABI (fa_api.cpp) and the kernels
// (fa_fwd.hip). Not installed; callers use include/fa.h.
#pragma once
#include <hip/hip_runtime.h>
#include <cstddef>

namespace fa {

// Everything one forward launch needs. Built and checked on the host.
struct Params {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* LSE;
  float* Opart;      // [nsplit][B*H*Sq][D] fp32 partial outputs (nsplit > 1)
  float* Lpart;      // [nsplit][B*H*Sq]    partial log-sum-exp    (nsplit > 1)
  int B, H, HKV, Sq, Sk;
  int group;         // H / HKV
  float sl;          // scale * log2(e): scores are kept in base-2 units
                     // (16-bit kernel: |scale| * log2(e) > 0, see neg_q)
  int neg_q;         // 16-bit kernel: 1 when scale < 0 (it then uses -Q and |scale|)
  int causal;
  int window;
  int nsplit;        // key-axis splits (1 = none)
  int split_len;     // keys per split, a multiple of the key tile
  int n_qblk;        // ceil(Sq / BM)
  int units;         // B * H * nsplit
  int xcd_remap;     // 1: group work so units sharing K/V stay on one XCD
  // Persistent launch (fp32 kernel): nslot workgroups, workgroup s runs the
  // items sched[nslot + 1 + k] for k in [sched[s], sched[s + 1]), item =
  // qblk * units + unit. Null: one workgroup per item in the default order.
  const int* sched;
  int nslot;
  // Element strides (batch, head, row) of Q, K, V and O; the head dimension
  // is contiguous. Contiguous [B, heads, S, D] tensors have (heads S D, S D, D);
  // the kernels read them only in their strided form (Strided = true), where
  // the row strides of K and V are multiples of D.
  long long qs[3], ks[3], vs[3], os[3];
  // Block mask (kFormBlockSparse): bytes [mask batch][mask heads][n_qblk][bm_nkb];
  // a nonzero byte makes its kBlockM-row x kMaskBlockK-key block visible.
  // Row (b, h, qblk) of the mask starts at bmask + b bm_sb + hm bm_sh + qblk bm_nkb
  // with hm = kv head if bm_by_kv, else query head (strides 0 = shared axis).
  const unsigned char* bmask;
  long long bm_sb, bm_sh;
  int bm_nkb;
  int bm_by_kv;
};

// Kernel forms: contiguous tensors, strided tensors (p.qs .. p.os), and
// contiguous tensors under a block mask.
constexpr int kFormContiguous = 0;
constexpr int kFormStrided = 1;
constexpr int kFormBlockSparse = 2;
// Keys per block-mask byte, and the most key tiles one workgroup's range may
// hold under a block mask (its visible-tile list lives in LDS).
constexpr int kMaskBlockK = 64;
constexpr int kMaxListTiles = 2048;

// Tile shape per (dtype, D): query rows per workgroup and keys per K/V tile.
constexpr int kBlockM = 128;
int key_tile(int dtype, int D);
int block_m(int dtype, int D);
// Workgroups of the fp32 kernel (in the given form) that fit on one CU at
// head dim D (0 on error).
int f32_blocks_per_cu(int D, int form);

// Queue the forward kernel (and the merge kernel when p.nsplit > 1) in the
// given form (kFormContiguous: p.qs .. p.os and the mask are not read).
hipError_t launch_forward(const Params& p, int dtype, int D, int form, hipStream_t stream);

}  // namespace fa

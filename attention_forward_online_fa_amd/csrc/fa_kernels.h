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
  float* Opart;      // [nsplit][B*H*Sq][DT] fp32 partial outputs (nsplit > 1; DT = tile dim)
  float* Lpart;      // [nsplit][B*H*Sq]    partial log-sum-exp    (nsplit > 1)
  int B, H, HKV, Sq, Sk;
  int dv;            // head dim of the tensors (kFormPadded: below the kernel's tile dim)
  int group;         // H / HKV
  float sl;          // scale * log2(e): scores are kept in base-2 units
                     // (16-bit kernel: |scale| * log2(e) > 0, see neg_q)
  int neg_q;         // 16-bit kernel: 1 when scale < 0 (it then uses -Q and |scale|)
  int causal;
  int window;
  int nsplit;        // key-axis splits (1 = none)
  int split_len;     // keys per split, a multiple of the key tile
  int n_qblk;        // ceil(Sq / rows per workgroup)
  int units;         // B * HKV * packs * nsplit
  // Query heads per workgroup (16-bit kernel: 1, 2 or 4; fp32 kernel: 1).
  // Its four wavefronts take hp heads of one kv head times 4 / hp groups of
  // 32 rows, so a workgroup holds kBlockM / hp query rows of each of its
  // heads; packs = group / hp workgroups cover a kv head's query heads.
  int hp;
  int packs;
  int bm;            // query rows per workgroup (of each of its hp heads): kBlockM / hp
  int xcd_remap;     // 1: units sharing K/V stay on one XCD (query tile major);
                     // 2: sliding windows over fewer than 8 kv units (see map_tile)
  // Persistent launch (fp32 kernel): nslot workgroups, workgroup s runs the
  // items sched[nslot + 1 + k] for k in [sched[s], sched[s + 1]), item =
  // qblk * units + unit. Null: one workgroup per item in the default order.
  const int* sched;
  int nslot;
  // Element strides (batch, head, row) of Q, K, V and O; the head dimension
  // is contiguous. Contiguous [B, heads, S, D] tensors have (heads S D, S D, D);
  // the kernels read them only in their strided and padded forms. In the
  // strided form the row strides of K and V are multiples of D; the padded
  // form takes any row stride that keeps rows 16-byte aligned.
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

// Kernel forms: contiguous tensors, strided tensors (p.qs .. p.os),
// contiguous tensors under a block mask, and padded: strided tensors whose
// head dim p.dv (a multiple of 16) is below the kernel's tile dim, the
// remaining dims of every Q row and K/V tile row held as zeros on chip.
constexpr int kFormContiguous = 0;
constexpr int kFormStrided = 1;
constexpr int kFormBlockSparse = 2;
constexpr int kFormPadded = 3;
constexpr int kForms = 4;
// Keys per block-mask byte, and the most key tiles one workgroup's range may
// hold under a block mask (its visible-tile list lives in LDS).
constexpr int kMaskBlockK = 64;
constexpr int kMaxListTiles = 2048;

// Tile shape per (dtype, D): query rows per workgroup and keys per K/V tile.
constexpr int kBlockM = 128;
// Query tiles per chunk of the sliding-window XCD order (Params::xcd_remap 2).
constexpr int kXcdChunk = 8;
int key_tile(int dtype, int D);
int block_m(int dtype, int D);
// Workgroups of the fp32 kernel (in the given form) that fit on one CU at
// tile dim D (0 on error).
int f32_blocks_per_cu(int D, int form);

// Tile dim of the kernel that serves head dim dv for the input type (0:
// unsupported). 16-bit kernels: 64, 128, 256 natively; 16, 32, 48 padded to
// 64 and 80, 96 to 128. fp32 kernel: 32, 64, 96, 128, 256 natively; 16
// padded to 32, 48 to 64 and 80 to 96.
constexpr int tile_dim(int dv, int dtype) {
  if (dv == 64 || dv == 128 || dv == 256) return dv;
  if (dtype == 0) {
    return dv == 32 || dv == 96 ? dv : dv == 16 ? 32 : dv == 48 ? 64 : dv == 80 ? 96 : 0;
  }
  return (dv == 16 || dv == 32 || dv == 48) ? 64 : (dv == 80 || dv == 96) ? 128 : 0;
}

// A fixed workspace for the split partials: `address` stores the current
// device's address of `bytes` bytes of device memory (256-byte aligned) and
// returns an fa_status; the forward calls it once, after the argument checks,
// and then allocates nothing.
struct FixedWorkspace {
  int (*address)(void** out);
  size_t bytes;
};

// fa_fwd_ex into a fixed workspace (fa_api.cpp): no persistent schedule, and
// an automatic split count lowered until the partials fit; an explicit count
// that does not fit returns FA_ERR_WORKSPACE.
int forward_fixed_workspace(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int B, int H, int HKV, int Sq, int Sk, int D, float scale,
                            int causal, int window, int dtype, int num_splits, void* stream,
                            const FixedWorkspace& ws);

// Queue the forward kernel (and the merge kernel when p.nsplit > 1) in the
// given form at tile dim D (kFormContiguous: p.qs .. p.os and the mask are
// not read; kFormPadded: D = tile_dim(p.dv, dtype) > p.dv).
hipError_t launch_forward(const Params& p, int dtype, int D, int form, hipStream_t stream);

}  // namespace fa

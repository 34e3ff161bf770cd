// Device helpers shared by the backward kernels (fa_bwd.hip and
// fa_bwd_f32.hip): block-mask rows and the visible-tile lists of the masked
// backward. Not installed; callers use include/fa.h.
#pragma once
#include <hip/hip_runtime.h>

#include "fa_bwd.h"

namespace fa {

// Block masks: the mask row of query block qb for (b, h) (head axis indexed
// by the query head or the kv head, per p.bm_by_q; strides 0 for axes of
// extent 1).
__device__ __forceinline__ const unsigned char* bwd_mask_row(const BwdParams& p, int b, int h,
                                                             int hkv, int qb) {
  return p.bmask + b * p.bm_sb + (p.bm_by_q ? h : hkv) * p.bm_sh + (long long)qb * p.bm_nkb;
}

// Block masks: the candidates c in [c0, n) with nonzero flags vis(c) go, in
// order, to list[] as entry(c, flags), until the list is full (Cap entries); wave 0 scans 64 candidates per ballot round, with the mask reads
// of four rounds in flight at once. Returns the count (uniform) and sets
// *next to the first candidate not scanned (n once every candidate was). sh
// is two ints of LDS.
template <int Cap = kBwdMaxList, typename Vis, typename Ent>
__device__ __forceinline__ int bwd_build_list(int c0, int n, unsigned* list, int* sh, int wave,
                                              int lane, Vis vis, Ent entry, int* next) {
  constexpr int kAhead = 4;
  __syncthreads();   // the previous list's readers are done with it
  if (wave == 0) {
    int cnt = 0, c = c0;
    while (c < n && cnt + 64 <= Cap) {
      unsigned f[kAhead];
#pragma unroll
      for (int r = 0; r < kAhead; ++r) {
        const int t = c + 64 * r + lane;
        f[r] = t < n ? vis(t) : 0u;
      }
#pragma unroll
      for (int r = 0; r < kAhead; ++r) {
        if (c >= n || cnt + 64 > Cap) break;
        const unsigned long long bal = __ballot(f[r] != 0u);
        if (f[r] != 0u) list[cnt + __popcll(bal & ((1ull << lane) - 1ull))] = entry(c + lane, f[r]);
        cnt += __popcll(bal);
        c += 64;
      }
    }
    if (lane == 0) {
      sh[0] = cnt;
      sh[1] = min(c, n);
    }
  }
  __syncthreads();
  *next = __builtin_amdgcn_readfirstlane(sh[1]);
  return __builtin_amdgcn_readfirstlane(sh[0]);
}

}  // namespace fa

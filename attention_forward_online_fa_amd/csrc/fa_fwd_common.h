// Device helpers of the forward kernels (fa_fwd.hip): the mapping of
// workgroups to work tiles, the key range of a tile, the visibility rule, the
// epilogue of one query row and the cross-half row max.
// Not installed; callers use include/fa.h.
#pragma once
#include <hip/hip_runtime.h>

#include "fa_kernels.h"

namespace fa {

constexpr int kThreads = 256;   // 4 wavefronts of 64
constexpr float kLn2 = 0.693147180559945309f;


// ------------------------------------------------------------ work mapping
struct Tile {
  int b, h, hkv, qblk, split;
};

__device__ __forceinline__ Tile map_tile(const Params& p) {
  const int i = blockIdx.x;
  int t, u;
  if (p.xcd_remap == 2) {
    // Sliding windows with fewer than 8 kv units (K/V heads times splits):
    // the R = 8 / G XCDs of kv unit g = x / R share its query tiles in
    // chunks of kXcdChunk consecutive tiles (every pack of each), dealt in
    // snake order (r, 2R - 1 - r per period of 2R chunks) so that the light
    // tiles where the window is still filling spread evenly, and run
    // heaviest chunk first. The workgroups an XCD runs at once then hold
    // every query head of one K/V head over one or two runs of consecutive
    // tiles: their windows overlap and the keys they read at one time stay in
    // that XCD's L2 (the query-tile-major order below spreads an XCD's
    // concurrent workgroups over a whole window of keys).
    const int x = i & 7, k = i >> 3;
    const int R = 8 / (p.units / p.packs);
    const int g = x / R, r = x % R;
    const int per_chunk = kXcdChunk * p.packs;
    const int s = k / per_chunk, o = k % per_chunk;
    const int periods = p.n_qblk / (kXcdChunk * 2 * R);
    const int period = periods - 1 - (s >> 1);
    const int chunk = period * 2 * R + ((s & 1) ? r : 2 * R - 1 - r);
    const int qb = chunk * kXcdChunk + kXcdChunk - 1 - o / p.packs;
    t = p.n_qblk - 1 - qb;
    u = g * p.packs + o % p.packs;
  } else if (p.xcd_remap) {
    // Block i runs on XCD i % 8 as that XCD's (i / 8)-th block. Give XCD x
    // the contiguous unit range [x U/8, (x+1) U/8).
    // Within an XCD: query tile major (heaviest first), then unit; the units
    // of one XCD are consecutive, so query heads sharing a K/V head run there
    // together. (Ordering kv-head-group major instead measured ~1.5% slower.)
    const int upx = p.units >> 3;
    const int k = i >> 3;
    t = k / upx;
    u = (i & 7) * upx + k % upx;
  } else {
    t = i / p.units;
    u = i % p.units;
  }
  Tile w;
  w.qblk = p.n_qblk - 1 - t;
  const int pk = u % p.packs;
  int r = u / p.packs;
  w.split = r % p.nsplit;
  r /= p.nsplit;
  w.hkv = r % p.HKV;
  w.b = r / p.HKV;
  w.h = w.hkv * p.group + pk * p.hp;   // the workgroup's first query head
  return w;
}

// Work tile of item qblk * units + unit in a persistent launch (the unit
// decomposition of map_tile, without its XCD grouping).
__device__ __forceinline__ Tile item_tile(const Params& p, int item) {
  Tile w;
  w.qblk = item / p.units;
  const int u = item % p.units;
  const int pk = u % p.packs;
  int r = u / p.packs;
  w.split = r % p.nsplit;
  r /= p.nsplit;
  w.hkv = r % p.HKV;
  w.b = r / p.HKV;
  w.h = w.hkv * p.group + pk * p.hp;
  return w;
}

// Key range [lo, hi) a workgroup with rows [q0, q0 + bm) must visit.
__device__ __forceinline__ void key_range(const Params& p, int q0, int bm, int split, int& lo,
                                          int& hi) {
  lo = split * p.split_len;
  hi = min(p.Sk, lo + p.split_len);
  const int last = min(q0 + bm, p.Sq) - 1;
  if (p.causal) hi = min(hi, last + 1);
  if (p.window > 0) lo = max(lo, q0 - p.window + 1);
}

__device__ __forceinline__ bool visible(const Params& p, int i, int j) {
  return j < p.Sk && (!p.causal || j <= i) && (p.window <= 0 || j > i - p.window);
}

// Finish one query row: combine the two lane halves' row sums, then write
// LSE and hand 1/l to `store(partial, row, split, inv)`, which writes O (or
// the fp32 partial of this key split).
template <typename StoreFn>
__device__ __forceinline__ void finish_row(const Params& p, int b, int h, int split, int i,
                                           int g, float m, float l_lane, StoreFn store) {
  const float l = l_lane + __shfl_xor(l_lane, 32);
  const bool any = l > 0.f;
  const float inv = any ? 1.f / l : 0.f;
  const float lse = any ? (m + __log2f(l)) * kLn2 : -INFINITY;
  if (i >= p.Sq) return;
  const size_t row = (size_t)(b * p.H + h) * p.Sq + i;
  const bool partial = p.nsplit > 1;
  // A split row that saw no key needs only its LSE (-inf): the merge skips it.
  if (!partial || any) store(partial, row, split, inv);
  if (g == 0) {
    if (partial)
      p.Lpart[(size_t)split * p.B * p.H * p.Sq + row] = lse;
    else
      p.LSE[row] = lse;
  }
}

__device__ __forceinline__ float half_max(float x) {
  // max over lane and lane ^ 32 (the two halves of one query row's keys)
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace fa

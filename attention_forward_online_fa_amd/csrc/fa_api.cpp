// C ABI of the fused attention forward pass: argument checks, key-split
// planning, the split workspace, and the launch. Declared in include/fa.h.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <queue>
#include <vector>

#include "fa_bwd.h"
#include "fa_kernels.h"

namespace {

constexpr int kMaxDevices = 64;

// A persistent-launch schedule: [nslot + 1] offsets, then item ids, on the
// host and (uploaded once) on the device.
struct Sched {
  std::vector<int> host;
  int* dev = nullptr;
};
using SchedKey = std::array<int, 12>;

struct DeviceState {
  bool init = false;
  int num_cus = 0;
  int f32_bpc[fa::kForms][5];   // fp32 workgroups per CU [form][D = 32, 64, 96, 128, 256]; -1 = not queried
  DeviceState() {
    for (auto& f : f32_bpc)
      for (int& x : f) x = -1;
  }
  hipMemPool_t pool = nullptr;
  std::map<SchedKey, Sched> scheds;
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];

// Per-device facts and the split-workspace pool, created on first use.
// The pool keeps freed blocks cached (release threshold = max) so steady-state
// calls do not go back to the driver; fa_release() trims it.
int device_state(DeviceState** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lk(g_mu);
  DeviceState& s = g_dev[dev];
  if (!s.init) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return FA_ERR_HIP;
    s.num_cus = cus > 0 ? cus : 1;
    s.init = true;
  }
  *out = &s;
  return FA_OK;
}

int workspace_pool(int dev_index, DeviceState& s, hipMemPool_t* pool) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!s.pool) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev_index;
    if (hipMemPoolCreate(&s.pool, &props) != hipSuccess) {
      s.pool = nullptr;
      return FA_ERR_WORKSPACE;
    }
    uint64_t thr = UINT64_MAX;
    // Best effort: without the threshold the pool still works, it only hands
    // memory back at synchronisation points.
    (void)hipMemPoolSetAttribute(s.pool, hipMemPoolAttrReleaseThreshold, &thr);
  }
  *pool = s.pool;
  return FA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_args(int B, int H, int HKV, int Sq, int Sk, int D, int causal, int window,
               int dtype) {
  if (B < 1 || H < 1 || HKV < 1 || Sq < 1 || Sk < 1 || D < 1) return FA_ERR_SHAPE;
  if (dtype != FA_F32 && dtype != FA_BF16 && dtype != FA_F16) return FA_ERR_DTYPE;
  if (fa::tile_dim(D, dtype) == 0) return FA_ERR_HEAD_DIM;
  if (H % HKV != 0) return FA_ERR_GQA;
  if (window < 0 || (causal != 0 && causal != 1)) return FA_ERR_WINDOW;
  const int esz = dtype == FA_F32 ? 4 : 2;
  // Element counts must stay far from 64-bit overflow in every address.
  const double q_bytes = (double)B * H * Sq * D * esz;
  const double kv_bytes = (double)B * HKV * Sk * D * esz;
  if (q_bytes > 4.0e18 || kv_bytes > 4.0e18) return FA_ERR_SHAPE;
  // Row indices (b*H + h)*Sq + i are computed in 32-bit signed products of
  // int operands before widening; keep every operand product in range.
  if ((double)B * H * Sq >= 2147483647.0 || (double)B * HKV * Sk >= 2147483647.0)
    return FA_ERR_SHAPE;
  return FA_OK;
}

// Number of key-axis splits: only when the query tiles alone cannot fill the
// GPU (fewer tiles than compute units), and never below 4 key tiles per split.
int auto_splits(int B, int H, int Sq, int Sk, int D, int causal, int window, int dtype,
                int num_cus) {
  const int BM = fa::block_m(dtype, D), BN = fa::key_tile(dtype, D);
  const long n_qblk = (Sq + BM - 1) / BM;
  const long work = (long)B * H * n_qblk;
  if (work >= num_cus) return 1;
  long span = Sk;
  if (causal) span = std::min<long>(span, Sq);
  if (window > 0) span = std::min<long>(span, (long)window + BM);
  const long tiles = (span + BN - 1) / BN;
  long ns = (2L * num_cus + work - 1) / work;
  ns = std::min<long>(ns, tiles / 4);
  ns = std::min<long>(ns, FA_MAX_SPLITS);
  return ns < 1 ? 1 : (int)ns;
}

// ---- persistent schedules for the fp32 kernel on small causal / windowed grids
// Query tiles of a causal or windowed problem see very different numbers of
// keys. With too few tiles to give every CU several, the longest tile sets
// the kernel time and most CUs idle at the end. Such launches split the key
// axis so that no piece is much longer than the average load of a workgroup
// slot, and run one persistent workgroup per slot (as many slots as the
// kernel's occupancy allows) over a host-computed list of pieces whose total
// cost is balanced: longest first onto the least loaded slot, then moves and
// swaps out of the most loaded slot while they lower the maximum.
constexpr int kItemCost2 = 5;   // fixed cost per piece (start-up, epilogue), in half key tiles

// Key tiles a workgroup visits: the host twin of key_range in the kernels.
int item_tiles(int q0, int BM, int BN, int split, int split_len, int Sq, int Sk, int causal,
               int window) {
  int lo = split * split_len;
  int hi = std::min(Sk, lo + split_len);
  const int last = std::min(q0 + BM, Sq) - 1;
  if (causal) hi = std::min(hi, last + 1);
  if (window > 0) lo = std::max(lo, q0 - window + 1);
  const int t0 = (lo / BN) * BN;
  return hi > lo ? (hi - t0 + BN - 1) / BN : 0;
}

// Slots of a persistent launch for this problem, or 0 when it runs one
// workgroup per item.
int persistent_slots(DeviceState& s, int B, int H, int Sq, int D, int causal, int window,
                     int dtype, int form) {
  if (dtype != FA_F32 || (!causal && window <= 0)) return 0;
  const int BM = fa::block_m(dtype, D);
  const long qtiles = (long)B * H * ((Sq + BM - 1) / BM);
  if (qtiles >= 2L * s.num_cus) return 0;
  const int di = D == 32 ? 0 : D == 64 ? 1 : D == 96 ? 2 : D == 128 ? 3 : 4;
  int& bpc = s.f32_bpc[form][di];
  if (bpc < 0) bpc = fa::f32_blocks_per_cu(D, form);
  return bpc > 0 ? bpc * s.num_cus : 0;
}

// Key splits for a persistent launch: the longest query tile cut into pieces
// of about the average slot load.
int persistent_splits(int B, int H, int Sq, int Sk, int D, int causal, int window, int dtype,
                      int nslot) {
  const int BM = fa::block_m(dtype, D), BN = fa::key_tile(dtype, D);
  const int n_qblk = (Sq + BM - 1) / BM;
  long total = 0;
  int longest = 0;
  for (int qb = 0; qb < n_qblk; ++qb) {
    const int t = item_tiles(qb * BM, BM, BN, 0, Sk, Sq, Sk, causal, window);
    total += t;
    longest = std::max(longest, t);
  }
  total *= (long)B * H;
  const double avg = (double)total / nslot + kItemCost2 / 2.0;
  const int sk_tiles = (Sk + BN - 1) / BN;
  int ns = (int)std::ceil(longest / avg);
  return std::max(1, std::min({ns, FA_MAX_SPLITS, sk_tiles}));
}

// Balanced item lists for nslot workgroups: [nslot + 1] offsets, then the
// item ids (item = qblk * units + unit, unit = ((b HKV + hkv) ns + split)
// group + head-in-group, as the kernel decodes it).
std::vector<int> build_schedule(int B, int H, int HKV, int Sq, int Sk, int D, int causal,
                                int window, int dtype, int ns, int split_len, int nslot) {
  const int BM = fa::block_m(dtype, D), BN = fa::key_tile(dtype, D);
  const int n_qblk = (Sq + BM - 1) / BM;
  const int group = H / HKV, units = B * H * ns;
  const int n = n_qblk * units;
  std::vector<int> tiles(n), cost(n);
  for (int it = 0; it < n; ++it) {
    const int qb = it / units, split = (it % units / group) % ns;
    tiles[it] = item_tiles(qb * BM, BM, BN, split, split_len, Sq, Sk, causal, window);
    cost[it] = 2 * tiles[it] + kItemCost2;
  }
  // longest first onto the least loaded slot
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return cost[a] > cost[b]; });
  std::vector<std::vector<int>> slot(nslot);
  std::vector<long> load(nslot, 0);
  using LS = std::pair<long, int>;
  std::priority_queue<LS, std::vector<LS>, std::greater<LS>> heap;
  for (int sl = 0; sl < nslot; ++sl) heap.push({0, sl});
  for (int it : order) {
    const LS top = heap.top();
    heap.pop();
    slot[top.second].push_back(it);
    load[top.second] = top.first + cost[it];
    heap.push({load[top.second], top.second});
  }
  // moves and swaps out of the most loaded slot while they lower its load
  // below the old maximum without raising the other slot to it
  for (int iter = 0; iter < 2000; ++iter) {
    const int mx = (int)(std::max_element(load.begin(), load.end()) - load.begin());
    long best_gain = 0;
    int bi = -1, bs = -1, bj = -1;
    for (int a = 0; a < (int)slot[mx].size(); ++a) {
      const int ci = cost[slot[mx][a]];
      for (int sl = 0; sl < nslot; ++sl) {
        if (sl == mx) continue;
        if (load[sl] + ci < load[mx]) {
          const long gain = load[mx] - std::max(load[sl] + ci, load[mx] - ci);
          if (gain > best_gain) { best_gain = gain; bi = a; bs = sl; bj = -1; }
        }
        for (int b = 0; b < (int)slot[sl].size(); ++b) {
          const int d = ci - cost[slot[sl][b]];
          if (d > 0 && load[sl] + d < load[mx]) {
            const long gain = load[mx] - std::max(load[sl] + d, load[mx] - d);
            if (gain > best_gain) { best_gain = gain; bi = a; bs = sl; bj = b; }
          }
        }
      }
    }
    if (bi < 0) break;
    const int it = slot[mx][bi];
    slot[mx].erase(slot[mx].begin() + bi);
    load[mx] -= cost[it];
    if (bj >= 0) {
      const int jt = slot[bs][bj];
      slot[bs].erase(slot[bs].begin() + bj);
      load[bs] -= cost[jt];
      slot[mx].push_back(jt);
      load[mx] += cost[jt];
    }
    slot[bs].push_back(it);
    load[bs] += cost[it];
  }
  std::vector<int> table;
  table.reserve(nslot + 1 + n);
  table.push_back(0);
  for (int sl = 0; sl < nslot; ++sl) table.push_back(table.back() + (int)slot[sl].size());
  for (int sl = 0; sl < nslot; ++sl) {
    std::stable_sort(slot[sl].begin(), slot[sl].end(), [&](int a, int b) { return tiles[a] > tiles[b]; });
    table.insert(table.end(), slot[sl].begin(), slot[sl].end());
  }
  return table;
}

// Final split count and keys per split for a requested count (0 = auto).
void resolve_splits(int requested, int B, int H, int Sq, int Sk, int D, int causal, int window,
                    int dtype, int num_cus, int* ns_out, int* split_len_out) {
  const int BN = fa::key_tile(dtype, D);
  int ns = requested == 0 ? auto_splits(B, H, Sq, Sk, D, causal, window, dtype, num_cus)
                          : requested;
  const int sk_tiles = (Sk + BN - 1) / BN;
  if (ns > sk_tiles) ns = sk_tiles;
  if (ns < 1) ns = 1;
  // Keys per split, a whole number of tiles; the last split may be shorter.
  const int split_len = ((sk_tiles + ns - 1) / ns) * BN;
  *ns_out = (Sk + split_len - 1) / split_len;
  *split_len_out = split_len;
}

// Splits, keys per split and persistent slots (0 = none) for one call.
// (persistent = false: one workgroup per item, whatever the shape)
void plan(DeviceState& s, int requested, int B, int H, int Sq, int Sk, int D, int causal,
          int window, int dtype, int form, int* ns, int* split_len, int* nslot,
          bool persistent = true) {
  *nslot = 0;
  if (persistent) {
    std::lock_guard<std::mutex> lk(g_mu);
    *nslot = persistent_slots(s, B, H, Sq, D, causal, window, dtype, form);
  }
  if (*nslot > 0 && requested == 0)
    requested = persistent_splits(B, H, Sq, Sk, D, causal, window, dtype, *nslot);
  resolve_splits(requested, B, H, Sq, Sk, D, causal, window, dtype, s.num_cus, ns, split_len);
  if (form == fa::kFormBlockSparse && *split_len / fa::key_tile(dtype, D) > fa::kMaxListTiles) {
    // a workgroup's visible-tile list holds at most kMaxListTiles tiles: split
    // the key axis at least that finely
    const int sk_tiles = (Sk + fa::key_tile(dtype, D) - 1) / fa::key_tile(dtype, D);
    const int need = (sk_tiles + fa::kMaxListTiles - 1) / fa::kMaxListTiles;
    resolve_splits(std::min(std::max(need, *ns), FA_MAX_SPLITS), B, H, Sq, Sk, D, causal, window,
                   dtype, s.num_cus, ns, split_len);
  }
}

// The device copy of a persistent schedule, built and uploaded on first use
// (a synchronous copy, so every stream sees it) and kept until fa_release.
int schedule_for(DeviceState& s, int B, int H, int HKV, int Sq, int Sk, int D, int causal,
                 int window, int dtype, int ns, int split_len, int nslot, const int** out) {
  const SchedKey key = {B, H, HKV, Sq, Sk, D, causal, window, dtype, ns, split_len, nslot};
  std::lock_guard<std::mutex> lk(g_mu);
  auto found = s.scheds.find(key);
  if (found == s.scheds.end()) {
    Sched sc;
    sc.host = build_schedule(B, H, HKV, Sq, Sk, D, causal, window, dtype, ns, split_len, nslot);
    const size_t bytes = sc.host.size() * sizeof(int);
    if (hipMalloc(reinterpret_cast<void**>(&sc.dev), bytes) != hipSuccess) return FA_ERR_WORKSPACE;
    if (hipMemcpy(sc.dev, sc.host.data(), bytes, hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipFree(sc.dev);
      return FA_ERR_HIP;
    }
    found = s.scheds.emplace(key, std::move(sc)).first;
  }
  *out = found->second.dev;
  return FA_OK;
}

// Element strides (batch, head, row) of one tensor: the caller's, or those of a
// contiguous [B, heads, S, D] tensor when `given` is NULL.
void tensor_strides(const long long* given, int heads, int S, int D, long long out[3]) {
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

// Stride rules: non-negative; every row start 16-byte aligned; rows of one
// head do not overlap (row stride >= D); for K and V a key tile spans less
// than 2^31 bytes and, at D = 64, 128 and 256, the row stride is a multiple
// of D (the strided form's swizzled LDS copies need it; the padded form of
// the other head dims addresses each copied chunk in full); every element
// offset fits far inside int64.
int check_strides(const long long st[3], int B, int heads, int S, int D, int esz, bool kv) {
  const int dtype = esz == 4 ? FA_F32 : FA_BF16;   // (the 16-bit types share their tiles)
  for (int a = 0; a < 3; ++a)
    if (st[a] < 0 || (st[a] * esz) % 16 != 0) return FA_ERR_STRIDE;
  if (st[2] < D) return FA_ERR_STRIDE;
  if (kv && ((fa::tile_dim(D, dtype) == D && st[2] % D != 0) ||
             (double)st[2] * esz * 64 >= 2147483647.0))
    return FA_ERR_STRIDE;
  const double last = (double)(B - 1) * st[0] + (double)(heads - 1) * st[1] +
                      (double)(S - 1) * st[2] + D;
  if (last * esz > 4.0e18) return FA_ERR_SHAPE;
  return FA_OK;
}

// Block mask of fa_fwd_block_sparse (NULL for the dense entry points).
struct MaskArg {
  const unsigned char* mask;
  int batch, heads;
};

// Split workspace bytes: fp32 partial rows of the tile dim, then the partial
// log-sum-exps.
size_t split_workspace_bytes(int ns, int B, int H, int Sq, int DT) {
  const size_t rows = (size_t)B * H * Sq;
  return (size_t)ns * rows * DT * sizeof(float) + (size_t)ns * rows * sizeof(float);
}

}  // namespace

namespace fa {
// O's rows must be disjoint: with its (batch, head, row) axes sorted by stride
// (axes of extent 1 left out), every stride must reach past the extent the
// smaller axes span (a row spans D elements).
bool output_rows_disjoint(const long long st[3], int B, int H, int Sq, int D) {
  std::array<std::pair<long long, long long>, 3> ax = {
      std::make_pair(st[2], (long long)Sq), std::make_pair(st[1], (long long)H),
      std::make_pair(st[0], (long long)B)};
  std::sort(ax.begin(), ax.end());
  long long span = D;   // elements covered by the axes already placed
  for (const auto& a : ax) {
    if (a.second == 1) continue;
    if (a.first < span) return false;
    span = a.first * (a.second - 1) + span;
  }
  return true;
}
}  // namespace fa

namespace {
using fa::output_rows_disjoint;

int forward(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
            int HKV, int Sq, int Sk, int D, const long long* q_strides,
            const long long* k_strides, const long long* v_strides, const long long* o_strides,
            float scale, int causal, int window, int dtype, int num_splits, void* stream_ptr,
            const MaskArg* bm = nullptr, const fa::FixedWorkspace* fixed = nullptr) {
  if (!Q || !K || !V || !O || !LSE || (bm && !bm->mask)) return FA_ERR_NULLPTR;
  int st = check_args(B, H, HKV, Sq, Sk, D, causal, window, dtype);
  if (st != FA_OK) return st;
  if (bm && ((bm->batch != 1 && bm->batch != B) ||
             (bm->heads != 1 && bm->heads != HKV && bm->heads != H)))
    return FA_ERR_MASK;
  if (num_splits < 0 || num_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return FA_ERR_ALIGN;
  const int esz = dtype == FA_F32 ? 4 : 2;
  long long qs[3], ks[3], vs[3], os[3];
  tensor_strides(q_strides, H, Sq, D, qs);
  tensor_strides(k_strides, HKV, Sk, D, ks);
  tensor_strides(v_strides, HKV, Sk, D, vs);
  tensor_strides(o_strides, H, Sq, D, os);
  if ((st = check_strides(qs, B, H, Sq, D, esz, false)) != FA_OK ||
      (st = check_strides(ks, B, HKV, Sk, D, esz, true)) != FA_OK ||
      (st = check_strides(vs, B, HKV, Sk, D, esz, true)) != FA_OK ||
      (st = check_strides(os, B, H, Sq, D, esz, false)) != FA_OK)
    return st;
  if (!output_rows_disjoint(os, B, H, Sq, D)) return FA_ERR_STRIDE;
  // The kernels' contiguous form whenever the strides are those of contiguous tensors.
  long long cq[3], ck[3];
  tensor_strides(nullptr, H, Sq, D, cq);
  tensor_strides(nullptr, HKV, Sk, D, ck);
  const bool same_q = std::equal(qs, qs + 3, cq) && std::equal(os, os + 3, cq);
  const bool same_kv = std::equal(ks, ks + 3, ck) && std::equal(vs, vs + 3, ck);
  // Head dims below their kernel's tile dim run the padded form (any
  // strides); block masks take D = 64, 128 or 256.
  const int DT = fa::tile_dim(D, dtype);
  if (bm && D != 64 && D != 128 && D != 256) return FA_ERR_HEAD_DIM;
  const int form = DT != D ? fa::kFormPadded
                   : bm    ? fa::kFormBlockSparse
                   : (same_q && same_kv) ? fa::kFormContiguous : fa::kFormStrided;

  DeviceState* ds = nullptr;
  st = device_state(&ds);
  if (st != FA_OK) return st;
  void* fixed_ptr = nullptr;
  if (fixed && (st = fixed->address(&fixed_ptr)) != FA_OK) return st;

  const int BM = fa::block_m(dtype, D);
  int ns = 1, split_len = 0, nslot = 0;
  // A fixed workspace: no persistent schedule (its device table would be
  // allocated), and the split count must fit the workspace.
  plan(*ds, num_splits, B, H, Sq, Sk, DT, causal, window, dtype, form, &ns, &split_len, &nslot,
       fixed == nullptr);
  if (fixed && ns > 1 && split_workspace_bytes(ns, B, H, Sq, DT) > fixed->bytes) {
    if (num_splits != 0) return FA_ERR_WORKSPACE;   // the caller's count does not fit
    // automatic count: the largest that fits (1 needs no workspace)
    int want = ns - 1;
    while (want > 1 && split_workspace_bytes(want, B, H, Sq, DT) > fixed->bytes) --want;
    for (;; --want) {
      resolve_splits(want, B, H, Sq, Sk, DT, causal, window, dtype, ds->num_cus, &ns, &split_len);
      if (ns == 1 || split_workspace_bytes(ns, B, H, Sq, DT) <= fixed->bytes) break;
    }
  }
  if (split_len / fa::key_tile(dtype, DT) > fa::kMaxListTiles && form == fa::kFormBlockSparse)
    return FA_ERR_SHAPE;   // more key tiles than FA_MAX_SPLITS lists can hold

  fa::Params p = {};
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.LSE = LSE;
  p.B = B;
  p.H = H;
  p.HKV = HKV;
  p.Sq = Sq;
  p.Sk = Sk;
  p.dv = D;
  p.group = H / HKV;
  p.sl = (float)((double)scale * 1.4426950408889634);
  if (dtype != FA_F32) {
    // The 16-bit kernel needs a positive multiplier: q.k * scale = (-q).k * |scale|
    // exactly, and for scale = 0 a multiplier of 1e-30 leaves every exp2
    // argument within 1e-20 of 0, where exp2 rounds to exactly 1.
    p.neg_q = scale < 0.f ? 1 : 0;
    const double mag = std::fabs((double)scale) * 1.4426950408889634;
    p.sl = mag > 0.0 ? (float)mag : 1e-30f;
  }
  p.causal = causal;
  p.window = window;
  p.nsplit = ns;
  p.split_len = split_len;
  // 16-bit kernel: the query heads sharing a kv head go into one workgroup
  // (four, or two), each wavefront taking 32 rows of one head, so every
  // wavefront of a workgroup sees the same key range (causal diagonal and
  // window edges fall on fewer key tiles). Block masks keep one head and
  // 128 rows per workgroup (the mask's row blocks).
  const int group = H / HKV;
  p.hp = (dtype == FA_F32 || form == fa::kFormBlockSparse) ? 1
         : group % 4 == 0                                 ? 4
         : group % 2 == 0                                 ? 2
                                                          : 1;
  p.packs = group / p.hp;
  p.bm = BM / p.hp;
  p.n_qblk = (Sq + p.bm - 1) / p.bm;
  const long units = (long)B * HKV * p.packs * ns;
  const long blocks = units * p.n_qblk;
  if (blocks < 1 || blocks > 2147483647L) return FA_ERR_SHAPE;
  p.units = (int)units;
  // Sliding windows over G < 8 kv units (G dividing 8) whose query tiles
  // split into whole snake periods across the R = 8 / G XCDs of a kv unit:
  // the chunked order of map_tile; otherwise query tile major when the units
  // split evenly over the 8 XCDs.
  const int kv_units = p.units / p.packs;
  const bool chunked = window > 0 && kv_units < 8 && 8 % kv_units == 0 &&
                       p.n_qblk % (fa::kXcdChunk * 2 * (8 / kv_units)) == 0;
  p.xcd_remap = chunked ? 2 : (p.units % 8 == 0) ? 1 : 0;
  std::copy(qs, qs + 3, p.qs);
  std::copy(ks, ks + 3, p.ks);
  std::copy(vs, vs + 3, p.vs);
  std::copy(os, os + 3, p.os);
  if (bm) {
    const long long nqb = p.n_qblk, nkb = (Sk + fa::kMaskBlockK - 1) / fa::kMaskBlockK;
    p.bmask = bm->mask;
    p.bm_nkb = (int)nkb;
    p.bm_sh = bm->heads == 1 ? 0 : nqb * nkb;
    p.bm_sb = bm->batch == 1 ? 0 : (long long)bm->heads * nqb * nkb;
    p.bm_by_kv = (bm->heads == HKV && HKV != H) ? 1 : 0;
  }
  if (nslot > 0) {
    st = schedule_for(*ds, B, H, HKV, Sq, Sk, DT, causal, window, dtype, ns, split_len, nslot,
                      &p.sched);
    if (st != FA_OK) return st;
    p.nslot = nslot;
  }

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  void* ws = nullptr;
  if (ns > 1 && fixed) {
    const size_t o_bytes = (size_t)ns * B * H * Sq * DT * sizeof(float);
    p.Opart = static_cast<float*>(fixed_ptr);
    p.Lpart = reinterpret_cast<float*>(static_cast<char*>(fixed_ptr) + o_bytes);
  } else if (ns > 1) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
    hipMemPool_t pool = nullptr;
    st = workspace_pool(dev, *ds, &pool);
    if (st != FA_OK) return st;
    const size_t rows = (size_t)B * H * Sq;
    const size_t o_bytes = (size_t)ns * rows * DT * sizeof(float);
    if (hipMallocFromPoolAsync(&ws, split_workspace_bytes(ns, B, H, Sq, DT), pool, stream) !=
        hipSuccess)
      return FA_ERR_WORKSPACE;
    p.Opart = static_cast<float*>(ws);
    p.Lpart = reinterpret_cast<float*>(static_cast<char*>(ws) + o_bytes);
  }
  const hipError_t e = fa::launch_forward(p, dtype, DT, form, stream);
  const hipError_t f = ws ? hipFreeAsync(ws, stream) : hipSuccess;
  return (e == hipSuccess && f == hipSuccess) ? FA_OK : FA_ERR_HIP;
}

}  // namespace

namespace fa {
int device_cus() {
  DeviceState* ds = nullptr;
  return device_state(&ds) == FA_OK ? ds->num_cus : 0;
}

int forward_fixed_workspace(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int B, int H, int HKV, int Sq, int Sk, int D, float scale,
                            int causal, int window, int dtype, int num_splits, void* stream,
                            const FixedWorkspace& ws) {
  return forward(Q, K, V, O, LSE, B, H, HKV, Sq, Sk, D, nullptr, nullptr, nullptr, nullptr, scale,
                 causal, window, dtype, num_splits, stream, nullptr, &ws);
}

// Stream-ordered workspace from this library's pool on the current device
// (the pool of the split workspace; freed blocks stay cached until fa_release).
int library_workspace(size_t bytes, hipStream_t stream, void** out) {
  DeviceState* ds = nullptr;
  int st = device_state(&ds);
  if (st != FA_OK) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  hipMemPool_t pool = nullptr;
  st = workspace_pool(dev, *ds, &pool);
  if (st != FA_OK) return st;
  return hipMallocFromPoolAsync(out, bytes, pool, stream) == hipSuccess ? FA_OK : FA_ERR_WORKSPACE;
}
}  // namespace fa

extern "C" {

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
           int HKV, int Sq, int Sk, int D, float scale, int causal, int window, int dtype,
           void* stream) {
  return forward(Q, K, V, O, LSE, B, H, HKV, Sq, Sk, D, nullptr, nullptr, nullptr, nullptr, scale,
                 causal, window, dtype, 0, stream);
}

int fa_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
              int HKV, int Sq, int Sk, int D, float scale, int causal, int window, int dtype,
              int num_splits, void* stream) {
  return forward(Q, K, V, O, LSE, B, H, HKV, Sq, Sk, D, nullptr, nullptr, nullptr, nullptr, scale,
                 causal, window, dtype, num_splits, stream);
}

int fa_fwd_strided(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                   int H, int HKV, int Sq, int Sk, int D, const long long* q_strides,
                   const long long* k_strides, const long long* v_strides,
                   const long long* o_strides, float scale, int causal, int window, int dtype,
                   int num_splits, void* stream) {
  return forward(Q, K, V, O, LSE, B, H, HKV, Sq, Sk, D, q_strides, k_strides, v_strides,
                 o_strides, scale, causal, window, dtype, num_splits, stream);
}

int fa_fwd_block_sparse(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                        int H, int HKV, int Sq, int Sk, int D, const unsigned char* block_mask,
                        int mask_batch, int mask_heads, float scale, int causal, int window,
                        int dtype, int num_splits, void* stream) {
  const MaskArg bm = {block_mask, mask_batch, mask_heads};
  return forward(Q, K, V, O, LSE, B, H, HKV, Sq, Sk, D, nullptr, nullptr, nullptr, nullptr, scale,
                 causal, window, dtype, num_splits, stream, &bm);
}

int fa_plan_splits(int B, int H, int HKV, int Sq, int Sk, int D, int causal, int window,
                   int dtype) {
  int st = check_args(B, H, HKV, Sq, Sk, D, causal, window, dtype);
  if (st != FA_OK) return -st;
  DeviceState* ds = nullptr;
  st = device_state(&ds);
  if (st != FA_OK) return -st;
  int ns = 1, split_len = 0, nslot = 0;
  const int DT = fa::tile_dim(D, dtype);
  plan(*ds, 0, B, H, Sq, Sk, DT, causal, window, dtype,
       DT != D ? fa::kFormPadded : fa::kFormContiguous, &ns, &split_len, &nslot);
  return ns;
}

int fa_schedule_table(int B, int H, int HKV, int Sq, int Sk, int D, int causal, int window,
                      int dtype, int nslot, int* table, int capacity, int* num_splits) {
  const int st = check_args(B, H, HKV, Sq, Sk, D, causal, window, dtype);
  if (st != FA_OK) return -st;
  if (nslot < 1 || capacity < 0 || (capacity > 0 && !table)) return -FA_ERR_SHAPE;
  const int BM = fa::block_m(dtype, D);
  const long items = (long)B * H * FA_MAX_SPLITS * ((Sq + BM - 1) / BM);
  if (items + nslot + 1 > 2147483647L) return -FA_ERR_SHAPE;
  int ns = 1, split_len = 0;
  const int DT = fa::tile_dim(D, dtype);
  resolve_splits(persistent_splits(B, H, Sq, Sk, DT, causal, window, dtype, nslot), B, H, Sq, Sk,
                 DT, causal, window, dtype, 1, &ns, &split_len);
  const std::vector<int> t =
      build_schedule(B, H, HKV, Sq, Sk, DT, causal, window, dtype, ns, split_len, nslot);
  if (num_splits) *num_splits = ns;
  for (int i = 0; i < (int)t.size() && i < capacity; ++i) table[i] = t[i];
  return (int)t.size();
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULLPTR: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape: a dimension is < 1 or the problem is too large";
    case FA_ERR_GQA: return "H must be a multiple of HKV";
    case FA_ERR_HEAD_DIM: return "head dimension D must be 16, 32, 48, 64, 80, 96, 128 or 256 (block masks: 64, 128 or 256)";
    case FA_ERR_DTYPE: return "dtype must be FA_F32 (0), FA_BF16 (1) or FA_F16 (2)";
    case FA_ERR_WINDOW: return "window must be >= 0 and causal 0 or 1";
    case FA_ERR_ALIGN: return "every buffer must be 16-byte aligned";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_WORKSPACE: return "could not allocate the split-K workspace";
    case FA_ERR_SPLITS: return "num_splits must be in [0, FA_MAX_SPLITS]";
    case FA_ERR_MASK: return "block mask: batch axis must be 1 or B, head axis 1, HKV or H";
    case FA_ERR_STRIDE: return "invalid strides: negative, not 16-byte multiples, rows overlapping, or a K/V row stride that is not a multiple of D";
    default: return "unknown status";
  }
}

void fa_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  int cur = -1;
  (void)hipGetDevice(&cur);
  for (int d = 0; d < kMaxDevices; ++d) {
    DeviceState& s = g_dev[d];
    if (s.pool) (void)hipMemPoolTrimTo(s.pool, 0);   // nothing to report
    if (!s.scheds.empty() && hipSetDevice(d) == hipSuccess) {
      // schedules may still be read by queued kernels: wait for the device first
      (void)hipDeviceSynchronize();
      for (auto& kv : s.scheds) (void)hipFree(kv.second.dev);
      s.scheds.clear();
    }
  }
  if (cur >= 0) (void)hipSetDevice(cur);
}

}  // extern "C"

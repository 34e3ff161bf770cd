// C ABI of the fused attention forward pass: argument checks, key-split
// planning, the split workspace, and the launch. Declared in include/fa.h.
#include "fa.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "fa_kernels.h"

namespace {

constexpr int kMaxDevices = 64;

struct DeviceState {
  bool init = false;
  int num_cus = 0;
  hipMemPool_t pool = nullptr;
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
  if (dtype != FA_F32 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (D != 64 && D != 128 && D != 256) return FA_ERR_HEAD_DIM;
  if (H % HKV != 0) return FA_ERR_GQA;
  if (window < 0 || (causal != 0 && causal != 1)) return FA_ERR_WINDOW;
  const int esz = dtype == FA_BF16 ? 2 : 4;
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

int forward(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
            int HKV, int Sq, int Sk, int D, float scale, int causal, int window, int dtype,
            int num_splits, void* stream_ptr) {
  if (!Q || !K || !V || !O || !LSE) return FA_ERR_NULLPTR;
  int st = check_args(B, H, HKV, Sq, Sk, D, causal, window, dtype);
  if (st != FA_OK) return st;
  if (num_splits < 0 || num_splits > FA_MAX_SPLITS) return FA_ERR_SPLITS;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return FA_ERR_ALIGN;

  DeviceState* ds = nullptr;
  st = device_state(&ds);
  if (st != FA_OK) return st;

  const int BM = fa::block_m(dtype, D);
  int ns = 1, split_len = 0;
  resolve_splits(num_splits, B, H, Sq, Sk, D, causal, window, dtype, ds->num_cus, &ns,
                 &split_len);

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
  p.group = H / HKV;
  p.sl = (float)((double)scale * 1.4426950408889634);
  if (dtype == FA_BF16) {
    // The bf16 kernel needs a positive multiplier: q.k * scale = (-q).k * |scale|
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
  p.n_qblk = (Sq + BM - 1) / BM;
  const long units = (long)B * H * ns;
  const long blocks = units * p.n_qblk;
  if (blocks < 1 || blocks > 2147483647L) return FA_ERR_SHAPE;
  p.units = (int)units;
  p.xcd_remap = (p.units % 8 == 0) ? 1 : 0;

  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_ptr);
  void* ws = nullptr;
  if (ns > 1) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
    hipMemPool_t pool = nullptr;
    st = workspace_pool(dev, *ds, &pool);
    if (st != FA_OK) return st;
    const size_t rows = (size_t)B * H * Sq;
    const size_t o_bytes = (size_t)ns * rows * D * sizeof(float);
    const size_t l_bytes = (size_t)ns * rows * sizeof(float);
    if (hipMallocFromPoolAsync(&ws, o_bytes + l_bytes, pool, stream) != hipSuccess)
      return FA_ERR_WORKSPACE;
    p.Opart = static_cast<float*>(ws);
    p.Lpart = reinterpret_cast<float*>(static_cast<char*>(ws) + o_bytes);
  }
  const hipError_t e = fa::launch_forward(p, dtype, D, stream);
  const hipError_t f = ws ? hipFreeAsync(ws, stream) : hipSuccess;
  return (e == hipSuccess && f == hipSuccess) ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
           int HKV, int Sq, int Sk, int D, float scale, int causal, int window, int dtype,
           void* stream) {
  return forward(Q, K, V, O, LSE, B, H, HKV, Sq, Sk, D, scale, causal, window, dtype, 0, stream);
}

int fa_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
              int HKV, int Sq, int Sk, int D, float scale, int causal, int window, int dtype,
              int num_splits, void* stream) {
  return forward(Q, K, V, O, LSE, B, H, HKV, Sq, Sk, D, scale, causal, window, dtype,
                 num_splits, stream);
}

int fa_plan_splits(int B, int H, int HKV, int Sq, int Sk, int D, int causal, int window,
                   int dtype) {
  int st = check_args(B, H, HKV, Sq, Sk, D, causal, window, dtype);
  if (st != FA_OK) return -st;
  DeviceState* ds = nullptr;
  st = device_state(&ds);
  if (st != FA_OK) return -st;
  int ns = 1, split_len = 0;
  resolve_splits(0, B, H, Sq, Sk, D, causal, window, dtype, ds->num_cus, &ns, &split_len);
  return ns;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_NULLPTR: return "a required pointer is NULL";
    case FA_ERR_SHAPE: return "invalid shape: a dimension is < 1 or the problem is too large";
    case FA_ERR_GQA: return "H must be a multiple of HKV";
    case FA_ERR_HEAD_DIM: return "head dimension D must be 64, 128 or 256";
    case FA_ERR_DTYPE: return "dtype must be FA_F32 (0) or FA_BF16 (1)";
    case FA_ERR_WINDOW: return "window must be >= 0 and causal 0 or 1";
    case FA_ERR_ALIGN: return "every buffer must be 16-byte aligned";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_WORKSPACE: return "could not allocate the split-K workspace";
    case FA_ERR_SPLITS: return "num_splits must be in [0, FA_MAX_SPLITS]";
    default: return "unknown status";
  }
}

void fa_release(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (int d = 0; d < kMaxDevices; ++d) {
    if (g_dev[d].pool) (void)hipMemPoolTrimTo(g_dev[d].pool, 0);   // nothing to report
  }
}

}  // extern "C"

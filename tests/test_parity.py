"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.

Tolerances: max |dO| and max |dLSE| <= 1e-4 for float32 inputs, <= 2e-2 for
bfloat16 inputs and <= 5e-3 for float16 inputs (absolute, over every checked
element, GPU output upcast to fp64). Rows with no visible key must be exactly
O = 0 and LSE = -inf. The float16 bound follows from the arithmetic: P is
rounded to float16 for the PV product (relative error <= 2^-11 per weight, so
|dO| <= 2^-11 max|V|) and O is rounded once more on output (<= 2^-11 |O| <=
2^-11 max|V|); with |V| <= 2.5 in these inputs that is <= 2.5e-3, and the
float32 accumulation adds orders of magnitude less.

Small cases are compared element by element on every row and span several
query and key tiles with ragged tails. The benchmark workloads run at full
size in the launch configuration the benchmark times: the tiny, fp32 causal
and bf16 causal GQA workloads (and the variants of the last one: fp16,
token-major, block mask, head dim 96) on every row; the sliding-window and
long-key workloads, whose full oracle would take minutes, on seeded row
samples (random rows plus the first and last 64 rows of every head for the
window workload)."""
import sys

import numpy as np
import pytest

import workloads as W
from oracle import attention, attention_rows, visible_count

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 5e-3}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(inp):
    import attention_forward_online_fa_amd  # noqa: F401  (fails loudly if the library is missing)
    return W.device_tensors(inp, torch, "cuda")


def run_gpu(inp, num_splits=0, scale=None):
    import attention_forward_online_fa_amd as fa
    wl = inp.wl
    q, k, v = to_device(inp)
    o, lse = fa.fwd(q, k, v, causal=bool(wl.causal), window=wl.window,
                    scale=wl.scale() if scale is None else scale, num_splits=num_splits,
                    block_mask=W.device_mask(inp, torch, "cuda"))
    torch.cuda.synchronize()
    return o, lse


def host64(t):
    return t.float().cpu().numpy().astype(np.float64)


def compare(o_gpu, l_gpu, o_ref, l_ref, tol, what):
    empty = np.isneginf(l_ref)
    assert np.all(np.isneginf(l_gpu[empty])), f"{what}: empty rows must have LSE = -inf"
    assert np.all(o_gpu[empty] == 0.0), f"{what}: empty rows must have O = 0"
    assert np.all(np.isfinite(l_gpu[~empty])), f"{what}: non-finite LSE on a non-empty row"
    assert np.all(np.isfinite(o_gpu)), f"{what}: non-finite O"
    dO = float(np.max(np.abs(o_gpu[~empty] - o_ref[~empty]))) if (~empty).any() else 0.0
    dL = float(np.max(np.abs(l_gpu[~empty] - l_ref[~empty]))) if (~empty).any() else 0.0
    _say(f"  {what}: max|dO|={dO:.3e} max|dLSE|={dL:.3e} (tol {tol:g})")
    assert dO <= tol and dL <= tol, f"{what}: max|dO|={dO:.3e} max|dLSE|={dL:.3e} > {tol}"


def check_full(wl, num_splits=0, scale=None, inp=None):
    inp = inp or W.make_inputs(wl)
    _say(f"[parity] {wl} splits={num_splits}")
    s = wl.scale() if scale is None else scale
    o, lse = run_gpu(inp, num_splits, s)
    O, L = attention(inp.q, inp.k, inp.v, s, bool(wl.causal), wl.window,
                     block_mask=inp.block_mask)
    compare(host64(o), host64(lse), O, L, TOL[wl.dtype], wl.name)
    return o, lse


def wl_small(dtype, B, H, HKV, Sq, Sk, D, causal, window, name="small", seed=0):
    return W.Workload(name, B, H, HKV, Sq, Sk, D, dtype, causal, window,
                      amplitude=0.5 if dtype != "f32" else 1.0, seed_index=100 + seed)


SMALL = [
    # dtype, B, H, HKV, Sq, Sk, D, causal, window
    ("f32", 1, 1, 1, 128, 128, 64, 0, 0),
    ("f32", 2, 4, 2, 300, 300, 64, 1, 0),       # ragged, causal, GQA
    ("f32", 1, 4, 1, 257, 190, 128, 1, 0),      # Sq > Sk, top-left causal
    ("f32", 1, 2, 2, 200, 333, 128, 0, 77),     # window without causal, ragged
    ("f32", 1, 4, 2, 384, 384, 128, 1, 100),    # sliding window GQA
    ("f32", 1, 2, 1, 150, 170, 256, 1, 0),
    ("bf16", 1, 1, 1, 128, 128, 64, 0, 0),
    ("bf16", 2, 4, 2, 300, 300, 64, 1, 0),
    ("bf16", 1, 8, 2, 257, 190, 128, 1, 0),
    ("bf16", 1, 4, 4, 200, 333, 128, 0, 77),
    ("bf16", 1, 4, 1, 384, 500, 128, 1, 100),
    ("bf16", 1, 2, 1, 150, 170, 256, 1, 0),
    ("bf16", 1, 1, 1, 96, 1000, 256, 0, 0),
    # long enough for the interior-tile path, entered after window-edge tiles
    # and left before a partial last tile
    ("bf16", 1, 2, 1, 1024, 1024, 128, 1, 300),
    ("bf16", 1, 2, 2, 512, 1000, 64, 0, 0),
    ("bf16", 1, 2, 1, 640, 2100, 256, 0, 0),
    # 32-key tiles at D = 128: long causal interior run (odd tile count per pair
    # loop), non-causal with a partial last tile, one-sided window with ragged ends
    ("bf16", 1, 4, 1, 1536, 1536, 128, 1, 0),
    ("bf16", 1, 2, 2, 256, 1500, 128, 0, 0),
    ("bf16", 2, 2, 1, 333, 1111, 128, 0, 500),
    # sliding windows over 4 kv units: the chunked XCD order of the work
    # mapping (query-tile chunks dealt in snake order over two XCDs per kv unit)
    ("bf16", 1, 8, 4, 2048, 2048, 128, 1, 300),
    ("f32", 1, 4, 4, 4096, 4096, 64, 1, 500),
    # float16 inputs (same kernel as bfloat16, fp16 MFMA and fp16 P)
    ("f16", 1, 1, 1, 128, 128, 64, 0, 0),
    ("f16", 2, 4, 2, 300, 300, 64, 1, 0),
    ("f16", 1, 8, 2, 257, 190, 128, 1, 0),
    ("f16", 1, 4, 1, 384, 500, 128, 1, 100),
    ("f16", 1, 4, 1, 1536, 1536, 128, 1, 0),
    ("f16", 2, 2, 1, 333, 1111, 128, 0, 500),
    ("f16", 1, 2, 1, 150, 170, 256, 1, 0),
    ("f16", 1, 2, 1, 640, 2100, 256, 0, 0),
]


@pytest.mark.parametrize("case", SMALL, ids=["-".join(map(str, c)) for c in SMALL])
def test_small_full(case):
    check_full(wl_small(*case, seed=sum(case[1:])))


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 128), ("bf16", 128), ("bf16", 256),
                                     ("f16", 64), ("f16", 256)])
@pytest.mark.parametrize("splits", [2, 3, 7])
def test_forced_key_splits(dtype, D, splits):
    wl = wl_small(dtype, 1, 2, 1, 200, 700, D, 0, 0, seed=splits + D)
    check_full(wl, num_splits=splits)
    wl = wl_small(dtype, 1, 2, 2, 260, 700, D, 1, 150, seed=splits + D + 1)
    check_full(wl, num_splits=splits)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_empty_rows_exact(dtype):
    # Sq=8, Sk=2, causal, window=1: rows i >= 2 see no key.
    wl = wl_small(dtype, 1, 2, 1, 8, 2, 64, 1, 1, seed=5)
    o, lse = check_full(wl)
    o, lse = host64(o), host64(lse)
    assert np.all(o[:, :, 2:] == 0) and np.all(np.isneginf(lse[:, :, 2:]))
    # and with key splits (every split of those rows is empty too)
    wl = wl_small(dtype, 1, 2, 1, 300, 130, 128, 1, 5, seed=6)
    check_full(wl, num_splits=3)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1, 64, 0, 0), (1, 2, 2, 5, 1, 128, 1, 0),
                                   (1, 2, 1, 129, 129, 128, 1, 1), (1, 2, 1, 200, 150, 64, 1, 1000)])
def test_degenerate_shapes(dtype, shape):
    check_full(wl_small(dtype, *shape, seed=sum(shape)))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_gqa_equals_mha_with_repeated_kv(dtype):
    import attention_forward_online_fa_amd as fa
    wl = wl_small(dtype, 2, 8, 2, 256, 256, 128, 1, 0, seed=7)
    q, k, v = to_device(W.make_inputs(wl))
    o1, l1 = fa.fwd(q, k, v, causal=True)
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    o2, l2 = fa.fwd(q, kr, vr, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_deterministic(dtype):
    import attention_forward_online_fa_amd as fa
    wl = wl_small(dtype, 1, 4, 2, 512, 512, 128, 1, 0, seed=8)
    q, k, v = to_device(W.make_inputs(wl))
    a = fa.fwd(q, k, v, causal=True)
    b = fa.fwd(q, k, v, causal=True)
    c = fa.fwd(q, k, v, causal=True, num_splits=3)
    d = fa.fwd(q, k, v, causal=True, num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(c[0], d[0]) and torch.equal(c[1], d[1])


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 64), ("bf16", 128), ("bf16", 256),
                                     ("f16", 128)])
@pytest.mark.parametrize("scale", [0.37, -0.2, 0.0])
def test_scale_passed_through(dtype, D, scale):
    # negative scale flips the softmax; zero scale gives the mean of the visible V
    wl = wl_small(dtype, 1, 2, 1, 130, 150, D, 1, 0, seed=9)
    check_full(wl, scale=scale)


def rising_inputs(wl, rise):
    """Inputs whose scores climb by about `rise` (natural-log units) per key:
    every key tile raises each row's maximum, so the softmax's running
    reference goes stale on every tile and must be rescaled (for float16 the
    exponentials against the stale reference would overflow the type)."""
    rng = np.random.default_rng(wl.seed)
    q = (0.1 * rng.standard_normal((wl.B, wl.H, wl.Sq, wl.D))).astype(np.float32)
    k = (0.1 * rng.standard_normal((wl.B, wl.HKV, wl.Sk, wl.D))).astype(np.float32)
    v = (0.5 * rng.standard_normal((wl.B, wl.HKV, wl.Sk, wl.D))).astype(np.float32)
    q[..., 0] = 1.0
    k[..., 0] = (rise / wl.scale()) * np.arange(wl.Sk, dtype=np.float32)
    inp = W.Inputs(wl, q, k, v)
    if wl.dtype in W.ROUNDING:
        to_bits, to_f32 = W.ROUNDING[wl.dtype]
        inp.q_bits, inp.k_bits, inp.v_bits = to_bits(q), to_bits(k), to_bits(v)
        inp.q, inp.k, inp.v = to_f32(inp.q_bits), to_f32(inp.k_bits), to_f32(inp.v_bits)
    return inp


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128), ("bf16", 256), ("f16", 64),
                                     ("f16", 128), ("f16", 256)])
@pytest.mark.parametrize("splits", [1, 3])
def test_rising_scores_rescale_every_tile(dtype, D, splits):
    # ~0.4 per key: a 32-key tile raises the maximum by ~13 (2^18 in base 2)
    # (scores reach ~120, where a float32 ulp of the LSE is ~1e-5)
    wl = wl_small(dtype, 1, 2, 1, 160, 300, D, 0, 0, seed=11 + D)
    check_full(wl, num_splits=splits, inp=rising_inputs(wl, 0.4))
    wl = wl_small(dtype, 1, 2, 2, 300, 300, D, 1, 0, seed=12 + D)
    check_full(wl, num_splits=splits, inp=rising_inputs(wl, 0.4))


# ------------------------------------------------------- benchmark workloads
@pytest.mark.parametrize("idx", range(len(W.CONFIGS)), ids=[c.name for c in W.CONFIGS])
def test_benchmark_workload(idx):
    wl = W.CONFIGS[idx]
    _say(f"[parity] workload {idx}: {wl.name}")
    inp = W.make_inputs(wl)
    o, lse = run_gpu(inp)          # fa_fwd's own split choice, as the benchmark runs it
    rows = W.check_rows(inp)
    s = wl.scale()
    if rows is None:
        # every row of every (batch, head) against the oracle
        O, L = attention(inp.q, inp.k, inp.v, s, bool(wl.causal), wl.window,
                         block_mask=inp.block_mask)
        compare(host64(o), host64(lse), O, L, TOL[wl.dtype],
                f"{wl.name} (all {wl.B * wl.H * wl.Sq} rows)")
        return
    idx_t = torch.from_numpy(rows).cuda()
    og = o[idx_t[:, 0], idx_t[:, 1], idx_t[:, 2]]
    lg = lse[idx_t[:, 0], idx_t[:, 1], idx_t[:, 2]]
    O, L = attention_rows(inp.q, inp.k, inp.v, s, bool(wl.causal), wl.window, rows,
                          block_mask=inp.block_mask)
    compare(host64(og), host64(lg), O, L, TOL[wl.dtype], f"{wl.name} ({len(rows)} rows)")
    # properties over every row: finite outputs, LSE >= max score lower bound
    # (LSE >= log of one term) is not cheap here; check finiteness everywhere.
    lh = host64(lse)
    if inp.block_mask is None:
        cnt = visible_count(wl.Sq, wl.Sk, bool(wl.causal), wl.window)
        assert np.all(np.isfinite(lh[:, :, cnt > 0]))
    else:   # every row of these masks sees its own diagonal block and key block 0
        assert np.all(np.isfinite(lh))
    assert torch.isfinite(o.float()).all().item()


def test_fp32_causal_small_grid_runs_persistent_pieces():
    # the fp32 causal MHA workload has 256 query tiles (fewer than two per CU):
    # it runs as persistent workgroups over key-split pieces and a merge
    import attention_forward_online_fa_amd as fa
    wl = W.CONFIGS[1]
    ns = fa.plan_splits(wl.B, wl.H, wl.HKV, wl.Sq, wl.Sk, wl.D, causal=bool(wl.causal),
                        window=wl.window, dtype=wl.dtype)
    assert ns > 1
    # every piece list, and the result against the oracle on a smaller grid of
    # the same kind (all rows), with two calls in a row using the cached list
    small = wl_small("f32", 2, 4, 4, 640, 640, 64, 1, 0, seed=77)
    assert fa.plan_splits(2, 4, 4, 640, 640, 64, causal=True, dtype="f32") > 1
    check_full(small)
    check_full(small)


# ------------------------------------------------------- very long key axis
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("splits", [0, 64])
def test_very_long_key_axis(dtype, splits):
    # one query tile over a million keys (ragged): the key axis is split into
    # up to FA_MAX_SPLITS pieces of ~16k keys each and merged; every row checked
    import attention_forward_online_fa_amd as fa
    wl = wl_small(dtype, 1, 1, 1, 64, 1_000_003, 64, 0, 0, name="longkeys", seed=77)
    inp = W.make_inputs(wl)
    _say(f"[parity] {wl} splits={splits}")
    q, k, v = to_device(inp)
    o, lse = fa.fwd(q, k, v, scale=wl.scale(), num_splits=splits)
    torch.cuda.synchronize()
    if splits == 0:
        assert fa.plan_splits(1, 1, 1, 64, wl.Sk, 64, dtype=dtype) == 64
    rows = np.array([(0, 0, i) for i in range(wl.Sq)])
    O, L = attention_rows(inp.q, inp.k, inp.v, wl.scale(), False, 0, rows)
    compare(host64(o)[0, 0], host64(lse)[0, 0], O, L, TOL[wl.dtype], wl.name)


# ------------------------------------------------- fa_fwd called directly
def _fa_fwd_direct(inp):
    """o, lse from lib().fa_fwd itself (the entry point with the benchmark's
    16-argument signature), on torch-allocated device buffers."""
    from attention_forward_online_fa_amd import _lib
    wl = inp.wl
    q, k, v = to_device(inp)
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.Sq), dtype=torch.float32, device=q.device)
    code = {"f32": _lib.FA_F32, "bf16": _lib.FA_BF16, "f16": _lib.FA_F16}[wl.dtype]
    stream = torch.cuda.current_stream()
    st = _lib.lib().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           wl.B, wl.H, wl.HKV, wl.Sq, wl.Sk, wl.D, wl.scale(), wl.causal,
                           wl.window, code, stream.cuda_stream)
    assert st == 0, _lib.STATUS.get(st, st)
    torch.cuda.synchronize()
    return o, lse


DIRECT = [W.CONFIGS[0], W.CONFIGS[1],
          W.Workload("direct_gqa_causal_bf16", 1, 8, 2, 700, 700, 128, "bf16", 1, 0,
                     amplitude=0.5, seed_index=60)]


@pytest.mark.parametrize("wl", DIRECT, ids=[w.name for w in DIRECT])
def test_fa_fwd_entry_point_direct(wl):
    inp = W.make_inputs(wl)
    _say(f"[parity] fa_fwd direct: {wl}")
    o, lse = _fa_fwd_direct(inp)
    O, L = attention(inp.q, inp.k, inp.v, wl.scale(), bool(wl.causal), wl.window)
    compare(host64(o), host64(lse), O, L, TOL[wl.dtype], f"fa_fwd {wl.name}")
    # the same buffers through fa_fwd_ex (automatic splits): identical bits
    o2, l2 = run_gpu(inp)
    assert torch.equal(o, o2) and torch.equal(lse, l2)

"""fa_fwd_noalloc (through the C ABI) against fa_fwd_ex: the same results
from the library's static per-GPU workspace, on two calls in a row (the
second with a smaller input, so it reuses the array the first one wrote), and
against the fp64 oracle at the tolerances of the parity tests. Also: an
explicit split count whose partials do not fit the array is rejected before
any device work, and an automatic count is lowered until they fit."""
import sys

import numpy as np
import pytest

import workloads as W
from oracle import attention, attention_rows

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 5e-3}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _call(fn_name, wl, q, k, v, num_splits):
    from attention_forward_online_fa_amd import _lib
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.Sq), dtype=torch.float32, device=q.device)
    code = {"f32": _lib.FA_F32, "bf16": _lib.FA_BF16, "f16": _lib.FA_F16}[wl.dtype]
    fn = getattr(_lib.lib(), fn_name)
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), wl.B, wl.H,
            wl.HKV, wl.Sq, wl.Sk, wl.D, wl.scale(), wl.causal, wl.window, code, num_splits,
            torch.cuda.current_stream().cuda_stream)
    return st, o, lse


def _rows_check(inp, o, lse, rows=None):
    wl = inp.wl
    if rows is None:
        O, L = attention(inp.q, inp.k, inp.v, wl.scale(), bool(wl.causal), wl.window)
        og, lg = o.float().cpu().numpy(), lse.cpu().numpy()
    else:
        O, L = attention_rows(inp.q, inp.k, inp.v, wl.scale(), bool(wl.causal), wl.window, rows)
        og = o.float().cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
        lg = lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    ne = ~np.isneginf(L)
    assert np.all(np.isneginf(lg[~ne])) and np.all(og[~ne] == 0)
    dO = float(np.abs(og[ne] - O[ne]).max())
    dL = float(np.abs(lg[ne] - L[ne]).max())
    _say(f"  {wl.name}: max|dO|={dO:.3e} max|dLSE|={dL:.3e} (tol {TOL[wl.dtype]:g})")
    assert dO <= TOL[wl.dtype] and dL <= TOL[wl.dtype]


def _pair(wl, num_splits, expect_splits):
    """fa_fwd_noalloc and fa_fwd_ex (with the split count the no-alloc call
    uses) on the same inputs: bit-identical outputs."""
    from attention_forward_online_fa_amd import _lib
    inp = W.make_inputs(wl)
    q, k, v = W.device_tensors(inp, torch, "cuda")
    _say(f"[no-alloc] {wl} num_splits={num_splits}")
    st, o1, l1 = _call("fa_fwd_noalloc", wl, q, k, v, num_splits)
    assert st == 0, _lib.STATUS.get(st, st)
    st, o2, l2 = _call("fa_fwd_ex", wl, q, k, v, expect_splits)
    assert st == 0, _lib.STATUS.get(st, st)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "fa_fwd_noalloc differs from fa_fwd_ex"
    return inp, o1, l1


def test_noalloc_matches_fa_fwd_ex_two_calls_second_smaller():
    import attention_forward_online_fa_amd as fa
    # a long key axis with few query tiles: the automatic count splits it
    big = W.Workload("noalloc_long_bf16", 1, 2, 1, 640, 30000, 128, "bf16", 0, 0,
                     amplitude=0.5, seed_index=70)
    small = W.Workload("noalloc_causal_gqa_bf16", 1, 4, 2, 300, 2500, 128, "bf16", 1, 0,
                       amplitude=0.5, seed_index=71)
    ns_big = fa.plan_splits(big.B, big.H, big.HKV, big.Sq, big.Sk, big.D, dtype="bf16")
    ns_small = fa.plan_splits(small.B, small.H, small.HKV, small.Sq, small.Sk, small.D,
                              causal=True, dtype="bf16")
    assert ns_big > 1 and ns_small > 1
    inp, o, lse = _pair(big, 0, ns_big)
    rng = np.random.default_rng(5)
    rows = np.stack([np.zeros(200, np.int64), rng.integers(0, big.H, 200),
                     rng.integers(0, big.Sq, 200)], axis=1)
    _rows_check(inp, o, lse, rows)
    inp, o, lse = _pair(small, 0, ns_small)
    _rows_check(inp, o, lse)
    # and an explicit count, again smaller, then no split at all
    inp, o, lse = _pair(small, 3, 3)
    _rows_check(inp, o, lse)
    tiny = W.Workload("noalloc_tiny_f32", 1, 2, 1, 100, 90, 64, "f32", 1, 0, seed_index=72)
    inp, o, lse = _pair(tiny, 1, 1)
    _rows_check(inp, o, lse)


def test_noalloc_fp32_causal_small_grid_runs_without_the_persistent_schedule():
    import attention_forward_online_fa_amd as fa
    # fa_fwd_ex runs this shape persistently; fa_fwd_noalloc one workgroup per
    # item with the plain automatic split count. Same results to tolerance.
    wl = W.Workload("noalloc_f32_causal", 2, 4, 4, 640, 640, 64, "f32", 1, 0, seed_index=73)
    assert fa.plan_splits(2, 4, 4, 640, 640, 64, causal=True, dtype="f32") > 1
    inp = W.make_inputs(wl)
    q, k, v = W.device_tensors(inp, torch, "cuda")
    st, o, lse = _call("fa_fwd_noalloc", wl, q, k, v, 0)
    assert st == 0
    torch.cuda.synchronize()
    _rows_check(inp, o, lse)


def test_noalloc_split_count_bounded_by_the_static_array():
    from attention_forward_online_fa_amd import _lib
    import attention_forward_online_fa_amd as fa
    # bf16 D256, 3 heads x 64 query tiles: fa_fwd_ex splits 3 ways, whose
    # partials (3 x 24576 rows x 257 floats = 75.8 MB) exceed the 68 MiB array
    wl = W.Workload("noalloc_lowered_bf16_d256", 1, 3, 1, 8192, 4096, 256, "bf16", 0, 0,
                    amplitude=0.5, seed_index=74)
    assert fa.plan_splits(1, 3, 1, 8192, 4096, 256, dtype="bf16") == 3
    need = 3 * 3 * 8192 * (256 + 1) * 4
    assert need > _lib.FA_NOALLOC_SCRATCH_BYTES
    inp = W.make_inputs(wl)
    q, k, v = W.device_tensors(inp, torch, "cuda")
    # an explicit count that does not fit: rejected before any device work
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 3, 8192), 7.0, dtype=torch.float32, device=q.device)
    st = _lib.lib().fa_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), 1, 3, 1, 8192, 4096, 256, wl.scale(), 0, 0,
                                   _lib.FA_BF16, 3, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert _lib.STATUS[st] == "FA_ERR_WORKSPACE"
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
    # the automatic count is lowered to 2, which fits: identical to fa_fwd_ex at 2
    inp, o, lse = _pair(wl, 0, 2)
    rng = np.random.default_rng(6)
    rows = np.stack([np.zeros(128, np.int64), rng.integers(0, 3, 128),
                     rng.integers(0, 8192, 128)], axis=1)
    _rows_check(inp, o, lse, rows)

"""GPU parity over seeded random configurations of every forward entry point
(contiguous, strided and block-sparse, with forced or automatic key splits)
and of every backward entry point (the same three forms), against the fp64
oracle.

Each case draws dtype, head dim (any supported one), batch, heads and GQA group, query and key
lengths (ragged, Sq != Sk), causal and window flags, the split count, the
layout (contiguous or token-major) and, for block-sparse cases, a random mask
with a random axis form. Shapes stay small enough for the oracle to check
every row. Tolerances as in test_parity.py (forward) and test_backward.py
(backward)."""
import os

import numpy as np
import pytest

import workloads as W
from oracle import attention, attention_backward
from test_parity import TOL, compare, host64, to_device, wl_small

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BWD_TOL = {"f32": 1e-5, "bf16": 1e-2, "f16": 2e-3}   # the bounds of test_backward.py


def draw(seed):
    r = np.random.default_rng(seed)
    dtype = ["f32", "bf16", "f16"][r.integers(3)]
    D = [16, 32, 48, 64, 80, 96, 128, 256][r.integers(8)]
    HKV = int(r.integers(1, 3))
    H = HKV * int(r.choice([1, 2, 4]))
    B = int(r.integers(1, 3))
    Sq = int(r.integers(1, 400))
    Sk = int(r.integers(1, 600))
    causal = int(r.integers(2))
    window = int(r.choice([0, 0, int(r.integers(1, 300))]))
    splits = int(r.choice([0, 0, 1, 2, 3, 5]))
    kind = ["dense", "strided", "sparse"][r.integers(3)]
    if kind == "sparse" and D not in (64, 128, 256):   # block masks take these head dims
        kind = "dense"
    return dict(dtype=dtype, D=D, B=B, H=H, HKV=HKV, Sq=Sq, Sk=Sk, causal=causal,
                window=window, splits=splits, kind=kind, rng=r)


@pytest.mark.parametrize("seed", range(64))
def test_random_forward(seed):
    import attention_forward_online_fa_amd as fa
    c = draw(1000 + seed)
    wl = wl_small(c["dtype"], c["B"], c["H"], c["HKV"], c["Sq"], c["Sk"], c["D"], c["causal"],
                  c["window"], name=f"rand{seed}", seed=200 + seed)
    inp = W.make_inputs(wl)
    print(f"[random] seed {seed}: {c['kind']} {wl} splits={c['splits']}", flush=True)
    q, k, v = to_device(inp)
    mask = None
    if c["kind"] == "strided":
        q, k, v = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    elif c["kind"] == "sparse":
        r = c["rng"]
        mB = [1, wl.B][r.integers(2)]
        mH = [1, wl.HKV, wl.H][r.integers(3)]
        nqb, nkb = -(-wl.Sq // W.MASK_BLOCK_Q), -(-wl.Sk // W.MASK_BLOCK_K)
        mask = (r.random((mB, mH, nqb, nkb)) < r.uniform(0.2, 0.9)).astype(np.uint8)
    o, lse = fa.fwd(q, k, v, causal=bool(wl.causal), window=wl.window, scale=wl.scale(),
                    num_splits=c["splits"],
                    block_mask=None if mask is None else torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    O, L = attention(inp.q, inp.k, inp.v, wl.scale(), bool(wl.causal), wl.window, block_mask=mask)
    compare(host64(o), host64(lse), O, L, TOL[wl.dtype], wl.name)


@pytest.mark.parametrize("seed", range(24))
def test_random_backward(seed):
    # the three backward entry points: fa_bwd (contiguous), fa_bwd_strided
    # (token-major views, gradients in the same layout), fa_bwd_block_sparse
    # (a random mask with a random axis form)
    c = draw(5000 + seed)
    Sq, Sk = min(c["Sq"], 200), min(c["Sk"], 200)
    wl = wl_small(c["dtype"], c["B"], c["H"], c["HKV"], Sq, Sk, c["D"], c["causal"],
                  c["window"], name=f"randbwd{seed}", seed=300 + seed)
    _check_backward(c, wl, f"backward seed {seed}")


@pytest.mark.parametrize("seed", range(int(os.environ.get("FA_RANDOM_LONG_SEEDS", "8"))))
def test_random_backward_long_rows(seed):
    # the same on small grids with long row walks (one batch, few kv heads,
    # 1000 .. 2200 query rows): the dK/dV row chunks, the dQ key chunks, the
    # staged fp32 head dims 16 / 48 / 80 and the one reduction launch
    c = draw(9000 + seed)
    r = c["rng"]
    HKV = int(r.integers(1, 3))
    H = HKV * int(r.choice([1, 2, 4, 8]))
    while H * c["D"] > 512 and H > HKV:   # (keeps the oracle to seconds)
        H //= 2
    Sq, Sk = int(r.integers(1000, 2200)), int(r.integers(200, 1000))
    wl = wl_small(c["dtype"], 1, H, HKV, Sq, Sk, c["D"], c["causal"], c["window"],
                  name=f"randbwdlong{seed}", seed=500 + seed)
    _check_backward(c, wl, f"long-row backward seed {seed}")


def _check_backward(c, wl, what):
    import attention_forward_online_fa_amd as fa
    inp = W.make_inputs(wl)
    print(f"[random] {what}: {c['kind']} {wl}", flush=True)
    q, k, v = to_device(inp)
    g, bits = W.make_grad_output(inp)
    if bits is not None:
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
        src = torch.from_numpy(bits.view(np.int16)).view(tdt)
    else:
        src = torch.from_numpy(g)
    mask = None
    if c["kind"] == "strided":
        q, k, v = (x.transpose(1, 2).contiguous().transpose(1, 2) for x in (q, k, v))
    elif c["kind"] == "sparse":
        r = c["rng"]
        mB = [1, wl.B][r.integers(2)]
        mH = [1, wl.HKV, wl.H][r.integers(3)]
        nqb, nkb = -(-wl.Sq // W.MASK_BLOCK_Q), -(-wl.Sk // W.MASK_BLOCK_K)
        mask = (r.random((mB, mH, nqb, nkb)) < r.uniform(0.2, 0.9)).astype(np.uint8)
    m = None if mask is None else torch.from_numpy(mask).cuda()
    o, lse = fa.fwd(q, k, v, causal=bool(wl.causal), window=wl.window, scale=wl.scale(),
                    block_mask=m)
    do = torch.empty_like(o)      # o's layout
    do.copy_(src.cuda())
    got = fa.bwd(q, k, v, o, lse, do, causal=bool(wl.causal), window=wl.window,
                 scale=wl.scale(), block_mask=m)
    torch.cuda.synchronize()
    ref = attention_backward(inp.q, inp.k, inp.v, g, wl.scale(), bool(wl.causal), wl.window,
                             block_mask=mask)
    for name, x, r in zip(("dQ", "dK", "dV"), got, ref):
        x = host64(x)
        err = float(np.abs(x - r).max()) if r.size else 0.0
        tol = BWD_TOL[wl.dtype] * max(1.0, float(np.abs(r).max()) if r.size else 1.0)
        print(f"  {name}: max|d|={err:.3e} (tol {tol:.3e})", flush=True)
        assert np.all(np.isfinite(x)) and err <= tol, f"{name}: {err:.3e} > {tol:.3e}"


@pytest.mark.parametrize("seed", range(12))
def test_random_backward_block_mask(seed):
    # fa_bwd_block_sparse on random shapes (the block-mask head dims), masks
    # of random density and axis form, causal and window flags
    import attention_forward_online_fa_amd as fa
    c = draw(7000 + seed)
    r = c["rng"]
    D = [64, 128, 256][r.integers(3)]
    Sq, Sk = min(c["Sq"] + 100, 400), min(c["Sk"] + 100, 500)
    wl = wl_small(c["dtype"], c["B"], c["H"], c["HKV"], Sq, Sk, D, c["causal"], c["window"],
                  name=f"randbwdmask{seed}", seed=400 + seed)
    inp = W.make_inputs(wl)
    mB = [1, wl.B][r.integers(2)]
    mH = [1, wl.HKV, wl.H][r.integers(3)]
    nqb, nkb = -(-Sq // W.MASK_BLOCK_Q), -(-Sk // W.MASK_BLOCK_K)
    mask = (r.random((mB, mH, nqb, nkb)) < r.uniform(0.2, 0.9)).astype(np.uint8)
    print(f"[random] masked backward seed {seed}: {wl} mask {mask.shape}", flush=True)
    q, k, v = to_device(inp)
    g, bits = W.make_grad_output(inp)
    if bits is not None:
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
        do = torch.from_numpy(bits.view(np.int16)).view(tdt).cuda()
    else:
        do = torch.from_numpy(g).cuda()
    m = torch.from_numpy(mask).cuda()
    o, lse = fa.fwd(q, k, v, causal=bool(wl.causal), window=wl.window, scale=wl.scale(),
                    block_mask=m)
    got = fa.bwd(q, k, v, o, lse, do, causal=bool(wl.causal), window=wl.window,
                 scale=wl.scale(), block_mask=m)
    torch.cuda.synchronize()
    ref = attention_backward(inp.q, inp.k, inp.v, g, wl.scale(), bool(wl.causal), wl.window,
                             block_mask=mask)
    for name, x, rr in zip(("dQ", "dK", "dV"), got, ref):
        x = host64(x)
        err = float(np.abs(x - rr).max())
        tol = BWD_TOL[wl.dtype] * max(1.0, float(np.abs(rr).max()))
        print(f"  {name}: max|d|={err:.3e} (tol {tol:.3e})", flush=True)
        assert np.all(np.isfinite(x)) and err <= tol, f"{name}: {err:.3e} > {tol:.3e}"

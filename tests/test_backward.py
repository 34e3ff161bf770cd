"""GPU parity of the backward pass (fa_bwd) against the fp64 oracle's
gradients, on the same seeded inputs; O and LSE come from the library's own
forward pass, as a caller would use them.

Tolerance (absolute, scaled by the largest reference magnitude r = max(1,
max|ref|) of each gradient): bf16 1e-2 r, fp16 2e-3 r, fp32 1e-5 r. The
16-bit errors come from three roundings to the input type, each of relative
size at most its unit roundoff u (2^-8 for bf16, 2^-11 for fp16): the backward
reads O rounded, so D_i = dO_i . O_i is off by up to u sum|dO||O|, which every
dS_ij = P_ij (dP_ij - D_i) inherits; and P and dS are rounded as MFMA
operands. The rounding errors of a gradient's many terms have independent
signs, so its error stays a small multiple of u r: the bounds are 2.56 u
(bf16) and 4.1 u (fp16), 3.7x and 6.3x the largest errors measured over every
backward case of the test suite, the benchmark shape included (2.74e-3 r and
3.15e-4 r). fp32 (fp32 MFMA and per-row kernels, fp32 throughout): 1e-5 r, 5x
the largest measured (2.0e-6 r). The inputs themselves are exact on both
sides."""
import numpy as np
import pytest

import workloads as W
from oracle import attention_backward
from test_parity import host64, to_device, wl_small

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2, "f16": 2e-3}


def grads(wl, seed=0):
    import attention_forward_online_fa_amd as fa
    inp = W.make_inputs(wl)
    q, k, v = to_device(inp)
    rng = np.random.default_rng(wl.seed + 1000 + seed)
    dO = rng.standard_normal(q.shape).astype(np.float32)
    if wl.dtype in W.ROUNDING:
        to_bits, to_f32 = W.ROUNDING[wl.dtype]
        bits = to_bits(dO)
        dO = to_f32(bits)
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
        do = torch.from_numpy(bits.view(np.int16)).view(tdt).cuda()
    else:
        do = torch.from_numpy(dO).cuda()
    print(f"[backward] {wl}", flush=True)
    o, lse = fa.fwd(q, k, v, causal=bool(wl.causal), window=wl.window, scale=wl.scale())
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=bool(wl.causal), window=wl.window,
                        scale=wl.scale())
    torch.cuda.synchronize()
    ref = attention_backward(inp.q, inp.k, inp.v, dO, wl.scale(), bool(wl.causal), wl.window)
    return (host64(dq), host64(dk), host64(dv)), ref


CASES = [
    # dtype, B, H, HKV, Sq, Sk, D, causal, window
    ("f32", 1, 1, 1, 64, 64, 64, 0, 0),
    ("f32", 2, 4, 2, 150, 150, 64, 1, 0),
    ("f32", 1, 4, 1, 130, 90, 128, 1, 0),        # Sq > Sk
    ("f32", 1, 2, 2, 100, 170, 128, 0, 40),      # window without causal
    ("f32", 1, 2, 1, 90, 120, 256, 1, 30),
    ("bf16", 2, 4, 2, 150, 150, 64, 1, 0),
    ("bf16", 1, 4, 1, 200, 230, 128, 0, 0),
    ("bf16", 1, 2, 1, 90, 120, 256, 1, 30),
    ("f16", 1, 4, 2, 160, 160, 128, 1, 50),
    ("f16", 1, 2, 1, 70, 100, 256, 0, 0),
]


# several query tiles and key blocks for the MFMA kernels (16-bit; at D = 256
# the dK/dV kernel takes half of the output dims per workgroup)
CASES += [
    ("bf16", 1, 4, 2, 700, 900, 256, 1, 0),
    ("f16", 1, 2, 1, 500, 1300, 256, 0, 200),
    ("bf16", 1, 8, 2, 1024, 1024, 128, 1, 0),
    ("bf16", 1, 4, 4, 700, 1100, 64, 0, 0),
    ("f16", 1, 4, 1, 1000, 1000, 128, 1, 300),
    ("bf16", 2, 2, 1, 900, 600, 128, 0, 250),
]

# small grids on the per-row kernels (fp32 at D = 16, 48, 80): the rows'
# ranges run in up to eight chunks whose partial sums are added afterwards
CASES += [
    ("f32", 1, 2, 1, 1024, 1024, 48, 1, 0),      # eight chunks, causal
    ("f32", 1, 2, 2, 600, 900, 16, 0, 100),      # a window alone: ranges up to Sk / Sq
    ("f32", 1, 4, 1, 800, 800, 80, 1, 300),      # causal band of 300
]

# fp32 at D = 256: the fp32 MFMA kernels with the head dims split over
# wavefront pairs (64 query rows or keys per workgroup; partial scores and dP
# added through LDS): several tiles, odd Sq and Sk, GQA, windows, dQ key
# chunks (Sk 3000 over one query tile group) and dK/dV row chunks
CASES += [
    ("f32", 1, 2, 1, 600, 700, 256, 0, 0),
    ("f32", 1, 2, 1, 91, 121, 256, 1, 30),
    ("f32", 1, 2, 2, 77, 133, 256, 0, 0),
    ("f32", 1, 4, 2, 700, 900, 256, 1, 0),       # row chunks of 128 rows
    ("f32", 1, 1, 1, 200, 3000, 256, 0, 0),      # five key chunks
    ("f32", 2, 2, 1, 333, 517, 256, 0, 100),
    ("f32", 1, 2, 1, 1100, 1100, 256, 1, 300),
]

# few query tiles on the MFMA kernels: the dQ kernel splits the key axis into
# chunks of whole key tiles whose partial sums are added in chunk order
CASES += [
    ("bf16", 1, 2, 1, 200, 4000, 128, 0, 0),
    ("bf16", 1, 2, 1, 200, 4000, 128, 1, 0),     # causal: every chunk past key 200 is empty
    ("f32", 1, 2, 2, 300, 3000, 64, 0, 500),
    ("bf16", 1, 1, 1, 256, 2048, 256, 0, 0),
    ("f16", 1, 4, 2, 130, 2600, 96, 1, 900),     # padded head dim, window and key chunks
]

# the same shapes on the MFMA kernels (fp32 at D = 64, 32, 96; bf16 at D = 256)
CASES += [
    ("f32", 1, 2, 1, 1024, 1024, 64, 1, 0),
    ("f32", 1, 2, 2, 600, 900, 32, 0, 100),
    ("f32", 1, 4, 1, 800, 800, 96, 1, 300),
    ("bf16", 1, 2, 1, 600, 700, 256, 0, 0),
    ("bf16", 1, 2, 1, 91, 121, 256, 1, 30),     # odd Sq and Sk
]


# small grids whose dK/dV workgroups walk long row ranges (Sq x H / HKV, fp32
# counted four times, at least 4096): the MFMA dK/dV kernels cut the query
# rows into chunks of 128-row blocks whose partial sums are added in chunk
# order (causal, windowed, non-causal with Sq > Sk, ragged Sq, the general
# form of a padded head dim, D = 256 with two output halves, fp32)
CASES += [
    ("bf16", 1, 4, 1, 1100, 700, 64, 0, 0),
    ("f16", 1, 8, 2, 1040, 1040, 128, 1, 200),
    ("bf16", 1, 8, 2, 1030, 1030, 96, 1, 0),
    ("bf16", 1, 4, 2, 2100, 2100, 256, 1, 0),
    ("f32", 1, 4, 1, 600, 600, 128, 1, 0),
    ("f32", 1, 2, 2, 1300, 500, 32, 0, 0),
]


# fp32 head dims 16, 48, 80 with enough work (B H visible pairs at least
# 2^23): staged into the fp32 MFMA kernels of the 32, 64, 96 tiles, the extra
# dims zero (the smaller cases above keep the per-row kernels)
CASES += [
    ("f32", 1, 8, 2, 1500, 1500, 48, 1, 0),
    ("f32", 1, 4, 1, 2100, 2100, 16, 0, 300),
    ("f32", 1, 8, 2, 1500, 1500, 80, 1, 0),
]


@pytest.mark.parametrize("case", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_backward_matches_oracle(case):
    wl = wl_small(*case, seed=sum(case[1:]) + 3)
    got, ref = grads(wl)
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        scale_r = max(1.0, float(np.abs(r).max()))
        err = float(np.abs(g - r).max())
        print(f"  {name}: max|d|={err:.3e} (tol {TOL[wl.dtype] * scale_r:.3e})", flush=True)
        assert np.all(np.isfinite(g)), name
        assert err <= TOL[wl.dtype] * scale_r, f"{name}: {err:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_backward_empty_rows_and_unseen_keys(dtype):
    # Sq=8, Sk=40, causal, window 1: rows 0..7 see only their own key; keys
    # 8..39 are seen by no row (dK = dV = 0 there); no row is empty.
    # Sq=40, Sk=8, causal, window 1: rows >= 8 see nothing (dQ = 0 there).
    for shape in [(1, 2, 1, 8, 40, 64, 1, 1), (1, 2, 1, 40, 8, 64, 1, 1)]:
        wl = wl_small(dtype, *shape, seed=sum(shape))
        (dq, dk, dv), ref = grads(wl)
        Sq, Sk = shape[3], shape[4]
        if Sk > Sq:
            assert np.all(dk[:, :, Sq:] == 0) and np.all(dv[:, :, Sq:] == 0)
        else:
            assert np.all(dq[:, :, Sk:] == 0)
        for g, r in zip((dq, dk, dv), ref):
            assert float(np.abs(g - r).max()) <= TOL[dtype] * max(1.0, float(np.abs(r).max()))


@pytest.mark.parametrize("D", [48, 64])
def test_backward_deterministic_fp32_chunked(D):
    # fp32 on a small grid: at D = 48 the per-row kernels' chunked ranges,
    # partial sums added in a fixed order; at D = 64 the fp32 MFMA kernels
    import attention_forward_online_fa_amd as fa
    wl = wl_small("f32", 1, 2, 1, 900, 900, D, 1, 0, seed=6)
    q, k, v = to_device(W.make_inputs(wl))
    do = torch.randn_like(q)
    o, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(q, k, v, o, lse, do, causal=True)
    b = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_backward_deterministic():
    import attention_forward_online_fa_amd as fa
    wl = wl_small("bf16", 1, 4, 1, 300, 300, 128, 1, 0, seed=5)
    q, k, v = to_device(W.make_inputs(wl))
    do = torch.randn_like(q)
    o, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(q, k, v, o, lse, do, causal=True)
    b = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


# ------------------------------------------------- the benchmarked shape
def test_backward_benchmark_shape():
    # bf16 causal GQA B2 H32/8 S4096 D128 (the shape bench.py --pass bwd
    # times), gradients of two whole kv-head groups against the oracle: dQ of
    # their 2 x 4 query heads on every row, dK and dV of the two kv heads (the
    # oracle's backward on a group's slice is exact for that group)
    import attention_forward_online_fa_amd as fa
    wl = W.CONFIGS[W.HEADLINE]
    inp = W.make_inputs(wl)
    q, k, v = to_device(inp)
    g_np, bits = W.make_grad_output(inp)
    do = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()
    print(f"[backward] {wl.name} (full size)", flush=True)
    o, lse = fa.fwd(q, k, v, causal=True, scale=wl.scale())
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True, scale=wl.scale())
    torch.cuda.synchronize()
    gsz = wl.H // wl.HKV
    for b, hk in ((0, 0), (1, wl.HKV - 1)):
        hs = slice(hk * gsz, (hk + 1) * gsz)
        ref = attention_backward(inp.q[b:b + 1, hs], inp.k[b:b + 1, hk:hk + 1],
                                 inp.v[b:b + 1, hk:hk + 1], g_np[b:b + 1, hs], wl.scale(), True, 0)
        got = (host64(dq[b:b + 1, hs]), host64(dk[b:b + 1, hk:hk + 1]),
               host64(dv[b:b + 1, hk:hk + 1]))
        for name, gg, r in zip(("dQ", "dK", "dV"), got, ref):
            scale_r = max(1.0, float(np.abs(r).max()))
            err = float(np.abs(gg - r).max())
            print(f"  b={b} kv head {hk} {name}: max|d|={err:.3e} max|ref|={scale_r:.3e} "
                  f"(tol {TOL['bf16'] * scale_r:.3e})", flush=True)
            assert np.all(np.isfinite(gg)), name
            assert err <= TOL["bf16"] * scale_r, f"{name}: {err:.3e}"

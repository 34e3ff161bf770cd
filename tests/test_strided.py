"""GPU parity of the strided entry point (fa_fwd_strided) against the fp64
oracle and against the contiguous path.

Layouts: token-major [B, S, heads, D] storage viewed as [B, heads, S, D] (the
layout of the forge flash_attention.metal kernels), one packed QKV buffer
[B, S, H + 2 HKV, D] with GQA, K/V broadcast over the batch (batch stride 0),
and a token-major output. The strided kernels run the same arithmetic in the
same order as the contiguous ones, so with the same key-split count the
results must be bit-identical to the contiguous path; each case also checks
the oracle within the dtype's tolerance (see test_parity.py)."""
import numpy as np
import pytest

import workloads as W
from oracle import attention
from test_parity import TOL, compare, host64, to_device, wl_small

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def token_major(t):
    """A [B, heads, S, D] view of a token-major copy of t."""
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def run_both(wl, q, k, v, o=None, num_splits=0):
    import attention_forward_online_fa_amd as fa
    qc, kc, vc = (x.contiguous() for x in (q, k, v))
    oc, lc = fa.fwd(qc, kc, vc, causal=bool(wl.causal), window=wl.window, scale=wl.scale(),
                    num_splits=num_splits)
    if o is None:
        os_, ls = fa.fwd(q, k, v, causal=bool(wl.causal), window=wl.window, scale=wl.scale(),
                         num_splits=num_splits)
    else:
        ls = torch.empty(wl.B, wl.H, wl.Sq, dtype=torch.float32, device=q.device)
        os_, ls = fa.fwd_into(q, k, v, o, ls, causal=bool(wl.causal), window=wl.window,
                              scale=wl.scale(), num_splits=num_splits)
    torch.cuda.synchronize()
    return (oc, lc), (os_, ls)


def check(wl, inp, q, k, v, o=None, num_splits=0, bitwise=True):
    _say(f"[strided] {wl} splits={num_splits} q.stride={q.stride()} k.stride={k.stride()}")
    (oc, lc), (os_, ls) = run_both(wl, q, k, v, o, num_splits)
    if bitwise:
        assert torch.equal(oc, os_.contiguous()), "strided O differs from the contiguous path"
        assert torch.equal(lc, ls), "strided LSE differs from the contiguous path"
    O, L = attention(inp.q, inp.k, inp.v, wl.scale(), bool(wl.causal), wl.window)
    compare(host64(os_), host64(ls), O, L, TOL[wl.dtype], f"{wl.name} strided")


CASES = [
    # dtype, B, H, HKV, Sq, Sk, D, causal, window
    ("f32", 2, 4, 2, 300, 300, 64, 1, 0),
    ("f32", 1, 4, 1, 257, 190, 128, 1, 0),
    ("f32", 1, 2, 1, 150, 170, 256, 0, 50),
    ("bf16", 2, 4, 2, 300, 300, 64, 1, 0),
    ("bf16", 1, 8, 2, 257, 190, 128, 1, 0),
    ("bf16", 2, 2, 1, 333, 1111, 128, 0, 500),
    ("bf16", 1, 4, 1, 1536, 1536, 128, 1, 0),
    ("bf16", 1, 2, 1, 150, 170, 256, 1, 0),
    ("f16", 1, 4, 1, 384, 500, 128, 1, 100),
    ("f16", 1, 2, 1, 640, 1000, 256, 0, 0),
]


@pytest.mark.parametrize("case", CASES, ids=["-".join(map(str, c)) for c in CASES])
@pytest.mark.parametrize("splits", [0, 3])
def test_token_major(case, splits):
    wl = wl_small(*case, seed=sum(case[1:]) + 1)
    inp = W.make_inputs(wl)
    q, k, v = (token_major(x) for x in to_device(inp))
    o = token_major(torch.empty_like(q.contiguous()))       # token-major output too
    # fp32 causal small grids run persistent pieces whose split count depends
    # on the kernel form's occupancy: compare bitwise only with a fixed count
    bitwise = splits != 0 or wl.dtype != "f32"
    check(wl, inp, q, k, v, o=o, num_splits=splits, bitwise=bitwise)


@pytest.mark.parametrize("dtype,D", [("f32", 128), ("bf16", 128), ("bf16", 64), ("f16", 256)])
def test_packed_qkv_gqa(dtype, D):
    B, H, HKV, S = 2, 8, 2, 333
    wl = wl_small(dtype, B, H, HKV, S, S, D, 1, 0, seed=21 + D)
    inp = W.make_inputs(wl)
    q0, k0, v0 = to_device(inp)
    buf = torch.empty(B, S, H + 2 * HKV, D, dtype=q0.dtype, device=q0.device)
    buf[:, :, :H] = q0.transpose(1, 2)
    buf[:, :, H:H + HKV] = k0.transpose(1, 2)
    buf[:, :, H + HKV:] = v0.transpose(1, 2)
    q = buf[:, :, :H].transpose(1, 2)
    k = buf[:, :, H:H + HKV].transpose(1, 2)
    v = buf[:, :, H + HKV:].transpose(1, 2)
    assert k.stride(2) == (H + 2 * HKV) * D
    check(wl, inp, q, k, v, num_splits=2)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_kv_broadcast_over_batch(dtype):
    # one K/V for every batch entry: batch stride 0
    B = 3
    wl1 = wl_small(dtype, 1, 4, 2, 200, 260, 128, 1, 0, seed=31)
    inp1 = W.make_inputs(wl1)
    _, k1, v1 = to_device(inp1)
    wl = wl_small(dtype, B, 4, 2, 200, 260, 128, 1, 0, seed=32)
    inp = W.make_inputs(wl)
    q, _, _ = to_device(inp)
    k = k1.expand(B, -1, -1, -1)
    v = v1.expand(B, -1, -1, -1)
    assert k.stride(0) == 0
    inp.k = np.broadcast_to(inp1.k, inp.k.shape).copy()
    inp.v = np.broadcast_to(inp1.v, inp.v.shape).copy()
    check(wl, inp, q, k, v, num_splits=1)



# ------------------------------------------------------- strided backward
BWD_TOL = {"f32": 1e-5, "bf16": 1e-2, "f16": 2e-3}   # the bounds of test_backward.py


def _bwd_check(wl, inp, q, k, v, do_np, do_dev):
    """fa.bwd on the given views (fa_bwd_strided) against the contiguous
    fa_bwd (the same kernels on contiguous rows: bit-identical) and the
    oracle's gradients."""
    import attention_forward_online_fa_amd as fa
    from oracle import attention_backward
    qc, kc, vc, doc = (x.contiguous() for x in (q, k, v, do_dev))
    o, lse = fa.fwd(qc, kc, vc, causal=bool(wl.causal), window=wl.window, scale=wl.scale())
    ref = fa.bwd(qc, kc, vc, o, lse, doc, causal=bool(wl.causal), window=wl.window,
                 scale=wl.scale())
    o_view = token_major(o) if not q.is_contiguous() else o
    got = fa.bwd(q, k, v, o_view, lse, do_dev, causal=bool(wl.causal), window=wl.window,
                 scale=wl.scale())
    torch.cuda.synchronize()
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        assert torch.equal(g.contiguous(), r), f"strided {name} differs from the contiguous path"
    oq = attention_backward(inp.q, inp.k, inp.v, do_np, wl.scale(), bool(wl.causal), wl.window)
    for name, g, r in zip(("dQ", "dK", "dV"), got, oq):
        err = float(np.abs(host64(g) - r).max())
        bound = BWD_TOL[wl.dtype] * max(1.0, float(np.abs(r).max()))
        _say(f"  strided bwd {name}: max|d|={err:.3e} (tol {bound:.3e})")
        assert err <= bound, name
    return got


def _grad_out(wl, q):
    rng = np.random.default_rng(wl.seed + 5000)
    g = rng.standard_normal(tuple(q.shape)).astype(np.float32)
    if wl.dtype in W.ROUNDING:
        to_bits, to_f32 = W.ROUNDING[wl.dtype]
        bits = to_bits(g)
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
        return to_f32(bits), torch.from_numpy(bits.view(np.int16)).view(tdt).cuda()
    return g, torch.from_numpy(g).cuda()


BWD_CASES = [
    ("f32", 1, 4, 2, 150, 150, 64, 1, 0),
    ("bf16", 1, 8, 2, 300, 300, 128, 1, 0),
    ("bf16", 1, 4, 2, 200, 260, 96, 0, 70),    # padded head dim and strides together
    ("f16", 1, 2, 1, 130, 170, 256, 1, 0),
    ("bf16", 1, 2, 1, 130, 2200, 128, 0, 0),   # key chunks of the dQ kernel on views
    ("f16", 1, 4, 2, 200, 300, 48, 1, 0),      # head dim 48 (the 64 tile) on views
    # row chunks of the dK/dV kernels on views: the chunk sums go to
    # contiguous rows, then into the dK / dV views
    ("bf16", 1, 8, 2, 1030, 1030, 128, 1, 0),
    ("f32", 1, 4, 1, 600, 600, 64, 1, 100),
    # fp32 head dim 48 staged into the 64 tile (enough work for it)
    ("f32", 1, 8, 2, 1500, 1500, 48, 1, 0),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=["-".join(map(str, c)) for c in BWD_CASES])
def test_backward_token_major(case):
    # forge's backward layout: Q, K, V, O, dO token-major [B, S, heads, D];
    # the gradients come back token-major too
    wl = wl_small(*case, seed=sum(case[1:]) + 7)
    inp = W.make_inputs(wl)
    _say(f"[strided bwd] token-major {wl}")
    q, k, v = (token_major(x) for x in to_device(inp))
    g_np, g_dev = _grad_out(wl, q)
    dq, dk, dv = _bwd_check(wl, inp, q, k, v, g_np, token_major(g_dev))
    assert dq.stride() == q.stride() and dk.stride() == k.stride()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_backward_packed_qkv(dtype):
    # Q, K, V slices of one packed [B, S, H + 2 HKV, D] buffer (GQA)
    B, H, HKV, S, D = 2, 4, 2, 200, 64
    wl = wl_small(dtype, B, H, HKV, S, S, D, 1, 0, seed=41)
    inp = W.make_inputs(wl)
    _say(f"[strided bwd] packed QKV {wl}")
    q0, k0, v0 = to_device(inp)
    buf = torch.empty(B, S, H + 2 * HKV, D, dtype=q0.dtype, device=q0.device)
    buf[:, :, :H] = q0.transpose(1, 2)
    buf[:, :, H:H + HKV] = k0.transpose(1, 2)
    buf[:, :, H + HKV:] = v0.transpose(1, 2)
    q = buf[:, :, :H].transpose(1, 2)
    k = buf[:, :, H:H + HKV].transpose(1, 2)
    v = buf[:, :, H + HKV:].transpose(1, 2)
    g_np, g_dev = _grad_out(wl, q0)
    _bwd_check(wl, inp, q, k, v, g_np, g_dev)

"""GPU parity of the head dims 16, 32, 48, 80 and 96 (the head dims the forge
flash_attention.metal page instantiates besides 64 and 128) against the fp64
oracle, forward and backward.

These dims run the padded kernel form: the 64- or 128-dim kernels with the
dims from D on held as zeros on chip (Q in registers, K/V chunks copied from
out of the buffer's range), whatever the row strides. Cases cover every
dtype, ragged lengths, causal and window masks, GQA, forced key splits (the
merge kernel then writes only D of each partial row), token-major views, K/V
rows with a stride that is not a multiple of D, and a multi-tile case long
enough for the interior-tile path. A padded-form call on contiguous tensors
and one on a token-major copy of them run the same arithmetic in the same
order, so their results must be bit-identical. Tolerances as in
test_parity.py (forward) and test_backward.py (backward)."""
import numpy as np
import pytest

import workloads as W
from oracle import attention, attention_backward
from test_parity import TOL, compare, host64, to_device, wl_small

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

BWD_TOL = {"f32": 1e-5, "bf16": 1e-2, "f16": 2e-3}   # the bounds of test_backward.py


def _say(msg):
    print(msg, flush=True)


def token_major(t):
    return t.transpose(1, 2).contiguous().transpose(1, 2)


def row_padded(t, extra=16):
    """A view of t whose rows sit extra elements apart beyond D."""
    B, Hh, S, D = t.shape
    buf = torch.zeros(B, Hh, S, D + extra, dtype=t.dtype, device=t.device)
    buf[..., :D] = t
    return buf[..., :D]


FWD_CASES = [
    # dtype, B, H, HKV, Sq, Sk, D, causal, window
    ("f32", 1, 4, 2, 300, 333, 16, 1, 0),
    ("f32", 2, 2, 1, 257, 190, 48, 0, 0),
    ("f32", 1, 4, 1, 200, 260, 80, 1, 70),
    ("f32", 1, 2, 2, 129, 400, 96, 0, 100),
    ("f32", 1, 2, 1, 64, 64, 32, 1, 0),
    ("bf16", 1, 4, 2, 300, 333, 16, 1, 0),
    ("bf16", 2, 4, 1, 257, 190, 32, 0, 0),
    ("bf16", 1, 8, 2, 333, 500, 48, 1, 0),
    ("bf16", 1, 4, 1, 200, 700, 80, 0, 150),
    ("bf16", 2, 2, 1, 384, 384, 96, 1, 0),
    ("f16", 1, 4, 2, 300, 333, 48, 1, 40),
    ("f16", 1, 2, 1, 250, 520, 96, 0, 0),
    ("f16", 1, 4, 4, 130, 130, 16, 1, 0),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=["-".join(map(str, c)) for c in FWD_CASES])
@pytest.mark.parametrize("splits", [0, 3])
def test_forward(case, splits):
    import attention_forward_online_fa_amd as fa
    wl = wl_small(*case, name=f"hd{case[6]}", seed=sum(case[1:]) + splits)
    inp = W.make_inputs(wl)
    _say(f"[head dims] {wl} splits={splits}")
    q, k, v = to_device(inp)
    o, lse = fa.fwd(q, k, v, causal=bool(wl.causal), window=wl.window, scale=wl.scale(),
                    num_splits=splits)
    torch.cuda.synchronize()
    O, L = attention(inp.q, inp.k, inp.v, wl.scale(), bool(wl.causal), wl.window)
    compare(host64(o), host64(lse), O, L, TOL[wl.dtype], wl.name)
    # the same call on token-major copies (the padded form either way)
    qt, kt, vt = (token_major(x) for x in (q, k, v))
    ot = token_major(torch.empty_like(q))
    lt = torch.empty_like(lse)
    fa.fwd_into(qt, kt, vt, ot, lt, causal=bool(wl.causal), window=wl.window,
                scale=wl.scale(), num_splits=splits)
    torch.cuda.synchronize()
    if splits != 0 or wl.dtype != "f32":   # (auto splits of fp32 may depend on the form)
        assert torch.equal(o, ot.contiguous()), "token-major O differs from the contiguous call"
        assert torch.equal(lse, lt), "token-major LSE differs from the contiguous call"
    compare(host64(ot), host64(lt), O, L, TOL[wl.dtype], wl.name + " token-major")


@pytest.mark.parametrize("dtype,D", [("f32", 48), ("bf16", 96), ("bf16", 16), ("f16", 80)])
def test_row_stride_not_a_multiple_of_d(dtype, D):
    import attention_forward_online_fa_amd as fa
    wl = wl_small(dtype, 2, 4, 2, 250, 280, D, 1, 0, name=f"rowpad{D}", seed=D)
    inp = W.make_inputs(wl)
    q, k, v = to_device(inp)
    kp, vp = row_padded(k), row_padded(v, extra=32)
    assert kp.stride(2) == D + 16 and vp.stride(2) == D + 32
    _say(f"[head dims] row-padded K/V {wl} k.stride={kp.stride()} v.stride={vp.stride()}")
    o, lse = fa.fwd(q, kp, vp, causal=True, scale=wl.scale(), num_splits=2)
    o2, lse2 = fa.fwd(q, k, v, causal=True, scale=wl.scale(), num_splits=2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    O, L = attention(inp.q, inp.k, inp.v, wl.scale(), True, 0)
    compare(host64(o), host64(lse), O, L, TOL[wl.dtype], wl.name)


@pytest.mark.parametrize("dtype,D", [("bf16", 96), ("f16", 48), ("f32", 80)])
def test_multi_tile_causal(dtype, D):
    # 1536 rows: twelve query tiles, most key tiles interior
    import attention_forward_online_fa_amd as fa
    wl = wl_small(dtype, 1, 4, 1, 1536, 1536, D, 1, 0, name=f"long{D}", seed=7 + D)
    inp = W.make_inputs(wl)
    _say(f"[head dims] {wl}")
    q, k, v = to_device(inp)
    o, lse = fa.fwd(q, k, v, causal=True, scale=wl.scale())
    torch.cuda.synchronize()
    O, L = attention(inp.q, inp.k, inp.v, wl.scale(), True, 0)
    compare(host64(o), host64(lse), O, L, TOL[wl.dtype], wl.name)


def test_output_row_tail_is_untouched():
    # O rows of D elements inside wider rows: the elements past D keep their values
    import attention_forward_online_fa_amd as fa
    wl = wl_small("bf16", 1, 2, 1, 200, 200, 48, 1, 0, name="otail", seed=5)
    inp = W.make_inputs(wl)
    q, k, v = to_device(inp)
    buf = torch.full((1, 2, 200, 64), 7.0, dtype=q.dtype, device=q.device)
    o = buf[..., :48]
    lse = torch.empty(1, 2, 200, dtype=torch.float32, device=q.device)
    for splits in (1, 3):
        fa.fwd_into(q, k, v, o, lse, causal=True, scale=wl.scale(), num_splits=splits)
        torch.cuda.synchronize()
        assert bool((buf[..., 48:] == 7.0).all()), f"splits={splits}: O row tail written"
    O, L = attention(inp.q, inp.k, inp.v, wl.scale(), True, 0)
    compare(host64(o), host64(lse), O, L, TOL["bf16"], wl.name)


BWD_CASES = [
    ("f32", 1, 4, 2, 130, 150, 16, 1, 0),
    ("f32", 1, 2, 1, 100, 170, 96, 0, 40),
    ("bf16", 1, 4, 2, 150, 150, 48, 1, 0),
    ("bf16", 1, 2, 1, 120, 200, 80, 0, 0),
    ("f16", 1, 4, 1, 140, 140, 32, 1, 50),
    ("f16", 1, 2, 2, 90, 110, 96, 1, 0),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=["-".join(map(str, c)) for c in BWD_CASES])
def test_backward(case):
    import attention_forward_online_fa_amd as fa
    wl = wl_small(*case, name=f"bwdhd{case[6]}", seed=50 + sum(case[1:]))
    inp = W.make_inputs(wl)
    _say(f"[head dims] backward {wl}")
    q, k, v = to_device(inp)
    g, bits = W.make_grad_output(inp)
    if bits is not None:
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
        do = torch.from_numpy(bits.view(np.int16)).view(tdt).cuda()
    else:
        do = torch.from_numpy(g).cuda()
    o, lse = fa.fwd(q, k, v, causal=bool(wl.causal), window=wl.window, scale=wl.scale())
    got = fa.bwd(q, k, v, o, lse, do, causal=bool(wl.causal), window=wl.window,
                 scale=wl.scale())
    torch.cuda.synchronize()
    ref = attention_backward(inp.q, inp.k, inp.v, g, wl.scale(), bool(wl.causal), wl.window)
    for name, x, r in zip(("dQ", "dK", "dV"), got, ref):
        x = host64(x)
        err = float(np.abs(x - r).max())
        tol = BWD_TOL[wl.dtype] * max(1.0, float(np.abs(r).max()))
        print(f"  {name}: max|d|={err:.3e} (tol {tol:.3e})", flush=True)
        assert np.all(np.isfinite(x)) and err <= tol, f"{name}: {err:.3e} > {tol:.3e}"


def test_padded_keys_with_a_copy_range_past_2gb():
    # K/V rows 32 KB apart over 65536 keys: for the early key tiles the bytes
    # from the tile's first row to the end of K exceed 2 GB, so a copy's range
    # is capped; the padded dims' chunks (sent out of range) must still read
    # as zeros. 64 query rows, head dim 96 (the 128 tile's padded form).
    import attention_forward_online_fa_amd as fa
    D, Sq, Sk, rs = 96, 64, 65536, 16448
    wl = wl_small("bf16", 1, 1, 1, Sq, Sk, D, 0, 0, name="long-stride", seed=3)
    inp = W.make_inputs(wl)
    q, k, v = to_device(inp)
    _say(f"[head dims] {wl} K/V row stride {rs} elements")
    kbuf = torch.full((Sk, rs), 3.0, dtype=k.dtype, device=k.device)   # nonzero filler
    vbuf = torch.full((Sk, rs), 3.0, dtype=v.dtype, device=v.device)
    kbuf[:, :D] = k[0, 0]
    vbuf[:, :D] = v[0, 0]
    kv = kbuf[:, :D].unsqueeze(0).unsqueeze(0)
    vv = vbuf[:, :D].unsqueeze(0).unsqueeze(0)
    assert kv.stride(2) == rs and (Sk - 1) * rs * 2 > 2 ** 31
    o, lse = fa.fwd(q, kv, vv, causal=False, scale=wl.scale(), num_splits=1)
    torch.cuda.synchronize()
    O, L = attention(inp.q, inp.k, inp.v, wl.scale(), False, 0)
    compare(host64(o), host64(lse), O, L, TOL[wl.dtype], wl.name)
    del kbuf, vbuf

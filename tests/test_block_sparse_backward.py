"""GPU parity of the backward pass under a block mask (fa_bwd_block_sparse)
against the fp64 oracle's masked gradients (oracle.attention_backward with
block_mask, pinned in test_oracle_backward_mask.py), on the same seeded
inputs; O and LSE come from the library's own masked forward pass, as a
caller would use them. Tolerances as in test_backward.py (the masked kernels
run the same arithmetic on fewer tiles)."""
import numpy as np
import pytest

import workloads as W
from oracle import attention_backward
from test_backward import TOL
from test_parity import host64, to_device, wl_small

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def random_mask(rng, mB, mH, Sq, Sk, density):
    nqb = -(-Sq // W.MASK_BLOCK_Q)
    nkb = -(-Sk // W.MASK_BLOCK_K)
    return (rng.random((mB, mH, nqb, nkb)) < density).astype(np.uint8)


def grad_output(wl, q, seed):
    rng = np.random.default_rng(wl.seed + 2000 + seed)
    dO = rng.standard_normal(q.shape).astype(np.float32)
    if wl.dtype in W.ROUNDING:
        to_bits, to_f32 = W.ROUNDING[wl.dtype]
        bits = to_bits(dO)
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
        return to_f32(bits), torch.from_numpy(bits.view(np.int16)).view(tdt).cuda()
    return dO, torch.from_numpy(dO).cuda()


def masked_grads(wl, inp, mask, seed=0):
    import attention_forward_online_fa_amd as fa
    q, k, v = to_device(inp)
    dO, do = grad_output(wl, q, seed)
    m = torch.from_numpy(mask).cuda()
    print(f"[masked backward] {wl} mask {mask.shape} density {mask.mean():.2f}", flush=True)
    o, lse = fa.fwd(q, k, v, causal=bool(wl.causal), window=wl.window, scale=wl.scale(),
                    block_mask=m)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=bool(wl.causal), window=wl.window,
                        scale=wl.scale(), block_mask=m)
    torch.cuda.synchronize()
    return (host64(dq), host64(dk), host64(dv)), dO


def check(wl, got, ref, kv_growth=1.0):
    # kv_growth widens the dK / dV tolerance where each key sums far more rows
    # than the cases the base tolerances were set on
    for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
        scale_r = max(1.0, float(np.abs(r).max())) * (kv_growth if name != "dQ" else 1.0)
        err = float(np.abs(g - r).max())
        print(f"  {name}: max|d|={err:.3e} (tol {TOL[wl.dtype] * scale_r:.3e})", flush=True)
        assert np.all(np.isfinite(g)), name
        assert err <= TOL[wl.dtype] * scale_r, f"{name}: {err:.3e}"


CASES = [
    # dtype, B, H, HKV, Sq, Sk, D, causal, window, mask batch ("1"/"B"), mask heads ("1"/"kv"/"q")
    ("bf16", 1, 4, 2, 300, 700, 128, 0, 0, "1", "kv"),
    ("bf16", 2, 4, 1, 520, 520, 128, 1, 0, "B", "q"),
    ("f16", 1, 2, 2, 260, 900, 64, 0, 300, "1", "1"),
    ("bf16", 1, 2, 1, 200, 650, 256, 1, 0, "1", "q"),
    ("bf16", 1, 1, 1, 130, 2100, 256, 0, 0, "1", "1"),   # key chunks of the D = 256 dQ kernel
    ("f32", 1, 4, 2, 300, 500, 64, 1, 0, "1", "kv"),
    ("f32", 2, 2, 1, 260, 390, 128, 0, 200, "B", "q"),
    ("f32", 1, 2, 1, 190, 330, 256, 1, 0, "1", "1"),    # fp32 D = 256: 64-key workgroups, one mask column
    ("f32", 1, 4, 2, 700, 1000, 256, 0, 300, "B", "kv"),  # with dK/dV row chunks
    # small grids with long row walks: dK/dV row chunks under the mask
    ("bf16", 1, 8, 2, 1100, 1100, 128, 0, 0, "1", "kv"),
    ("f32", 1, 4, 1, 700, 700, 64, 1, 0, "1", "q"),
]


@pytest.mark.parametrize("density", [0.5, 0.85])
@pytest.mark.parametrize("case", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_masked_backward_matches_oracle(case, density):
    dtype, B, H, HKV, Sq, Sk, D, causal, window, mb, mh = case
    wl = wl_small(dtype, B, H, HKV, Sq, Sk, D, causal, window, seed=sum(case[1:9]) + 7)
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(int(density * 100) + Sq + Sk)
    mask = random_mask(rng, B if mb == "B" else 1, {"1": 1, "kv": HKV, "q": H}[mh], Sq, Sk,
                       density)
    got, dO = masked_grads(wl, inp, mask)
    ref = attention_backward(inp.q, inp.k, inp.v, dO, wl.scale(), bool(causal), window,
                             block_mask=mask)
    check(wl, got, ref)


@pytest.mark.parametrize("dtype,D,Sq", [("bf16", 128, 300), ("f32", 64, 300), ("bf16", 256, 300),
                                        ("f32", 256, 300), ("bf16", 128, 1100), ("f32", 64, 1100),
                                        ("f32", 256, 1100)])
def test_all_ones_mask_equals_dense_backward(dtype, D, Sq):
    # every block visible: the same gradients as fa_bwd, bit for bit (Sq =
    # 1100: both with dK/dV row chunks)
    import attention_forward_online_fa_amd as fa
    wl = wl_small(dtype, 1, 8 if Sq > 1000 else 4, 2, Sq, 400, D, 1, 0, seed=21)
    q, k, v = to_device(W.make_inputs(wl))
    _, do = grad_output(wl, q, 1)
    ones = torch.ones(1, 1, -(-Sq // 128), 7, dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd(q, k, v, causal=True)
    a = fa.bwd(q, k, v, o, lse, do, causal=True)
    b = fa.bwd(q, k, v, o, lse, do, causal=True, block_mask=ones)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unseen_keys_and_empty_rows_get_zero_gradients(dtype):
    # key block 1 masked for every row: its keys get dK = dV = 0 exactly;
    # query block 1 sees no block: its rows get dQ = 0 exactly
    wl = wl_small(dtype, 1, 2, 1, 300, 300, 64, 0, 0, seed=22)
    inp = W.make_inputs(wl)
    mask = np.ones((1, 1, 3, 5), dtype=np.uint8)
    mask[:, :, :, 1] = 0
    mask[:, :, 1, :] = 0
    (dq, dk, dv), dO = masked_grads(wl, inp, mask)
    assert np.all(dk[:, :, 64:128] == 0) and np.all(dv[:, :, 64:128] == 0)
    assert np.all(dq[:, :, 128:256] == 0)
    ref = attention_backward(inp.q, inp.k, inp.v, dO, wl.scale(), False, 0, block_mask=mask)
    check(wl, (dq, dk, dv), ref)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 256)])
def test_dkdv_list_in_portions(dtype, D):
    # one key block seen by 16 query heads x 625 row tiles of 64 rows (fp32:
    # 1250 of 32) = 10000 (20000) pairs, more than a dK/dV workgroup's list
    # holds (8192; fp32 D = 256: 4096): the list
    # is built and worked in portions. 1024 key blocks of 64 keys or more, so
    # that the grid is too large for row chunks (and the forward's 2048-tile
    # list still holds the key axis); only the first 64 keys are visible, so
    # the oracle takes those alone, and every other key must get dK = dV = 0
    # exactly
    Sk = 1024 * (128 if dtype == "bf16" else 64)
    wl = wl_small(dtype, 1, 16, 1, 40000, Sk, D, 0, 0, seed=23)
    inp = W.make_inputs(wl)
    mask = np.zeros((1, 1, -(-40000 // 128), Sk // 64), dtype=np.uint8)
    mask[0, 0, :, 0] = 1
    mask[0, 0, 7::11, 0] = 0
    (dq, dk, dv), dO = masked_grads(wl, inp, mask)
    assert np.all(dk[:, :, 64:] == 0) and np.all(dv[:, :, 64:] == 0)
    ref = attention_backward(inp.q, inp.k[:, :, :64], inp.v[:, :, :64], dO, wl.scale(), False, 0,
                             block_mask=mask[:, :, :, :1])
    # each of the 64 keys sums ~580,000 (query head, row) terms in fp32, whose
    # rounding error grows like the square root of the term count: fp32 dK
    # and dV get the base tolerance (set on sums of up to ~4096 terms) times
    # sqrt(terms / 4096); the bf16 tolerance already covers it
    terms = 16 * int(mask[0, 0, :, 0].sum()) * 128
    check(wl, (dq, dk[:, :, :64], dv[:, :, :64]), ref,
          kv_growth=np.sqrt(terms / 4096) if dtype == "f32" else 1.0)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f32", 64), ("f32", 256)])
def test_dq_list_in_portions(dtype, D):
    # 128 query blocks x 4 heads (no key chunks) over 9000 key tiles (8470
    # visible): each dQ workgroup's list overflows its 8192 entries (fp32 D = 256:
    # 4096) and is worked in portions.
    # dQ of query block 5 of head 1, non-causal, against the oracle on that
    # block alone (a query row's dQ depends only on its own row and the keys)
    import attention_forward_online_fa_amd as fa
    Sq, Sk = 128 * 128, 9000 * 32
    wl = wl_small(dtype, 1, 4, 1, Sq, Sk, D, 0, 0, seed=24)
    inp = W.make_inputs(wl)
    q, k, v = to_device(inp)
    dO, do = grad_output(wl, q, 2)
    nkb = -(-Sk // W.MASK_BLOCK_K)
    mask = np.ones((1, 1, Sq // 128, nkb), dtype=np.uint8)
    mask[0, 0, :, 3::17] = 0
    m = torch.from_numpy(mask).cuda()
    print(f"[masked backward] {wl} (dQ portions)", flush=True)
    o, lse = fa.fwd(q, k, v, scale=wl.scale(), block_mask=m)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, scale=wl.scale(), block_mask=m)
    torch.cuda.synchronize()
    rows = slice(5 * 128, 6 * 128)
    ref = attention_backward(inp.q[:, 1:2, rows], inp.k, inp.v, dO[:, 1:2, rows], wl.scale(),
                             block_mask=mask[:, :, 5:6])
    g = host64(dq[:, 1:2, rows])
    scale_r = max(1.0, float(np.abs(ref[0]).max()))
    err = float(np.abs(g - ref[0]).max())
    print(f"  dQ: max|d|={err:.3e} (tol {TOL[dtype] * scale_r:.3e})", flush=True)
    assert err <= TOL[dtype] * scale_r


def test_block_mask_backward_argument_errors():
    import attention_forward_online_fa_amd as fa
    wl = wl_small("bf16", 1, 4, 2, 200, 200, 128, 0, 0, seed=25)
    q, k, v = to_device(W.make_inputs(wl))
    o, lse = fa.fwd(q, k, v)
    do = torch.randn_like(q)
    bad_heads = torch.ones(1, 3, 2, 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FaError) as e:
        fa.bwd(q, k, v, o, lse, do, block_mask=bad_heads)
    assert e.value.status == 12                                   # FA_ERR_MASK
    with pytest.raises(ValueError):                               # wrong block counts
        fa.bwd(q, k, v, o, lse, do, block_mask=torch.ones(1, 1, 2, 3, dtype=torch.uint8,
                                                          device="cuda"))
    wl96 = wl_small("bf16", 1, 2, 1, 200, 200, 96, 0, 0, seed=26)
    q9, k9, v9 = to_device(W.make_inputs(wl96))
    o9, l9 = fa.fwd(q9, k9, v9)
    with pytest.raises(fa.FaError) as e:
        fa.bwd(q9, k9, v9, o9, l9, torch.randn_like(q9),
               block_mask=torch.ones(1, 1, 2, 4, dtype=torch.uint8, device="cuda"))
    assert e.value.status == 4                                    # FA_ERR_HEAD_DIM

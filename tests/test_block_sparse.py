"""GPU parity of the block-sparse entry point (fa_fwd_block_sparse) against
the fp64 oracle's block masks (metal-flash-attention README, "Modifications
to FlashAttention": programmable block masks).

Masks of several densities (all blocks off, sparse, dense, all on), every
mask axis form (batch 1 or B; heads 1, HKV or H), with causal and window
rules on top, ragged shapes, forced key splits, and a key range long enough
that a workgroup's tile list forces splits. An all-ones mask runs the same
tiles in the same order as the dense kernels, so it must be bit-identical to
the dense path. Tolerances as in test_parity.py."""
import numpy as np
import pytest

import workloads as W
from oracle import attention
from test_parity import TOL, compare, host64, to_device, wl_small

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def random_mask(rng, mB, mH, Sq, Sk, density):
    nqb = -(-Sq // W.MASK_BLOCK_Q)
    nkb = -(-Sk // W.MASK_BLOCK_K)
    return (rng.random((mB, mH, nqb, nkb)) < density).astype(np.uint8)


def check_masked(wl, inp, mask, num_splits=0):
    import attention_forward_online_fa_amd as fa
    _say(f"[block-sparse] {wl} mask {mask.shape} density {mask.mean():.2f} splits={num_splits}")
    q, k, v = to_device(inp)
    o, lse = fa.fwd(q, k, v, causal=bool(wl.causal), window=wl.window, scale=wl.scale(),
                    num_splits=num_splits, block_mask=torch.from_numpy(mask).cuda())
    torch.cuda.synchronize()
    O, L = attention(inp.q, inp.k, inp.v, wl.scale(), bool(wl.causal), wl.window,
                     block_mask=mask)
    compare(host64(o), host64(lse), O, L, TOL[wl.dtype], f"{wl.name} masked")
    return o, lse


CASES = [
    # dtype, B, H, HKV, Sq, Sk, D, causal, window, mask batch, mask heads ("1", "kv", "q")
    ("f32", 2, 4, 2, 300, 333, 64, 0, 0, "B", "kv"),
    ("f32", 1, 4, 1, 384, 384, 128, 1, 0, "1", "q"),
    ("f32", 1, 2, 1, 260, 700, 256, 0, 200, "1", "1"),
    ("bf16", 2, 4, 2, 300, 333, 64, 0, 0, "B", "kv"),
    ("bf16", 1, 8, 2, 640, 1000, 128, 1, 0, "1", "q"),
    ("bf16", 2, 2, 1, 333, 1111, 128, 0, 500, "B", "1"),
    ("bf16", 1, 2, 1, 260, 700, 256, 1, 0, "1", "kv"),
    ("f16", 1, 4, 2, 500, 900, 128, 0, 0, "1", "kv"),
    ("f16", 1, 2, 1, 200, 640, 256, 0, 0, "1", "q"),
]


@pytest.mark.parametrize("case", CASES, ids=["-".join(map(str, c)) for c in CASES])
@pytest.mark.parametrize("density", [0.0, 0.3, 0.8])
def test_random_masks(case, density):
    dtype, B, H, HKV, Sq, Sk, D, causal, window, mb, mh = case
    wl = wl_small(dtype, B, H, HKV, Sq, Sk, D, causal, window, seed=Sq + Sk + D)
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(int(density * 10) + Sq)
    mask = random_mask(rng, B if mb == "B" else 1, {"1": 1, "kv": HKV, "q": H}[mh], Sq, Sk,
                       density)
    check_masked(wl, inp, mask)
    check_masked(wl, inp, mask, num_splits=3)


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128), ("bf16", 256), ("f16", 64)])
def test_all_ones_mask_equals_dense_path(dtype, D):
    import attention_forward_online_fa_amd as fa
    wl = wl_small(dtype, 1, 4, 2, 700, 700, D, 1, 0, seed=70 + D)
    inp = W.make_inputs(wl)
    q, k, v = to_device(inp)
    ones = torch.ones(1, 1, -(-700 // 128), -(-700 // 64), dtype=torch.uint8, device="cuda")
    for ns in (1, 2):
        a = fa.fwd(q, k, v, causal=True, num_splits=ns)
        b = fa.fwd(q, k, v, causal=True, num_splits=ns, block_mask=ones)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rows_with_no_visible_block_are_exactly_empty(dtype):
    wl = wl_small(dtype, 1, 2, 1, 400, 300, 128, 0, 0, seed=80)
    inp = W.make_inputs(wl)
    mask = np.ones((1, 1, 4, 5), np.uint8)
    mask[0, 0, 1] = 0                    # query block 1 (rows 128..255) sees nothing
    mask[0, 0, 3, :] = 0
    mask[0, 0, 3, 4] = 1                 # rows 384..399 see only keys 256..299
    o, lse = check_masked(wl, inp, mask)
    o, lse = host64(o), host64(lse)
    assert np.all(o[:, :, 128:256] == 0) and np.all(np.isneginf(lse[:, :, 128:256]))


def test_long_key_range_forces_splits():
    # 70000 keys = 2188 tiles of 32 > 2048 per workgroup list: the library splits
    wl = wl_small("bf16", 1, 1, 1, 130, 70000, 128, 0, 0, seed=90)
    inp = W.make_inputs(wl)
    mask = random_mask(np.random.default_rng(9), 1, 1, 130, 70000, 0.5)
    check_masked(wl, inp, mask)


def test_block_mask_argument_errors():
    import attention_forward_online_fa_amd as fa
    wl = wl_small("bf16", 1, 4, 2, 200, 200, 64, 0, 0, seed=91)
    q, k, v = to_device(W.make_inputs(wl))
    bad_heads = torch.ones(1, 3, 2, 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(fa.FaError):
        fa.fwd(q, k, v, block_mask=bad_heads)
    with pytest.raises(ValueError):
        fa.fwd(q, k, v, block_mask=torch.ones(1, 1, 2, 3, dtype=torch.uint8, device="cuda"))

"""Pins for the oracle's backward pass under a block mask (metal-flash-attention
README, "Modifications to FlashAttention": programmable block masks held in
memory; forge flash_attention.metal backward kernels: P recomputed from the
saved log-sum-exp, dS = P (dP - D)).

The masked backward is the gradient of L = sum(O * dO) for the masked forward,
so it is pinned against torch float64 autograd of a masked softmax written
here with an element mask built by scalar loops from the block bytes (no
oracle code), against central finite differences through the oracle's masked
forward (pinned in test_oracle_block_mask.py), and against closed forms: an
all-ones mask is no mask, keys in blocks no row sees get zero dK and dV, an
all-zero mask gives zero gradients. A mutant that ignores the mask in the
backward is rejected. CPU only."""
import importlib
import math
import types

import numpy as np
import pytest
import torch

from oracle import attention, attention_backward

SHAPES = [
    # B, H, HKV, Sq, Sk, D, causal, window, bq, bk, mask heads ("1", "kv", "q"), mask batch
    (1, 1, 1, 7, 9, 3, 0, 0, 2, 3, "1", 1),
    (2, 4, 2, 8, 10, 3, 1, 0, 3, 2, "kv", 2),
    (1, 4, 2, 9, 9, 2, 1, 4, 2, 2, "q", 1),
    (2, 2, 1, 6, 11, 4, 0, 5, 4, 3, "q", 2),
]


def _case(shape, seed):
    B, H, HKV, Sq, Sk, D, causal, window, bq, bk, mh, mB = shape
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, Sq, D))
    K = rng.standard_normal((B, HKV, Sk, D))
    V = rng.standard_normal((B, HKV, Sk, D))
    dO = rng.standard_normal((B, H, Sq, D))
    nh = {"1": 1, "kv": HKV, "q": H}[mh]
    bm = (rng.random((mB, nh, -(-Sq // bq), -(-Sk // bk))) < 0.6).astype(np.uint8)
    return Q, K, V, dO, bool(causal), window, bm, bq, bk


def _element_mask(B, H, HKV, Sq, Sk, causal, window, bm, bq, bk):
    """Boolean [B, H, Sq, Sk] from scalar loops over the rules and the block bytes."""
    g = H // HKV
    vis = np.zeros((B, H, Sq, Sk), dtype=bool)
    for b in range(B):
        for h in range(H):
            mb = b if bm.shape[0] == B else 0
            mh = h if bm.shape[1] == H else (h // g if bm.shape[1] == HKV and HKV > 1 else 0)
            for i in range(Sq):
                for j in range(Sk):
                    vis[b, h, i, j] = ((not causal or j <= i) and (window == 0 or j >= i - window + 1)
                                       and bm[mb, mh, i // bq, j // bk] != 0)
    return vis


def _torch_masked_forward(Q, K, V, scale, vis):
    """softmax(scale Q K^T) V over the visible pairs, written directly in torch."""
    g = Q.shape[1] // K.shape[1]
    Kr = K.repeat_interleave(g, dim=1)
    Vr = V.repeat_interleave(g, dim=1)
    s = scale * torch.matmul(Q, Kr.transpose(-1, -2).contiguous())
    s = s.masked_fill(~torch.from_numpy(vis), -math.inf)
    p = torch.nan_to_num(torch.softmax(s, dim=-1), nan=0.0)   # empty rows: P = 0
    return torch.matmul(p, Vr)


def _autograd(Q, K, V, dO, scale, vis):
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    out = _torch_masked_forward(tq, tk, tv, scale, vis)
    return [t.numpy() for t in torch.autograd.grad(out, (tq, tk, tv), torch.tensor(dO))]


@pytest.mark.parametrize("shape", SHAPES)
def test_masked_backward_against_torch_autograd(shape):
    Q, K, V, dO, causal, window, bm, bq, bk = _case(shape, 300 + sum(shape[:10]))
    B, H, HKV, Sq, Sk = shape[:5]
    vis = _element_mask(B, H, HKV, Sq, Sk, causal, window, bm, bq, bk)
    gq, gk, gv = _autograd(Q, K, V, dO, 0.55, vis)
    dQ, dK, dV = attention_backward(Q, K, V, dO, 0.55, causal, window, block_mask=bm,
                                    block_q=bq, block_k=bk)
    np.testing.assert_allclose(dQ, gq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, gk, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, gv, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shape", SHAPES[:2])
def test_masked_backward_against_finite_differences(shape):
    Q, K, V, dO, causal, window, bm, bq, bk = _case(shape, 400 + sum(shape[:10]))
    scale = 0.6
    dQ, dK, dV = attention_backward(Q, K, V, dO, scale, causal, window, block_mask=bm,
                                    block_q=bq, block_k=bk)
    loss = lambda q, k, v: float((attention(q, k, v, scale, causal, window, block_mask=bm,
                                            block_q=bq, block_k=bk)[0] * dO).sum())
    h = 1e-6
    for X, G, name in ((Q, dQ, "dQ"), (K, dK, "dK"), (V, dV, "dV")):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            num[idx] = (loss(*[Xp if X is A else A for A in (Q, K, V)])
                        - loss(*[Xm if X is A else A for A in (Q, K, V)])) / (2 * h)
        np.testing.assert_allclose(G, num, rtol=0, atol=2e-7, err_msg=name)


@pytest.mark.parametrize("causal,window", [(0, 0), (1, 0), (1, 3)])
def test_all_ones_mask_is_no_mask(causal, window):
    Q, K, V, dO, _, _, _, _, _ = _case((2, 4, 2, 8, 10, 3, 0, 0, 3, 2, "kv", 2), 11)
    ones = np.ones((1, 1, 3, 5), dtype=np.uint8)
    a = attention_backward(Q, K, V, dO, 0.5, bool(causal), window, block_mask=ones, block_q=3,
                           block_k=2)
    b = attention_backward(Q, K, V, dO, 0.5, bool(causal), window)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_keys_no_row_sees_get_zero_gradients():
    # key block 1 (keys 2, 3) is masked for every row: their dK and dV are
    # exactly 0, and dQ is the gradient of attention over the other keys only
    Q, K, V, dO, _, _, _, _, _ = _case((1, 2, 1, 6, 6, 3, 0, 0, 2, 2, "1", 1), 12)
    bm = np.ones((1, 1, 3, 3), dtype=np.uint8)
    bm[:, :, :, 1] = 0
    dQ, dK, dV = attention_backward(Q, K, V, dO, 0.7, block_mask=bm, block_q=2, block_k=2)
    assert np.all(dK[:, :, 2:4] == 0) and np.all(dV[:, :, 2:4] == 0)
    keep = [0, 1, 4, 5]
    rQ, rK, rV = attention_backward(Q, K[:, :, keep], V[:, :, keep], dO, 0.7)
    np.testing.assert_allclose(dQ, rQ, rtol=0, atol=1e-14)
    np.testing.assert_allclose(dK[:, :, keep], rK, rtol=0, atol=1e-14)
    np.testing.assert_allclose(dV[:, :, keep], rV, rtol=0, atol=1e-14)


def test_all_zero_mask_gives_zero_gradients():
    Q, K, V, dO, _, _, _, _, _ = _case((1, 2, 2, 5, 7, 3, 0, 0, 2, 2, "1", 1), 13)
    zero = np.zeros((1, 2, 3, 4), dtype=np.uint8)
    for x in attention_backward(Q, K, V, dO, 0.5, block_mask=zero, block_q=2, block_k=2):
        assert np.all(x == 0)


MUTANTS = [
    ("mask_ignored", "vis = vis_rule & block_visible(", "vis = vis_rule | 0 * block_visible("),
    ("mask_head_is_q_head", "vis = vis_rule & block_visible(_mask_slice(block_mask, b, h, hk, H)",
     "vis = vis_rule & block_visible(_mask_slice(block_mask, b, h, h, H)"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_masked_backward_pins_reject_mutant(name, old, new):
    real = importlib.import_module("oracle.attention")
    src = open(real.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_bwd_mask_mutant")
    exec(compile(src.replace(old, new), "oracle_bwd_mask_mutant", "exec"), mod.__dict__)
    caught = False
    for shape in SHAPES:
        Q, K, V, dO, causal, window, bm, bq, bk = _case(shape, 300 + sum(shape[:10]))
        B, H, HKV, Sq, Sk = shape[:5]
        vis = _element_mask(B, H, HKV, Sq, Sk, causal, window, bm, bq, bk)
        gq, gk, gv = _autograd(Q, K, V, dO, 0.55, vis)
        try:
            mQ, mK, mV = mod.attention_backward(Q, K, V, dO, 0.55, causal, window, block_mask=bm,
                                                block_q=bq, block_k=bk)
        except (ValueError, IndexError):
            caught = True
            continue
        if not (np.allclose(mQ, gq, atol=1e-12) and np.allclose(mK, gk, atol=1e-12)
                and np.allclose(mV, gv, atol=1e-12)):
            caught = True
    assert caught, f"mutant {name} survived"

"""Pins for the oracle's backward pass (forge flash_attention.metal backward
kernels: recomputed P from the saved log-sum-exp, the FA2 identity
D_i = dO_i . O_i, dS = P (dP - D), GQA sums over a kv head's query heads).

Pinned against central finite differences of L = sum(O * dO) through the
oracle's forward (itself pinned in test_oracle.py), torch float64 autograd of
an independent masked-softmax forward, GQA == MHA with repeated K/V (summed
gradients), and closed forms. Mutants of the backward are rejected. CPU only."""
import importlib
import math
import types

import numpy as np
import pytest
import torch

from oracle import attention, attention_backward

SHAPES = [
    # B, H, HKV, Sq, Sk, D, causal, window
    (1, 1, 1, 5, 6, 3, 0, 0),
    (1, 2, 1, 6, 6, 4, 1, 0),
    (2, 4, 2, 5, 7, 3, 1, 3),
    (1, 2, 2, 7, 4, 2, 1, 2),       # Sq > Sk: empty rows
    (1, 3, 1, 6, 8, 3, 0, 4),       # window without causal, GQA
]


def _case(shape, seed):
    B, H, HKV, Sq, Sk, D, causal, window = shape
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((B, H, Sq, D))
    K = rng.standard_normal((B, HKV, Sk, D))
    V = rng.standard_normal((B, HKV, Sk, D))
    dO = rng.standard_normal((B, H, Sq, D))
    return Q, K, V, dO, bool(causal), window


@pytest.mark.parametrize("shape", SHAPES)
def test_backward_against_finite_differences(shape):
    Q, K, V, dO, causal, window = _case(shape, sum(shape))
    scale = 0.6
    dQ, dK, dV = attention_backward(Q, K, V, dO, scale, causal, window)
    loss = lambda q, k, v: float((attention(q, k, v, scale, causal, window)[0] * dO).sum())
    h = 1e-6
    for X, G, name in ((Q, dQ, "dQ"), (K, dK, "dK"), (V, dV, "dV")):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += h
            Xm[idx] -= h
            args_p = [Xp if X is A else A for A in (Q, K, V)]
            args_m = [Xm if X is A else A for A in (Q, K, V)]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(G, num, rtol=0, atol=2e-7, err_msg=name)


def _torch_forward(Q, K, V, scale, causal, window):
    """Masked softmax attention written directly in torch (float64)."""
    B, H, Sq, D = Q.shape
    HKV, Sk = K.shape[1], K.shape[2]
    g = H // HKV
    Kr = K.repeat_interleave(g, dim=1)
    Vr = V.repeat_interleave(g, dim=1)
    s = scale * torch.matmul(Q, Kr.transpose(-1, -2).contiguous())
    i = torch.arange(Sq)[:, None]
    j = torch.arange(Sk)[None, :]
    vis = torch.ones(Sq, Sk, dtype=torch.bool)
    if causal:
        vis &= j <= i
    if window:
        vis &= j >= i - window + 1
    s = s.masked_fill(~vis, -math.inf)
    p = torch.softmax(s, dim=-1)
    p = torch.nan_to_num(p, nan=0.0)          # rows with no visible key: P = 0
    return torch.matmul(p, Vr)


@pytest.mark.parametrize("shape", SHAPES)
def test_backward_against_torch_autograd(shape):
    Q, K, V, dO, causal, window = _case(shape, 100 + sum(shape))
    scale = 0.45
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
    out = _torch_forward(tq, tk, tv, scale, causal, window)
    gq, gk, gv = torch.autograd.grad(out, (tq, tk, tv), torch.tensor(dO))
    dQ, dK, dV = attention_backward(Q, K, V, dO, scale, causal, window)
    np.testing.assert_allclose(dQ, gq.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dK, gk.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dV, gv.numpy(), rtol=0, atol=1e-12)


def test_backward_gqa_equals_summed_mha():
    Q, K, V, dO, causal, window = _case((2, 4, 2, 6, 6, 3, 1, 0), 7)
    dQ, dK, dV = attention_backward(Q, K, V, dO, 0.5, causal, window)
    Kr, Vr = np.repeat(K, 2, axis=1), np.repeat(V, 2, axis=1)
    mQ, mK, mV = attention_backward(Q, Kr, Vr, dO, 0.5, causal, window)
    np.testing.assert_allclose(dQ, mQ, rtol=0, atol=1e-13)
    np.testing.assert_allclose(dK, mK.reshape(2, 2, 2, 6, 3).sum(axis=2), rtol=0, atol=1e-13)
    np.testing.assert_allclose(dV, mV.reshape(2, 2, 2, 6, 3).sum(axis=2), rtol=0, atol=1e-13)


def test_backward_single_key_closed_form():
    # Sk = 1: P = 1 for every row, O = V_0, so dV_0 = sum_i dO_i and dS = 0
    # (dP_i = dO_i . V_0 = D_i), hence dQ = 0 and dK = 0.
    rng = np.random.default_rng(8)
    Q = rng.standard_normal((1, 2, 5, 4))
    K = rng.standard_normal((1, 1, 1, 4))
    V = rng.standard_normal((1, 1, 1, 4))
    dO = rng.standard_normal((1, 2, 5, 4))
    dQ, dK, dV = attention_backward(Q, K, V, dO, 0.7)
    np.testing.assert_allclose(dV[0, 0, 0], dO[0].sum(axis=(0, 1)), rtol=0, atol=1e-13)
    assert np.abs(dQ).max() < 1e-14 and np.abs(dK).max() < 1e-14


def test_backward_zero_q_uniform_weights():
    # Q = 0, non-causal: P_ij = 1/Sk, so dV_j = mean over... = sum_i dO_i / Sk
    rng = np.random.default_rng(9)
    Q = np.zeros((1, 1, 4, 3))
    K = rng.standard_normal((1, 1, 5, 3))
    V = rng.standard_normal((1, 1, 5, 3))
    dO = rng.standard_normal((1, 1, 4, 3))
    _, dK, dV = attention_backward(Q, K, V, dO, 0.9)
    for j in range(5):
        np.testing.assert_allclose(dV[0, 0, j], dO[0, 0].sum(axis=0) / 5, rtol=0, atol=1e-14)
    assert np.abs(dK).max() < 1e-14            # dK_j = scale sum_i dS_ij Q_i = 0


def test_backward_empty_rows_contribute_nothing():
    Q, K, V, dO, _, _ = _case((1, 2, 1, 8, 2, 3, 1, 1), 10)
    dQ, dK, dV = attention_backward(Q, K, V, dO, 0.5, True, 1)
    assert np.all(dQ[:, :, 2:] == 0)
    # only rows 0 and 1 (each seeing its own key) reach dK, dV
    dQ2, dK2, dV2 = attention_backward(Q[:, :, :2], K, V, dO[:, :, :2], 0.5, True, 1)
    np.testing.assert_allclose(dK, dK2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(dV, dV2, rtol=0, atol=1e-14)


MUTANTS = [
    ("no_d_term", "dS = P * (dP - Drow[:, None])", "dS = P * dP"),
    ("dq_without_scale", "dQ[b, h] = scale * (dS @ K[b, hk])", "dQ[b, h] = (dS @ K[b, hk])"),
    ("dk_without_scale", "dK[b, hk] += scale * (dS.T @ Q[b, h])", "dK[b, hk] += (dS.T @ Q[b, h])"),
    ("gqa_not_summed", "dV[b, hk] += P.T @ dO[b, h]", "dV[b, hk] = P.T @ dO[b, h]"),
    ("dv_from_ds", "dV[b, hk] += P.T @ dO[b, h]", "dV[b, hk] += dS.T @ dO[b, h]"),
    ("dk_from_k", "dK[b, hk] += scale * (dS.T @ Q[b, h])", "dK[b, hk] += scale * (dS.T @ K[b, hk])"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_backward_pins_reject_mutant(name, old, new):
    real = importlib.import_module("oracle.attention")
    src = open(real.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle_bwd_mutant")
    exec(compile(src.replace(old, new), "oracle_bwd_mutant", "exec"), mod.__dict__)
    caught = False
    for shape in SHAPES:
        Q, K, V, dO, causal, window = _case(shape, 100 + sum(shape))
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (Q, K, V))
        out = _torch_forward(tq, tk, tv, 0.45, causal, window)
        gq, gk, gv = torch.autograd.grad(out, (tq, tk, tv), torch.tensor(dO))
        try:
            mQ, mK, mV = mod.attention_backward(Q, K, V, dO, 0.45, causal, window)
        except ValueError:          # e.g. a shape mismatch: rejected
            caught = True
            continue
        if not (np.allclose(mQ, gq.numpy(), atol=1e-12) and np.allclose(mK, gk.numpy(), atol=1e-12)
                and np.allclose(mV, gv.numpy(), atol=1e-12)):
            caught = True
    assert caught, f"mutant {name} survived"

"""Pins for the oracle's block masks (metal-flash-attention README,
"Modifications to FlashAttention": programmable block masks held in memory).

A block mask has one byte per (query block, key block); key j is visible to
row i only if the byte of (i // block_q, j // block_k) is nonzero, on top of
the causal and window rules. Pinned against scalar brute force with exactly
rounded sums, torch's float64 SDPA with the expanded element mask, closed
forms (one visible block, Q = 0), and the degenerate masks (all ones = no
mask, all zeros = every row empty). CPU only."""
import math

import numpy as np
import pytest
import torch

from oracle import MASK_BLOCK_K, MASK_BLOCK_Q, attention, attention_rows


def _brute_masked(Q, K, V, scale, causal, window, bm, bq, bk):
    """Scalar loops over an explicit per-element predicate, unshifted exp,
    math.fsum sums. bm is [mB, mH, nqb, nkb]; its head axis is 1, HKV or H."""
    B, H, Sq, D = Q.shape
    HKV, Sk = K.shape[1], K.shape[2]
    g = H // HKV
    O = np.zeros((B, H, Sq, D))
    L = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            hk = h // g
            mb = b if bm.shape[0] == B else 0
            mh = h if bm.shape[1] == H else (hk if bm.shape[1] == HKV and HKV > 1 else 0)
            for i in range(Sq):
                js = [j for j in range(Sk)
                      if (not causal or j <= i) and (window == 0 or j >= i - window + 1)
                      and bm[mb, mh, i // bq, j // bk] != 0]
                if not js:
                    L[b, h, i] = -math.inf
                    continue
                w = [math.exp(scale * math.fsum(Q[b, h, i, d] * K[b, hk, j, d] for d in range(D)))
                     for j in js]
                tot = math.fsum(w)
                L[b, h, i] = math.log(tot)
                for d in range(D):
                    O[b, h, i, d] = math.fsum(w[n] * V[b, hk, j, d] for n, j in enumerate(js)) / tot
    return O, L


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
    nh = {"1": 1, "kv": HKV, "q": H}[mh]
    bm = (rng.random((mB, nh, -(-Sq // bq), -(-Sk // bk))) < 0.6).astype(np.uint8)
    return Q, K, V, bool(causal), window, bm, bq, bk


@pytest.mark.parametrize("shape", SHAPES)
def test_block_mask_brute_force(shape):
    Q, K, V, causal, window, bm, bq, bk = _case(shape, sum(shape[:9]))
    O, L = attention(Q, K, V, 0.7, causal, window, block_mask=bm, block_q=bq, block_k=bk)
    bO, bL = _brute_masked(Q, K, V, 0.7, causal, window, bm, bq, bk)
    fin = np.isfinite(bL)
    assert np.array_equal(np.isfinite(L), fin)
    np.testing.assert_allclose(O, bO, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L[fin], bL[fin], rtol=0, atol=1e-12)
    assert np.all(O[~fin] == 0) and np.all(L[~fin] == -np.inf)


@pytest.mark.parametrize("shape", SHAPES)
def test_block_mask_against_torch_sdpa(shape):
    Q, K, V, causal, window, bm, bq, bk = _case(shape, 7 + sum(shape[:9]))
    B, H, Sq, D = Q.shape
    HKV, Sk = K.shape[1], K.shape[2]
    O, L = attention(Q, K, V, 0.45, causal, window, block_mask=bm, block_q=bq, block_k=bk)
    g = H // HKV
    i = torch.arange(Sq)[:, None]
    j = torch.arange(Sk)[None, :]
    base = torch.ones(Sq, Sk, dtype=torch.bool)
    if causal:
        base &= j <= i
    if window:
        base &= j >= i - window + 1
    for b in range(B):
        for h in range(H):
            hk = h // g
            mb = b if bm.shape[0] == B else 0
            mh = h if bm.shape[1] == H else (hk if bm.shape[1] == HKV and HKV > 1 else 0)
            blk = torch.from_numpy(bm[mb, mh].astype(bool))
            el = blk.repeat_interleave(bq, 0)[:Sq].repeat_interleave(bk, 1)[:, :Sk]
            m = base & el
            rows = m.any(1)
            q = torch.from_numpy(Q[b, h])[rows]
            k = torch.from_numpy(K[b, hk])
            v = torch.from_numpy(V[b, hk])
            o = torch.nn.functional.scaled_dot_product_attention(
                q[None], k[None], v[None], attn_mask=m[rows][None], scale=0.45)[0]
            s = (q @ k.T) * 0.45
            lse = torch.logsumexp(s.masked_fill(~m[rows], -math.inf), dim=1)
            np.testing.assert_allclose(O[b, h][rows.numpy()], o.numpy(), rtol=0, atol=1e-12)
            np.testing.assert_allclose(L[b, h][rows.numpy()], lse.numpy(), rtol=0, atol=1e-12)
            assert np.all(O[b, h][~rows.numpy()] == 0)
            assert np.all(L[b, h][~rows.numpy()] == -np.inf)


@pytest.mark.parametrize("causal,window", [(0, 0), (1, 0), (1, 100), (0, 77)])
def test_all_ones_mask_is_no_mask(causal, window):
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((1, 2, 300, 8))
    K = rng.standard_normal((1, 1, 270, 8))
    V = rng.standard_normal((1, 1, 270, 8))
    bm = np.ones((1, 1, 3, 5), dtype=np.uint8)                  # default 128 x 64 blocks
    a = attention(Q, K, V, 0.3, bool(causal), window)
    b = attention(Q, K, V, 0.3, bool(causal), window, block_mask=bm)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_all_zero_mask_empties_every_row():
    rng = np.random.default_rng(4)
    Q = rng.standard_normal((2, 2, 130, 8))
    K = rng.standard_normal((2, 2, 70, 8))
    V = rng.standard_normal((2, 2, 70, 8))
    O, L = attention(Q, K, V, 0.3, False, 0, block_mask=np.zeros((2, 2, 2, 2), np.uint8))
    assert np.all(O == 0) and np.all(L == -np.inf)


def test_one_visible_block_with_zero_q_is_block_mean():
    # Q = 0: every visible score is 0, so O is the mean of V over the visible
    # keys and LSE = ln(count). Row block r sees only key block c(r) = (2r+1) % 4.
    rng = np.random.default_rng(5)
    Sq, Sk = 3 * MASK_BLOCK_Q - 7, 4 * MASK_BLOCK_K - 5
    Q = np.zeros((1, 1, Sq, 4))
    K = rng.standard_normal((1, 1, Sk, 4))
    V = rng.standard_normal((1, 1, Sk, 4))
    bm = np.zeros((1, 1, 3, 4), np.uint8)
    for r in range(3):
        bm[0, 0, r, (2 * r + 1) % 4] = 1
    O, L = attention(Q, K, V, 0.5, False, 0, block_mask=bm)
    for i in range(Sq):
        c = (2 * (i // MASK_BLOCK_Q) + 1) % 4
        keys = np.arange(c * MASK_BLOCK_K, min((c + 1) * MASK_BLOCK_K, Sk))
        np.testing.assert_allclose(O[0, 0, i], V[0, 0, keys].mean(axis=0), rtol=0, atol=1e-13)
        assert abs(L[0, 0, i] - math.log(len(keys))) <= 1e-13


def test_mask_head_axis_broadcast_rules():
    # per-kv-head mask == per-query-head mask repeated over each group;
    # a shared mask == per-query-head mask equal for every head
    rng = np.random.default_rng(6)
    Q = rng.standard_normal((2, 4, 140, 4))
    K = rng.standard_normal((2, 2, 200, 4))
    V = rng.standard_normal((2, 2, 200, 4))
    kv = (rng.random((2, 2, 2, 4)) < 0.5).astype(np.uint8)
    a = attention(Q, K, V, 0.4, True, 0, block_mask=kv)
    b = attention(Q, K, V, 0.4, True, 0, block_mask=np.repeat(kv, 2, axis=1))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    one = kv[:1, :1]
    c = attention(Q, K, V, 0.4, True, 0, block_mask=one)
    d = attention(Q, K, V, 0.4, True, 0, block_mask=np.broadcast_to(one, (2, 4, 2, 4)).copy())
    assert np.array_equal(c[0], d[0]) and np.array_equal(c[1], d[1])


def test_rows_variant_matches_full_with_mask():
    Q, K, V, causal, window, bm, bq, bk = _case(SHAPES[1], 11)
    O, L = attention(Q, K, V, 0.7, causal, window, block_mask=bm, block_q=bq, block_k=bk)
    rows = np.array([[b, h, i] for b in range(Q.shape[0]) for h in range(Q.shape[1])
                     for i in range(Q.shape[2])])
    Or, Lr = attention_rows(Q, K, V, 0.7, causal, window, rows, block_mask=bm, block_q=bq,
                            block_k=bk)
    assert np.array_equal(Or, O.reshape(-1, Q.shape[3]))
    assert np.array_equal(Lr, L.reshape(-1))

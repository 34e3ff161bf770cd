"""Pins for the fp64 oracle: hand-derived closed forms, brute-force exact sums,
invariants and special cases, and torch's float64 SDPA as an independent
library route. CPU only.

Each pin targets a mistake the oracle could plausibly carry (dropped scale,
wrong causal/window bound, wrong GQA head map, K and V swapped, no max shift,
LSE off by the max, empty-row convention)."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, attention_rows, visible_count, visible_mask

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _to_f64(x):
    a = np.array(x, dtype=object)
    f = np.vectorize(lambda v: float(v))
    return f(a).astype(np.float64)


def _rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


# ---------------------------------------------------------------- golden
with open(GOLDEN) as fh:
    CASES = json.load(fh)["cases"]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_closed_forms(case):
    Q, K, V = (_to_f64(case[n]) for n in ("Q", "K", "V"))
    O, L = attention(Q, K, V, case["scale"], bool(case["causal"]), case["window"])
    eO, eL = _to_f64(case["O"]), _to_f64(case["LSE"])
    assert O.shape == eO.shape and L.shape == eL.shape
    np.testing.assert_allclose(O, eO, rtol=0, atol=1e-12)
    fin = np.isfinite(eL)
    np.testing.assert_allclose(L[fin], eL[fin], rtol=0, atol=1e-12)
    assert np.all(L[~fin] == -np.inf)


# ---------------------------------------------------------------- brute force
def _brute(Q, K, V, scale, causal, window):
    """Scalar loops, unshifted exp, exactly rounded sums (math.fsum)."""
    B, H, Sq, D = Q.shape
    HKV, Sk = K.shape[1], K.shape[2]
    g = H // HKV
    O = np.zeros((B, H, Sq, D))
    L = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            hk = h // g
            for i in range(Sq):
                js = [j for j in range(Sk)
                      if (not causal or j <= i) and (window == 0 or j >= i - window + 1)]
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


BRUTE_SHAPES = [
    # B, H, HKV, Sq, Sk, D, causal, window
    (1, 1, 1, 5, 5, 3, 0, 0),
    (1, 1, 1, 6, 6, 4, 1, 0),
    (2, 4, 2, 5, 7, 3, 1, 0),      # GQA, Sk > Sq, causal top-left
    (1, 2, 1, 7, 4, 2, 1, 2),      # Sq > Sk: empty rows with window
    (1, 3, 3, 6, 6, 4, 0, 3),      # window without causal
    (1, 4, 1, 8, 8, 2, 1, 3),
]


@pytest.mark.parametrize("shape", BRUTE_SHAPES)
def test_brute_force_exact_sums(shape):
    B, H, HKV, Sq, Sk, D, causal, window = shape
    rng = np.random.default_rng(7 + sum(shape))
    Q, K, V = _rand((B, H, Sq, D), rng), _rand((B, HKV, Sk, D), rng), _rand((B, HKV, Sk, D), rng)
    scale = 0.7
    O, L = attention(Q, K, V, scale, bool(causal), window)
    bO, bL = _brute(Q, K, V, scale, causal, window)
    np.testing.assert_allclose(O, bO, rtol=0, atol=1e-12)
    fin = np.isfinite(bL)
    np.testing.assert_allclose(L[fin], bL[fin], rtol=0, atol=1e-12)
    assert np.all(L[~fin] == -np.inf) and np.all(O[~np.isfinite(bL)] == 0)


# ---------------------------------------------------------------- closed forms
def test_constant_v_gives_v():
    rng = np.random.default_rng(1)
    B, H, HKV, Sq, Sk, D = 2, 4, 2, 9, 13, 5
    Q, K = _rand((B, H, Sq, D), rng, 3.0), _rand((B, HKV, Sk, D), rng, 3.0)
    c = rng.standard_normal(D)
    V = np.broadcast_to(c, (B, HKV, Sk, D)).copy()
    for causal, window in [(0, 0), (1, 0), (1, 4), (0, 3)]:
        O, L = attention(Q, K, V, 0.4, bool(causal), window)
        ne = np.isfinite(L)
        np.testing.assert_allclose(O[ne], np.broadcast_to(c, O[ne].shape), rtol=0, atol=1e-12)


def test_causal_row0_is_v0():
    rng = np.random.default_rng(2)
    Q, K, V = _rand((1, 3, 6, 4), rng), _rand((1, 3, 6, 4), rng), _rand((1, 3, 6, 4), rng)
    O, L = attention(Q, K, V, 0.5, True, 0)
    np.testing.assert_allclose(O[:, :, 0], V[:, :, 0], rtol=0, atol=1e-13)
    s00 = 0.5 * np.einsum("bhd,bhd->bh", Q[:, :, 0], K[:, :, 0])
    np.testing.assert_allclose(L[:, :, 0], s00, rtol=0, atol=1e-13)


def test_causal_window1_selects_diagonal():
    rng = np.random.default_rng(3)
    Sq, Sk = 10, 7
    Q, K, V = _rand((1, 2, Sq, 3), rng), _rand((1, 1, Sk, 3), rng), _rand((1, 1, Sk, 3), rng)
    O, L = attention(Q, K, V, 1.3, True, 1)
    for h in range(2):
        for i in range(Sq):
            if i < Sk:
                np.testing.assert_allclose(O[0, h, i], V[0, 0, i], rtol=0, atol=1e-13)
                assert abs(L[0, h, i] - 1.3 * Q[0, h, i] @ K[0, 0, i]) < 1e-13
            else:
                assert np.all(O[0, h, i] == 0) and L[0, h, i] == -np.inf


def test_zero_q_gives_mean_and_log_count():
    rng = np.random.default_rng(4)
    Sq, Sk, D = 12, 9, 3
    Q = np.zeros((1, 1, Sq, D))
    K, V = _rand((1, 1, Sk, D), rng), _rand((1, 1, Sk, D), rng)
    for causal, window in [(0, 0), (1, 0), (1, 3), (0, 4)]:
        O, L = attention(Q, K, V, 0.9, bool(causal), window)
        cnt = visible_count(Sq, Sk, bool(causal), window)
        vis = visible_mask(np.arange(Sq), Sk, bool(causal), window)
        for i in range(Sq):
            if cnt[i] == 0:
                assert L[0, 0, i] == -np.inf and np.all(O[0, 0, i] == 0)
            else:
                np.testing.assert_allclose(O[0, 0, i], V[0, 0][vis[i]].mean(0), rtol=0, atol=1e-13)
                assert abs(L[0, 0, i] - math.log(cnt[i])) < 1e-13


def test_single_key():
    rng = np.random.default_rng(5)
    Q, K, V = _rand((2, 2, 5, 4), rng), _rand((2, 1, 1, 4), rng), _rand((2, 1, 1, 4), rng)
    O, L = attention(Q, K, V, 0.25, False, 0)
    np.testing.assert_allclose(O, np.broadcast_to(V[:, :, :1], O.shape), rtol=0, atol=1e-13)
    s = 0.25 * np.einsum("bhid,bd->bhi", Q, K[:, 0, 0])
    np.testing.assert_allclose(L, s, rtol=0, atol=1e-13)


def test_empty_row_case_sq8_sk2():
    rng = np.random.default_rng(6)
    Q, K, V = _rand((1, 1, 8, 4), rng), _rand((1, 1, 2, 4), rng), _rand((1, 1, 2, 4), rng)
    O, L = attention(Q, K, V, 0.5, True, 1)
    assert np.all(O[0, 0, 2:] == 0) and np.all(L[0, 0, 2:] == -np.inf)
    np.testing.assert_allclose(O[0, 0, :2], V[0, 0], rtol=0, atol=1e-13)


# ---------------------------------------------------------------- invariants
def test_softmax_rows_sum_to_one():
    # With V = identity (Sk = D), each O row is the probability row itself.
    rng = np.random.default_rng(8)
    Sk = 6
    Q, K = _rand((1, 1, 6, Sk), rng, 2.0), _rand((1, 1, Sk, Sk), rng, 2.0)
    V = np.eye(Sk)[None, None]
    for causal, window in [(0, 0), (1, 0), (1, 2)]:
        O, L = attention(Q, K, V, 0.8, bool(causal), window)
        np.testing.assert_allclose(O.sum(-1), 1.0, rtol=0, atol=1e-13)
        assert np.all(O >= 0)
        vis = visible_mask(np.arange(6), Sk, bool(causal), window)
        assert np.all(O[0, 0][~vis] == 0)


def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(9)
    B, H, HKV, S, D = 2, 8, 2, 11, 4
    Q, K, V = _rand((B, H, S, D), rng), _rand((B, HKV, S, D), rng), _rand((B, HKV, S, D), rng)
    g = H // HKV
    Kr, Vr = np.repeat(K, g, axis=1), np.repeat(V, g, axis=1)
    for causal, window in [(0, 0), (1, 0), (1, 5)]:
        O1, L1 = attention(Q, K, V, 0.6, bool(causal), window)
        O2, L2 = attention(Q, Kr, Vr, 0.6, bool(causal), window)
        np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)
        np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-13)


def test_window_at_least_sk_is_no_window():
    rng = np.random.default_rng(10)
    Q, K, V = _rand((1, 2, 9, 3), rng), _rand((1, 2, 9, 3), rng), _rand((1, 2, 9, 3), rng)
    for causal in (0, 1):
        O1, L1 = attention(Q, K, V, 0.5, bool(causal), 0)
        O2, L2 = attention(Q, K, V, 0.5, bool(causal), 9)
        O3, L3 = attention(Q, K, V, 0.5, bool(causal), 1000)
        np.testing.assert_array_equal(O1, O2)
        np.testing.assert_array_equal(O1, O3)
        np.testing.assert_array_equal(L1, L3)


def test_key_permutation_invariance_noncausal():
    rng = np.random.default_rng(11)
    Q, K, V = _rand((1, 2, 7, 4), rng), _rand((1, 1, 10, 4), rng), _rand((1, 1, 10, 4), rng)
    perm = rng.permutation(10)
    O1, L1 = attention(Q, K, V, 0.5, False, 0)
    O2, L2 = attention(Q, K[:, :, perm], V[:, :, perm], 0.5, False, 0)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-13)


def test_query_scale_tradeoff():
    rng = np.random.default_rng(12)
    Q, K, V = _rand((1, 2, 7, 4), rng), _rand((1, 2, 7, 4), rng), _rand((1, 2, 7, 4), rng)
    O1, L1 = attention(Q, K, V, 0.5, True, 0)
    O2, L2 = attention(4.0 * Q, K, V, 0.125, True, 0)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L1, L2, rtol=0, atol=1e-13)
    # and the scale really enters: doubling it changes the result
    O3, _ = attention(Q, K, V, 1.0, True, 0)
    assert np.max(np.abs(O3 - O1)) > 1e-3


def test_shift_stability_large_scores():
    # Adding a constant c to every score of a row leaves O unchanged and adds c
    # to LSE. Realised by appending a constant feature to q and k.
    rng = np.random.default_rng(13)
    Q, K, V = _rand((1, 1, 6, 4), rng), _rand((1, 1, 6, 4), rng), _rand((1, 1, 6, 4), rng)
    c = 800.0
    Q[..., 3] = c          # the last feature adds exactly c to every score
    Kc = K.copy()
    Kc[..., 3] = 1.0
    Qc = Q.copy()
    Q = Q.copy()
    Q[..., 3] = 0.0
    O1, L1 = attention(Q, Kc, V, 1.0, True, 0)
    O2, L2 = attention(Qc, Kc, V, 1.0, True, 0)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-10)
    np.testing.assert_allclose(L2 - L1, c, rtol=0, atol=1e-10)


# ---------------------------------------------------------------- library route
@pytest.mark.parametrize("shape", [
    (2, 4, 2, 33, 33, 16, 0, 0),
    (1, 4, 4, 40, 40, 8, 1, 0),
    (1, 8, 2, 37, 53, 16, 1, 0),     # Sq != Sk, top-left causal
    (2, 2, 1, 50, 50, 8, 1, 7),      # sliding window
    (1, 2, 2, 30, 45, 8, 0, 9),      # window without causal
    (1, 4, 2, 24, 30, 48, 1, 0),     # head dims of the padded kernel form
    (1, 2, 1, 20, 20, 96, 0, 6),
])
def test_against_torch_sdpa_float64(shape):
    B, H, HKV, Sq, Sk, D, causal, window = shape
    rng = np.random.default_rng(100 + Sq)
    Q, K, V = _rand((B, H, Sq, D), rng), _rand((B, HKV, Sk, D), rng), _rand((B, HKV, Sk, D), rng)
    scale = 1.0 / math.sqrt(D)
    O, L = attention(Q, K, V, scale, bool(causal), window)
    g = H // HKV
    q = torch.from_numpy(Q)
    k = torch.from_numpy(np.repeat(K, g, axis=1))
    v = torch.from_numpy(np.repeat(V, g, axis=1))
    mask = torch.from_numpy(visible_mask(np.arange(Sq), Sk, bool(causal), window))
    ok = mask.any(dim=1).numpy()
    ref = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, attn_mask=mask, scale=scale).numpy()
    np.testing.assert_allclose(O[:, :, ok], ref[:, :, ok], rtol=0, atol=1e-12)
    s = torch.matmul(q, k.transpose(-1, -2)) * scale
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1).numpy()
    np.testing.assert_allclose(L[:, :, ok], lse[:, :, ok], rtol=0, atol=1e-12)
    assert np.all(L[:, :, ~ok] == -np.inf)


# ---------------------------------------------------------------- helpers
def test_rows_variant_matches_full():
    rng = np.random.default_rng(14)
    B, H, HKV, Sq, Sk, D = 2, 4, 2, 20, 24, 8
    Q, K, V = _rand((B, H, Sq, D), rng), _rand((B, HKV, Sk, D), rng), _rand((B, HKV, Sk, D), rng)
    O, L = attention(Q, K, V, 0.3, True, 6)
    rows = np.array([[1, 3, 19], [0, 0, 0], [1, 0, 7], [0, 2, 11], [1, 3, 2]])
    Or, Lr = attention_rows(Q, K, V, 0.3, True, 6, rows)
    # equal up to BLAS summation order
    np.testing.assert_allclose(Or, O[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=0, atol=1e-14)
    np.testing.assert_allclose(Lr, L[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=0, atol=1e-14)


@pytest.mark.parametrize("Sq,Sk,causal,window", [
    (10, 10, 0, 0), (10, 10, 1, 0), (10, 4, 1, 0), (4, 10, 1, 0), (16, 16, 1, 5),
    (16, 9, 1, 3), (12, 12, 0, 4)])
def test_visible_count_matches_mask(Sq, Sk, causal, window):
    vis = visible_mask(np.arange(Sq), Sk, bool(causal), window)
    np.testing.assert_array_equal(visible_count(Sq, Sk, bool(causal), window), vis.sum(1))
    # explicit spot checks of the bounds
    if causal and window == 0:
        assert vis[0, 0] and (Sk < 2 or not vis[0, 1])
    if window:
        i = Sq - 1
        lo = i - window + 1
        if 0 <= lo - 1 < Sk:
            assert not vis[i, lo - 1]
        if 0 <= lo < Sk and (not causal or lo <= i):
            assert vis[i, lo]

"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake into a private copy of the oracle's
source (wrong GQA map, causal or window off by one, dropped scale, K used in
place of V, LSE without the max, wrong empty-row LSE, no max shift, missing
normalisation) and asserts that the hand-derived golden fixtures or the
brute-force exact-sum comparison reject the mutant. The real oracle is never
modified."""
import importlib.util
import json
import math
import os
import types

import numpy as np
import pytest

real = importlib.import_module("oracle.attention")

HERE = os.path.dirname(__file__)
with open(os.path.join(HERE, "golden", "closed_forms.json")) as fh:
    CASES = json.load(fh)["cases"]

MUTANTS = [
    ("gqa_map", "hk = h // g                       # GQA head map", "hk = h % HKV"),
    ("causal_off_by_one", "vis &= j <= i", "vis &= j < i"),
    ("window_off_by_one", "vis &= j >= i - window + 1", "vis &= j >= i - window"),
    ("dropped_scale", "S = scale * (Q[b, h] @ K[b, hk].T)", "S = (Q[b, h] @ K[b, hk].T)"),
    ("k_for_v", "_softmax_rows(S, vbh, V[b, hk])", "_softmax_rows(S, vbh, K[b, hk])"),
    ("lse_without_max", "lse[ne] = m[ne] + np.log(l[ne])", "lse[ne] = np.log(l[ne])"),
    ("empty_lse_zero", "lse = np.full(S.shape[0], -np.inf, dtype=np.float64)",
     "lse = np.zeros(S.shape[0], dtype=np.float64)"),
    ("no_max_shift", "P = np.exp(S - m[:, None])", "P = np.exp(S)"),
    ("no_normalise", "O[ne] = (P[ne] @ Vh) / l[ne, None]", "O[ne] = (P[ne] @ Vh)"),
    ("transposed_scores", "S = scale * (Q[b, h] @ K[b, hk].T)", "S = scale * (K[b, hk] @ Q[b, h].T)"),
]

# Block-mask mistakes: rejected by the block-mask brute force.
MASK_MUTANTS = [
    ("mask_axes_swapped", "return mask_bh[(i // block_q)[:, None], (j // block_k)[None, :]] != 0",
     "return mask_bh[(i // block_k)[:, None] % mask_bh.shape[0], (j // block_q)[None, :] % mask_bh.shape[1]] != 0"),
    ("mask_head_shared", "hh = h if mh == H else (hk if mh > 1 else 0)", "hh = 0"),
    ("mask_head_by_q_for_kv", "hh = h if mh == H else (hk if mh > 1 else 0)",
     "hh = h % mh"),
    ("mask_batch_shared", "mb = 0 if block_mask.shape[0] == 1 else b", "mb = 0"),
    ("mask_ignored", "vbh = vis & block_visible(mbh, rows, Sk, block_q, block_k)", "vbh = vis"),
    ("mask_inverted", "vbh = vis & block_visible(mbh, rows, Sk, block_q, block_k)",
     "vbh = vis & ~block_visible(mbh, rows, Sk, block_q, block_k)"),
]


def _load_mutant(old, new):
    src = open(real.__file__).read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _f64(x):
    return np.vectorize(float)(np.array(x, dtype=object)).astype(np.float64)


def _golden_ok(attn):
    for c in CASES:
        try:
            with np.errstate(all="ignore"):
                O, L = attn(_f64(c["Q"]), _f64(c["K"]), _f64(c["V"]), c["scale"],
                            bool(c["causal"]), c["window"])
        except Exception:
            return False
        eO, eL = _f64(c["O"]), _f64(c["LSE"])
        if O.shape != eO.shape or not np.allclose(O, eO, rtol=0, atol=1e-12):
            return False
        fin = np.isfinite(eL)
        if not np.allclose(L[fin], eL[fin], rtol=0, atol=1e-12) or not np.all(L[~fin] == -np.inf):
            return False
    return True


def _brute_ok(attn):
    from test_oracle import _brute  # scalar fsum reference
    rng = np.random.default_rng(99)
    for (B, H, HKV, Sq, Sk, D, causal, window) in [(1, 4, 2, 6, 7, 3, 1, 2), (1, 2, 1, 5, 6, 4, 0, 0)]:
        Q = rng.standard_normal((B, H, Sq, D))
        K = rng.standard_normal((B, HKV, Sk, D))
        V = rng.standard_normal((B, HKV, Sk, D))
        try:
            with np.errstate(all="ignore"):
                O, L = attn(Q, K, V, 0.6, bool(causal), window)
        except Exception:
            return False
        bO, bL = _brute(Q, K, V, 0.6, causal, window)
        if O.shape != bO.shape or not np.allclose(O, bO, rtol=0, atol=1e-12):
            return False
        fin = np.isfinite(bL)
        if not np.allclose(L[fin], bL[fin], rtol=0, atol=1e-12):
            return False
    return True


def test_unmutated_oracle_passes_the_pins():
    assert _golden_ok(real.attention) and _brute_ok(real.attention)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, old, new):
    mod = _load_mutant(old, new)
    assert not (_golden_ok(mod.attention) and _brute_ok(mod.attention)), \
        f"mutant {name} survived every pin"


def _block_ok(attn):
    from test_oracle_block_mask import SHAPES, _brute_masked, _case
    for n, shape in enumerate(SHAPES):
        Q, K, V, causal, window, bm, bq, bk = _case(shape, 50 + n)
        try:
            with np.errstate(all="ignore"):
                O, L = attn(Q, K, V, 0.7, causal, window, block_mask=bm, block_q=bq, block_k=bk)
        except Exception:
            return False
        bO, bL = _brute_masked(Q, K, V, 0.7, causal, window, bm, bq, bk)
        fin = np.isfinite(bL)
        if not np.array_equal(np.isfinite(L), fin):
            return False
        if not np.allclose(O, bO, rtol=0, atol=1e-12) or not np.allclose(L[fin], bL[fin], rtol=0, atol=1e-12):
            return False
    return True


def test_unmutated_oracle_passes_the_block_mask_pins():
    assert _block_ok(real.attention)


@pytest.mark.parametrize("name,old,new", MASK_MUTANTS, ids=[m[0] for m in MASK_MUTANTS])
def test_block_mask_pins_reject_mutant(name, old, new):
    mod = _load_mutant(old, new)
    assert not _block_ok(mod.attention), f"mutant {name} survived the block-mask pins"

"""fp64 CPU oracle for the fused attention forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, links or runs
this module: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` call it. It shares no code with the HIP kernels.

What it computes (the plain definition, not the tiled recurrence):

    O   = softmax(scale * Q K^T + mask) V
    LSE = log(sum_j exp(scale * q_i . k_j))   over the visible keys j

Sources (four web pages on fused attention; cited by page and section):
  * rustytorch ``flash_attention_forward.metal``, kernel
    ``flash_attention_forward``: the operation "O = softmax(Q @ K^T * scale) @ V",
    the dot-then-scale score, the top-left causal test (key index greater
    than query index is skipped), and the per-row log-sum-exp output kept for
    the backward pass.
  * philipturner/metal-flash-attention README, "Modifications to
    FlashAttention": block sparsity with programmable block masks held in
    memory, covering causal and arbitrary sparsity patterns. Here a block
    mask has one byte per (query block, key block); a key is visible only if
    its block's byte is nonzero (on top of the causal and window rules).
  * spb/forge ``src/kernels/flash_attention.metal``, header comment, the
    forward kernel ``flash_attn_fwd`` and the backward kernels
    ``flash_attn_bwd_dq`` / ``_dk`` / ``_dv`` (the gradients below): the online-softmax identity whose
    end result is the plain softmax, the GQA head map hkv = h / (H / HKV),
    the sliding window (keys j >= i - window + 1, self included, 0 = full
    attention), and the stored L = m + log(l).
  * boostr ``flash.wgsl``, ``flash_attention_fwd_f32``: [B, H, S, D] layout,
    separate query/key lengths, the visible key range [start_k, end_k) with
    end_k = min(i + 1, S_k) under causal masking, and the safe (max-shifted)
    softmax evaluated in two passes.

Readings taken where the pages are silent or disagree (each is stated again in
the design notes):
  * a row with no visible key gets O = 0 (every page) and LSE = -inf (the
    rustytorch kernel yields -inf, the boostr shader's comment says "use
    -inf"; forge stores 0);
  * causal masking is top-left aligned (j <= i) also when Sq != Sk;
  * the window without causal is one-sided (only the lower bound applies);
  * inputs are taken exactly as stored (bf16 values upcast exactly), scale is
    the caller's float32 value upcast to fp64.

Pinned by tests/test_oracle.py against closed forms, brute-force exact sums,
invariants and torch's float64 scaled_dot_product_attention.
"""
from __future__ import annotations

import numpy as np


def visible_mask(i: np.ndarray, Sk: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [len(i), Sk]: key j is visible to query row i.

    causal: j <= i (top-left aligned, rustytorch causal test / boostr end_k).
    window > 0: j >= i - window + 1 (forge FlashParams.window, boostr start_k).
    """
    i = np.asarray(i, dtype=np.int64)[:, None]
    j = np.arange(Sk, dtype=np.int64)[None, :]
    vis = np.ones((i.shape[0], Sk), dtype=bool)
    if causal:
        vis &= j <= i
    if window > 0:
        vis &= j >= i - window + 1
    return vis


# Block sizes of the block-mask format (query rows x keys per mask byte).
MASK_BLOCK_Q = 128
MASK_BLOCK_K = 64


def block_visible(mask_bh: np.ndarray, i: np.ndarray, Sk: int, block_q: int = MASK_BLOCK_Q,
                  block_k: int = MASK_BLOCK_K) -> np.ndarray:
    """Boolean [len(i), Sk]: the mask byte of (i // block_q, j // block_k) is
    nonzero. mask_bh is one (batch, head) slice [n_qblocks, n_kblocks]."""
    i = np.asarray(i, dtype=np.int64)
    j = np.arange(Sk, dtype=np.int64)
    return mask_bh[(i // block_q)[:, None], (j // block_k)[None, :]] != 0


def _mask_slice(block_mask, b: int, h: int, hk: int, H: int):
    """The [n_qblocks, n_kblocks] slice a (b, h) row reads: the mask's batch
    axis is 1 (shared) or B, its head axis 1 (shared), HKV (per kv head) or
    H (per query head)."""
    mb = 0 if block_mask.shape[0] == 1 else b
    mh = block_mask.shape[1]
    hh = h if mh == H else (hk if mh > 1 else 0)
    return block_mask[mb, hh]


def _softmax_rows(S: np.ndarray, vis: np.ndarray, Vh: np.ndarray):
    """Masked softmax of score rows S [n, Sk] (fp64) applied to Vh [Sk, D].

    Max-shifted as in boostr's first pass; the shift cancels exactly in the
    ratio, and m + log(l) is the log-sum-exp of the visible scores."""
    S = np.where(vis, S, -np.inf)
    nonempty = vis.any(axis=1)
    m = np.where(nonempty, S.max(axis=1, initial=-np.inf), 0.0)
    P = np.exp(S - m[:, None])                 # masked entries -> exp(-inf) = 0
    l = P.sum(axis=1)
    O = np.zeros((S.shape[0], Vh.shape[1]), dtype=np.float64)
    lse = np.full(S.shape[0], -np.inf, dtype=np.float64)
    if nonempty.any():
        ne = nonempty
        O[ne] = (P[ne] @ Vh) / l[ne, None]
        lse[ne] = m[ne] + np.log(l[ne])
        # Internal consistency: every normalised softmax row sums to 1 and the
        # max term alone contributes exp(0) = 1 to l.
        rs = (P[ne] / l[ne, None]).sum(axis=1)
        assert np.all(np.abs(rs - 1.0) <= 1e-12), "softmax row does not sum to 1"
        assert np.all(l[ne] >= 1.0), "row sum below the max term"
    return O, lse


def attention(Q, K, V, scale: float, causal: bool = False, window: int = 0,
              block_mask=None, block_q: int = MASK_BLOCK_Q, block_k: int = MASK_BLOCK_K):
    """Full forward: returns (O [B,H,Sq,D] fp64, LSE [B,H,Sq] fp64).

    block_mask: None, or [1 or B, 1 or HKV or H, ceil(Sq/block_q),
    ceil(Sk/block_k)] of which nonzero entries mark visible blocks.
    Materialises the full Sq x Sk score matrix for one (b, h) at a time."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, H, Sq, D = Q.shape
    HKV, Sk = K.shape[1], K.shape[2]
    assert H % HKV == 0, "H must be a multiple of HKV"
    g = H // HKV
    scale = float(np.float64(scale))
    O = np.zeros((B, H, Sq, D), dtype=np.float64)
    LSE = np.zeros((B, H, Sq), dtype=np.float64)
    rows = np.arange(Sq)
    vis = visible_mask(rows, Sk, causal, window)
    for b in range(B):
        for h in range(H):
            hk = h // g                       # GQA head map
            S = scale * (Q[b, h] @ K[b, hk].T)
            vbh = vis
            if block_mask is not None:
                mbh = _mask_slice(block_mask, b, h, hk, H)
                vbh = vis & block_visible(mbh, rows, Sk, block_q, block_k)
            O[b, h], LSE[b, h] = _softmax_rows(S, vbh, V[b, hk])
    return O, LSE


def attention_rows(Q, K, V, scale: float, causal: bool, window: int, rows, block_mask=None,
                   block_q: int = MASK_BLOCK_Q, block_k: int = MASK_BLOCK_K):
    """Forward for selected query rows only (block_mask as in ``attention``).

    rows: int array [n, 3] of (b, h, i). Returns (O [n, D], LSE [n]) in the
    order given. Materialises the score rows [n_bh, Sk] per (b, h)."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    H = Q.shape[1]
    HKV, Sk, D = K.shape[1], K.shape[2], K.shape[3]
    assert H % HKV == 0
    g = H // HKV
    scale = float(np.float64(scale))
    O = np.zeros((rows.shape[0], D), dtype=np.float64)
    LSE = np.zeros(rows.shape[0], dtype=np.float64)
    key = rows[:, 0] * H + rows[:, 1]
    for bh in np.unique(key):
        sel = np.nonzero(key == bh)[0]
        b, h = int(bh // H), int(bh % H)
        hk = h // g
        ii = rows[sel, 2]
        q = np.asarray(Q[b, h, ii], dtype=np.float64)
        Kh = np.asarray(K[b, hk], dtype=np.float64)
        Vh = np.asarray(V[b, hk], dtype=np.float64)
        S = scale * (q @ Kh.T)
        vis = visible_mask(ii, Sk, causal, window)
        if block_mask is not None:
            vis = vis & block_visible(_mask_slice(block_mask, b, h, hk, H), ii, Sk, block_q,
                                      block_k)
        O[sel], LSE[sel] = _softmax_rows(S, vis, Vh)
    return O, LSE


def visible_count(Sq: int, Sk: int, causal: bool, window: int) -> np.ndarray:
    """|visible(i)| for every query row i (int64 [Sq])."""
    i = np.arange(Sq, dtype=np.int64)
    hi = np.minimum(i + 1, Sk) if causal else np.full(Sq, Sk, dtype=np.int64)
    lo = np.maximum(i - window + 1, 0) if window > 0 else np.zeros(Sq, dtype=np.int64)
    return np.maximum(hi - lo, 0)


def attention_backward(Q, K, V, dO, scale: float, causal: bool = False, window: int = 0,
                       block_mask=None, block_q: int = MASK_BLOCK_Q, block_k: int = MASK_BLOCK_K):
    """Gradients (dQ, dK, dV) of L = sum(O * dO), all fp64, for O = attention(...)
    with the same arguments (block_mask, block_q, block_k as in ``attention``:
    a key is visible only where the causal and window rules and the mask's
    block byte all allow it; masked pairs have P = 0 and get no gradient).

    From the definition (forge ``flash_attention.metal`` backward section): with
    P the masked softmax of scale * Q K^T (P_ij = exp(s_ij - LSE_i) on the
    visible keys, 0 elsewhere),
        dV_j  = sum_i P_ij dO_i
        dP_ij = dO_i . V_j
        D_i   = dO_i . O_i               (= sum_j P_ij dP_ij)
        dS_ij = P_ij (dP_ij - D_i)
        dQ_i  = scale sum_j dS_ij K_j
        dK_j  = scale sum_i dS_ij Q_i
    with dK and dV summed over the query heads that share a kv head (GQA).
    Rows with no visible key have P = 0: they contribute nothing and get dQ = 0.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, H, Sq, D = Q.shape
    HKV, Sk = K.shape[1], K.shape[2]
    assert H % HKV == 0, "H must be a multiple of HKV"
    g = H // HKV
    scale = float(np.float64(scale))
    rows = np.arange(Sq)
    vis_rule = visible_mask(rows, Sk, causal, window)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        for h in range(H):
            hk = h // g
            vis = vis_rule
            if block_mask is not None:
                vis = vis_rule & block_visible(_mask_slice(block_mask, b, h, hk, H), rows, Sk,
                                               block_q, block_k)
            nonempty = vis.any(axis=1)
            S = np.where(vis, scale * (Q[b, h] @ K[b, hk].T), -np.inf)
            m = np.where(nonempty, S.max(axis=1, initial=-np.inf), 0.0)
            E = np.exp(S - m[:, None])
            l = E.sum(axis=1)
            P = np.zeros_like(E)
            P[nonempty] = E[nonempty] / l[nonempty, None]
            O = P @ V[b, hk]
            dP = dO[b, h] @ V[b, hk].T
            Drow = (dO[b, h] * O).sum(axis=1)
            dS = P * (dP - Drow[:, None])
            dQ[b, h] = scale * (dS @ K[b, hk])
            dK[b, hk] += scale * (dS.T @ Q[b, h])
            dV[b, hk] += P.T @ dO[b, h]
    return dQ, dK, dV

"""Seeded synthetic workloads for the fused attention forward pass.

This module only *generates inputs*: shapes, seeded random tensors, bf16
rounding of the drawn values, and seeded samples of which query rows a check
looks at. It holds none of the attention arithmetic, so both the fp64 oracle
(under ``oracle/``) and the GPU path can consume the same buffers without
sharing any code of the method.

Workload shapes follow the five synthetic configurations of the benchmark
(small reference case, fp32 causal MHA, bf16 causal GQA, fp32 sliding-window
GQA, bf16 long non-square single head), plus the causal GQA shape with fp16
inputs (mixed precision, the "Support mixed precision" item of the
metal-flash-attention README's TODO list), with token-major [B, S, H, D]
storage (the layout of the forge flash_attention.metal kernels), and
non-causal under a block mask (the block sparsity of the metal-flash-attention
README's "Modifications to FlashAttention"; recipe in make_block_mask). Layout is [B, H, S, D] contiguous for
Q and O, [B, HKV, S, D] for K and V, as in the boostr ``flash.wgsl`` header
comment and the rustytorch ``flash_attention_forward.metal`` buffer comments.

Recipe (stated once, used everywhere):
  * generator: ``numpy.random.default_rng`` on a ``SeedSequence(seed)`` spawned
    into four independent streams (Q, K, V, row sample);
  * seed = 20261202 + config index (0-based);
  * values are drawn in float32; for bf16 and fp16 workloads they are rounded
    to the nearest bf16 / fp16 value (ties to even) and both sides read the
    rounded values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np

BASE_SEED = 20261202


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    HKV: int
    Sq: int
    Sk: int
    D: int
    dtype: str            # "f32", "bf16" or "f16"
    causal: int
    window: int
    q_dist: str = "normal"     # "normal" | "uniform"
    k_dist: str = "normal"
    v_dist: str = "normal"
    amplitude: float = 1.0      # multiplies every drawn value (before rounding)
    check: str = "all"          # "all" | "sampled"
    n_random_rows: int = 0      # for "sampled": distinct (b,h,i) drawn uniformly
    edge_rows: int = 0          # for "sampled": first/last rows of every (b,h)
    seed_index: int = 0
    layout: str = "bhsd"        # device storage: "bhsd" contiguous [B, heads, S, D], or
                                # "bshd" token-major [B, S, heads, D] (viewed as [B, heads, S, D])
    mask: str = ""              # "" (none) or "band_random": a block mask, see make_block_mask
    mask_p: float = 0.0         # "band_random": probability of each extra random block

    @property
    def group(self) -> int:
        return self.H // self.HKV

    @property
    def seed(self) -> int:
        return BASE_SEED + self.seed_index

    def scale(self) -> float:
        """1/sqrt(D) rounded to float32 (the value both sides use)."""
        return float(np.float32(1.0 / math.sqrt(self.D)))


CONFIGS = [
    Workload("tiny_f32_128", 1, 1, 1, 128, 128, 64, "f32", 0, 0,
             check="all", seed_index=0),
    Workload("mha_causal_f32_b4h8_s1024_d64", 4, 8, 8, 1024, 1024, 64, "f32", 1, 0,
             check="all", seed_index=1),
    Workload("gqa_causal_bf16_b2h32kv8_s4096_d128", 2, 32, 8, 4096, 4096, 128, "bf16", 1, 0,
             amplitude=0.5, check="all", seed_index=2),
    Workload("swa_gqa_f32_b1h16kv4_s16384_d128_w4096", 1, 16, 4, 16384, 16384, 128, "f32", 1, 4096,
             check="sampled", n_random_rows=512, edge_rows=64, seed_index=3),
    Workload("long_bf16_sq8192_sk65536_d256", 1, 1, 1, 8192, 65536, 256, "bf16", 0, 0,
             v_dist="uniform", check="sampled", n_random_rows=256, edge_rows=0,
             seed_index=4),
    Workload("gqa_causal_f16_b2h32kv8_s4096_d128", 2, 32, 8, 4096, 4096, 128, "f16", 1, 0,
             amplitude=0.5, check="all", seed_index=5),
    Workload("gqa_causal_bf16_bshd_b2h32kv8_s4096_d128", 2, 32, 8, 4096, 4096, 128, "bf16", 1,
             0, amplitude=0.5, check="all", seed_index=6, layout="bshd"),
    Workload("blocksparse_bf16_b2h32kv8_s4096_d128", 2, 32, 8, 4096, 4096, 128, "bf16", 0, 0,
             amplitude=0.5, check="all", seed_index=7, mask="band_random", mask_p=0.15),
    # head dims below the kernel tiles (the padded form): the bf16 headline
    # shape at D = 96 and the fp32 causal MHA shape at D = 32
    Workload("gqa_causal_bf16_b2h32kv8_s4096_d96", 2, 32, 8, 4096, 4096, 96, "bf16", 1, 0,
             amplitude=0.5, check="all", seed_index=8),
    Workload("mha_causal_f32_b4h8_s1024_d32", 4, 8, 8, 1024, 1024, 32, "f32", 1, 0,
             check="all", seed_index=9),
    # fp32 at head dim 256 (the backward's wavefront-pair split of the dims)
    Workload("mha_causal_f32_b1h16_s4096_d256", 1, 16, 16, 4096, 4096, 256, "f32", 1, 0,
             check="sampled", n_random_rows=256, edge_rows=64, seed_index=10),
]

# Block-mask granularity (query rows x keys per mask byte).
MASK_BLOCK_Q = 128
MASK_BLOCK_K = 64

# The configuration the throughput metric is quoted on (bf16 causal GQA).
HEADLINE = 2


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round to nearest, ties to even.

    Inputs here are finite, so no NaN special case is needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert np.all(np.isfinite(x)), "bf16 rounding expects finite inputs"
    # For finite inputs u + 0x8000 stays below 2**32, so uint32 arithmetic is exact.
    r = u + np.uint32(0x7FFF)
    r += (u >> np.uint32(16)) & np.uint32(1)
    return (r >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 IEEE half bit patterns, round to nearest, ties to
    even (numpy's float32 -> float16 conversion). Inputs must lie inside the
    half range."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert np.all(np.abs(x) <= 65504.0), "fp16 rounding expects inputs inside the half range"
    return x.astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return bits.view(np.float16).astype(np.float32)


# 16-bit input types: (float32 -> bits, bits -> float32)
ROUNDING = {"bf16": (round_to_bf16_bits, bf16_bits_to_f32),
            "f16": (round_to_f16_bits, f16_bits_to_f32)}


def _draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    raise ValueError(dist)


@dataclass
class Inputs:
    """Host copies of one workload's inputs.

    ``q``/``k``/``v`` are float32 arrays holding exactly the values the GPU
    reads (for 16-bit workloads they are the rounded values); ``*_bits`` are
    the bf16 / fp16 bit patterns (uint16) for 16-bit workloads, else None."""
    wl: Workload
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    q_bits: np.ndarray | None = None
    k_bits: np.ndarray | None = None
    v_bits: np.ndarray | None = None
    rows_rng: np.random.Generator | None = field(default=None, repr=False)
    block_mask: np.ndarray | None = None     # uint8 [1, HKV, nqb, nkb] for masked workloads


def make_inputs(wl: Workload, seed: int | None = None) -> Inputs:
    seed = wl.seed if seed is None else seed
    sq, sk, sv, srow = np.random.SeedSequence(seed).spawn(4)
    q = _draw(np.random.default_rng(sq), (wl.B, wl.H, wl.Sq, wl.D), wl.q_dist)
    k = _draw(np.random.default_rng(sk), (wl.B, wl.HKV, wl.Sk, wl.D), wl.k_dist)
    v = _draw(np.random.default_rng(sv), (wl.B, wl.HKV, wl.Sk, wl.D), wl.v_dist)
    if wl.amplitude != 1.0:
        a = np.float32(wl.amplitude)
        q, k, v = q * a, k * a, v * a
    out = Inputs(wl, q, k, v, rows_rng=np.random.default_rng(srow))
    if wl.mask:
        out.block_mask = make_block_mask(wl, np.random.default_rng(
            np.random.SeedSequence(seed).spawn(5)[4]))
    if wl.dtype in ROUNDING:
        to_bits, to_f32 = ROUNDING[wl.dtype]
        out.q_bits, out.k_bits, out.v_bits = to_bits(q), to_bits(k), to_bits(v)
        out.q, out.k, out.v = to_f32(out.q_bits), to_f32(out.k_bits), to_f32(out.v_bits)
    return out


def make_block_mask(wl: Workload, rng: np.random.Generator) -> np.ndarray:
    """Seeded block mask [1, HKV, nqb, nkb] (uint8), one per kv head, shared
    over the batch. "band_random": query block r (rows 128 r ..) sees the key
    blocks of its own rows and the two before them (c in [2r - 2, 2r + 1], a
    local band), key block 0 (a global prefix), and each other block with
    probability mask_p."""
    assert wl.mask == "band_random", wl.mask
    nqb = -(-wl.Sq // MASK_BLOCK_Q)
    nkb = -(-wl.Sk // MASK_BLOCK_K)
    r = np.arange(nqb)[:, None]
    c = np.arange(nkb)[None, :]
    per = MASK_BLOCK_Q // MASK_BLOCK_K
    band = (c >= per * r - 2) & (c <= per * r + per - 1)
    base = band | (c == 0)
    extra = rng.random((1, wl.HKV, nqb, nkb)) < wl.mask_p
    return (base[None, None] | extra).astype(np.uint8)


def make_grad_output(inp: Inputs):
    """Seeded gradient of the loss with respect to O (same shape as Q), for
    the backward pass: N(0, 1) drawn in float32 from a sixth stream of the
    workload's seed, rounded like the inputs for 16-bit workloads. Returns
    (values as float32, bits or None)."""
    wl = inp.wl
    rng = np.random.default_rng(np.random.SeedSequence(wl.seed).spawn(6)[5])
    g = rng.standard_normal((wl.B, wl.H, wl.Sq, wl.D), dtype=np.float32)
    if wl.dtype in ROUNDING:
        to_bits, to_f32 = ROUNDING[wl.dtype]
        bits = to_bits(g)
        return to_f32(bits), bits
    return g, None


def device_mask(inp: Inputs, torch, device="cuda"):
    """The workload's block mask on `device`, or None."""
    if inp.block_mask is None:
        return None
    return torch.from_numpy(inp.block_mask).to(device)


def check_rows(inp: Inputs) -> np.ndarray | None:
    """Rows (b, h, i) a parity check compares, as an int64 array [n, 3].

    None means every row. For "sampled" workloads: ``n_random_rows`` distinct
    rows drawn uniformly from all B*H*Sq rows, united with the first and last
    ``edge_rows`` rows of every (b, h)."""
    wl = inp.wl
    if wl.check == "all":
        return None
    rng = inp.rows_rng if inp.rows_rng is not None else np.random.default_rng(wl.seed)
    total = wl.B * wl.H * wl.Sq
    pick = rng.choice(total, size=min(wl.n_random_rows, total), replace=False)
    flat = set(int(x) for x in pick)
    if wl.edge_rows:
        e = min(wl.edge_rows, wl.Sq)
        for bh in range(wl.B * wl.H):
            for i in list(range(e)) + list(range(wl.Sq - e, wl.Sq)):
                flat.add(bh * wl.Sq + i)
    flat = np.array(sorted(flat), dtype=np.int64)
    b = flat // (wl.H * wl.Sq)
    h = (flat // wl.Sq) % wl.H
    i = flat % wl.Sq
    return np.stack([b, h, i], axis=1)


def small(wl: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (for reduced-size tests)."""
    return replace(wl, **kw)


def device_tensors(inp: Inputs, torch, device="cuda"):
    """(q, k, v) as torch tensors on `device` holding exactly the workload's
    values, shaped [B, heads, S, D]. "bshd" workloads are stored token-major
    and handed over as the [B, heads, S, D] view of that storage."""
    wl = inp.wl
    if wl.dtype in ROUNDING:
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float16
        arrs = [inp.q_bits.view(np.int16), inp.k_bits.view(np.int16), inp.v_bits.view(np.int16)]
    else:
        tdt = None
        arrs = [inp.q, inp.k, inp.v]
    out = []
    for a in arrs:
        if wl.layout == "bshd":
            a = np.ascontiguousarray(a.transpose(0, 2, 1, 3))
        t = torch.from_numpy(a)
        if tdt is not None:
            t = t.view(tdt)
        t = t.to(device)
        out.append(t.transpose(1, 2) if wl.layout == "bshd" else t)
    return tuple(out)

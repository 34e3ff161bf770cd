"""Host-only checks of the backward's launch plan (fa_bwd_plan): the tile
head dim, how inputs reach the kernels, and the small-grid chunks of the key
axis (dQ) and the query rows (dK/dV). No GPU: the plan is pure host logic,
and the partial sums it implies are checked for exactness against the oracle
by the chunked cases of the GPU backward tests."""
import ctypes

import numpy as np
import pytest

import attention_forward_online_fa_amd as fa
from attention_forward_online_fa_amd._lib import lib

CUS = 256   # MI355X compute units


def test_headline_shapes():
    # bf16 GQA causal B2 H32/8 S4096 D128: 2048 dQ tiles and 512 dK/dV blocks
    # fill 256 CUs, so no chunks
    p = fa.bwd_plan(2, 32, 8, 4096, 4096, 128, CUS, causal=True)
    assert p == dict(head_dim=128, general=0, staged=0, per_row=0, key_chunks=1,
                     keys_per_chunk=0, row_chunks=1, rows_per_chunk=4096)
    # fp32 B4 H8 S1024 D64 causal: 256 dQ tiles (< 2 per CU) -> 2 key chunks of
    # 16 tiles; 256 dK/dV blocks against 1024 fp32 slots -> 4 row chunks
    p = fa.bwd_plan(4, 8, 8, 1024, 1024, 64, CUS, causal=True, dtype="f32")
    assert (p["key_chunks"], p["keys_per_chunk"]) == (2, 512)
    assert (p["row_chunks"], p["rows_per_chunk"]) == (4, 256)
    assert p["per_row"] == 0 and p["staged"] == 0


def test_head_dim_routes():
    # 16-bit D 96 runs the 128 tile's general form in place
    p = fa.bwd_plan(1, 2, 1, 300, 300, 96, CUS)
    assert (p["head_dim"], p["general"], p["staged"]) == (128, 1, 0)
    # fp32 D 48: staged into the 64 tile when the work is large (B H pairs >= 2^23) ...
    p = fa.bwd_plan(4, 8, 8, 1024, 1024, 48, CUS, dtype="f32")
    assert (p["head_dim"], p["staged"], p["per_row"]) == (64, 1, 0)
    # ... the per-row kernels when it is small
    p = fa.bwd_plan(1, 1, 1, 256, 256, 48, CUS, dtype="f32")
    assert (p["head_dim"], p["staged"], p["per_row"]) == (48, 0, 1)
    # D 256 runs MFMA kernels for every type (fp32: the dims split over
    # wavefront pairs; only a block mask keeps fp32 D 256 on the per-row kernels)
    assert fa.bwd_plan(8, 16, 16, 4096, 4096, 256, CUS, dtype="f32")["per_row"] == 0
    assert fa.bwd_plan(1, 1, 1, 128, 128, 256, CUS, dtype="f32")["per_row"] == 0
    assert fa.bwd_plan(1, 1, 1, 128, 128, 256, CUS, dtype="bf16")["per_row"] == 0


def test_fp32_d256_chunks_count_64_row_workgroups():
    # 64 query rows (keys) per workgroup: B1 H4 S2048 has 128 dQ workgroups
    # (< 512) -> key chunks; 128 dK/dV workgroups against 512 fp32 slots and
    # a walk of 2048 rows -> 4 row chunks of 512 rows
    p = fa.bwd_plan(1, 4, 4, 2048, 2048, 256, CUS, causal=True, dtype="f32")
    assert p["per_row"] == 0 and p["head_dim"] == 256
    assert (p["key_chunks"], p["keys_per_chunk"]) == (4, 512)
    assert (p["row_chunks"], p["rows_per_chunk"]) == (4, 512)


def test_big_grid_has_no_chunks_small_grid_has():
    big = fa.bwd_plan(1, 8, 8, 2048, 2048, 128, 1)
    assert big["key_chunks"] == 1 and big["row_chunks"] == 1
    small = fa.bwd_plan(1, 8, 8, 2048, 2048, 128, CUS)
    assert small["key_chunks"] == 4 and small["row_chunks"] == 2
    # short walks (Sq H/HKV < 2048 for 16-bit) keep whole rows
    assert fa.bwd_plan(1, 8, 8, 1024, 1024, 128, CUS)["row_chunks"] == 1


def _span(p, Sq, Sk, causal, window):
    band = causal and window > 0
    return (min(Sk, window) if band else Sk), (min(Sq, window) if band else Sq)


@pytest.mark.parametrize("seed", range(40))
def test_random_plans_cover_the_axes(seed):
    rng = np.random.default_rng(seed)
    dtype = ["f32", "bf16", "f16"][seed % 3]
    D = int(rng.choice([16, 32, 48, 64, 80, 96, 128, 256]))
    HKV = int(rng.integers(1, 9))
    H = HKV * int(rng.choice([1, 2, 4]))
    B = int(rng.integers(1, 4))
    Sq, Sk = (int(x) for x in rng.integers(1, 9000, size=2))
    causal = int(rng.integers(0, 2))
    window = int(rng.choice([0, 0, 100, 3000]))
    p = fa.bwd_plan(B, H, HKV, Sq, Sk, D, CUS, causal=bool(causal), window=window, dtype=dtype)
    assert p["head_dim"] >= D
    if dtype != "f32":
        assert p["per_row"] == 0 and p["staged"] == 0
        assert p["general"] == int(p["head_dim"] != D)
    if p["per_row"]:
        assert 1 <= p["key_chunks"] <= 8 and p["row_chunks"] == 1
        sq, sk = _span(p, Sq, Sk, causal, window)
        assert p["key_chunks"] * p["keys_per_chunk"] >= sq
    else:
        assert 1 <= p["key_chunks"] <= 16
        if p["key_chunks"] > 1:   # whole 32-key tiles, every chunk non-empty
            c = p["keys_per_chunk"]
            assert c % 32 == 0 and (p["key_chunks"] - 1) * c < Sk <= p["key_chunks"] * c
        assert 1 <= p["row_chunks"] <= 8
        if p["row_chunks"] > 1:   # whole 128-row blocks, every chunk non-empty
            r = p["rows_per_chunk"]
            assert r % 128 == 0 and (p["row_chunks"] - 1) * r < Sq <= p["row_chunks"] * r
        else:
            assert p["rows_per_chunk"] == Sq
        # partial-sum workspaces stay at most 512 MiB
        DT = p["head_dim"]
        if p["key_chunks"] > 1:
            assert p["key_chunks"] * B * H * Sq * DT * 4 <= 512 << 20
        if p["row_chunks"] > 1:
            assert 2 * p["row_chunks"] * B * HKV * Sk * DT * 4 <= 512 << 20


def test_plan_argument_errors():
    buf = (ctypes.c_int * 8)()
    ptr = ctypes.cast(buf, ctypes.c_void_p)
    L = lib()
    assert L.fa_bwd_plan(1, 4, 4, 64, 64, 64, 0, 0, 1, 256, None) == 1    # FA_ERR_NULLPTR
    assert L.fa_bwd_plan(1, 4, 4, 64, 64, 64, 0, 0, 1, 0, ptr) == 2      # num_cus < 1
    assert L.fa_bwd_plan(1, 4, 3, 64, 64, 64, 0, 0, 1, 256, ptr) == 3    # FA_ERR_GQA
    assert L.fa_bwd_plan(1, 4, 4, 64, 64, 40, 0, 0, 1, 256, ptr) == 4    # FA_ERR_HEAD_DIM
    assert L.fa_bwd_plan(1, 4, 4, 64, 64, 64, 0, 0, 7, 256, ptr) == 5    # FA_ERR_DTYPE
    assert L.fa_bwd_plan(1, 4, 4, 64, 64, 64, 2, 0, 1, 256, ptr) == 6    # FA_ERR_WINDOW
    with pytest.raises(fa.FaError):
        fa.bwd_plan(1, 4, 4, 64, 64, 64, 0)

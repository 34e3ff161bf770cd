"""Seeded input generation: bf16 rounding, determinism, row sampling. CPU only."""
import numpy as np

import workloads as W


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)          # bf16 spacing at 1.0
    x = np.array([1.0,
                  one + ulp / 2,          # tie -> even (1.0)
                  one + ulp + ulp / 2,    # tie -> even (1 + 2 ulp)
                  one + ulp / 2 + np.float32(2.0 ** -20),   # just above tie -> up
                  -2.5, 3.0e-3, 65504.0], dtype=np.float32)
    bits = W.round_to_bf16_bits(x)
    assert bits[0] == 0x3F80
    assert bits[1] == 0x3F80
    assert bits[2] == 0x3F82
    assert bits[3] == 0x3F81
    assert bits[4] == 0xC020
    back = W.bf16_bits_to_f32(bits)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)


def test_inputs_are_deterministic_and_rounded():
    wl = W.small(W.CONFIGS[2], B=1, H=4, HKV=1, Sq=64, Sk=64)
    a, b = W.make_inputs(wl), W.make_inputs(wl)
    np.testing.assert_array_equal(a.q, b.q)
    np.testing.assert_array_equal(a.v_bits, b.v_bits)
    np.testing.assert_array_equal(W.bf16_bits_to_f32(a.k_bits), a.k)
    assert a.q.shape == (1, 4, 64, 128) and a.k.shape == (1, 1, 64, 128)
    # amplitude 0.5 N(0,1): sample std near 0.5
    assert 0.45 < float(a.q.std()) < 0.55


def test_uniform_v_range():
    wl = W.small(W.CONFIGS[4], Sq=16, Sk=512)
    inp = W.make_inputs(wl)
    assert inp.v.min() >= -1.0 and inp.v.max() <= 1.0 and inp.v.std() > 0.5


def test_sampled_rows_union_of_random_and_edges():
    wl = W.small(W.CONFIGS[3], Sq=512, Sk=512, n_random_rows=40, edge_rows=8)
    rows = W.check_rows(W.make_inputs(wl))
    assert rows.shape[1] == 3
    keys = {tuple(r) for r in rows.tolist()}
    assert len(keys) == len(rows)
    for h in range(wl.H):
        assert (0, h, 0) in keys and (0, h, 511) in keys and (0, h, 7) in keys
    assert len(rows) <= 40 + wl.H * 16
    assert W.check_rows(W.make_inputs(W.CONFIGS[0])) is None


def test_f16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -10)         # fp16 spacing at 1.0
    x = np.array([1.0,
                  one + ulp / 2,          # tie -> even (1.0)
                  one + ulp + ulp / 2,    # tie -> even (1 + 2 ulp)
                  one + ulp / 2 + np.float32(2.0 ** -20),   # just above tie -> up
                  -2.5, 65504.0, 2.0 ** -24], dtype=np.float32)
    bits = W.round_to_f16_bits(x)
    assert bits[0] == 0x3C00
    assert bits[1] == 0x3C00
    assert bits[2] == 0x3C02
    assert bits[3] == 0x3C01
    assert bits[4] == 0xC100
    assert bits[5] == 0x7BFF
    assert bits[6] == 0x0001               # smallest subnormal
    back = W.f16_bits_to_f32(bits)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -11)


def test_f16_workload_inputs_are_rounded():
    wl = W.small(W.CONFIGS[5], B=1, H=4, HKV=1, Sq=64, Sk=64)
    assert wl.dtype == "f16"
    a = W.make_inputs(wl)
    np.testing.assert_array_equal(W.f16_bits_to_f32(a.q_bits), a.q)
    np.testing.assert_array_equal(a.k.astype(np.float16).astype(np.float32), a.k)


def test_device_tensors_token_major_view():
    import torch
    wl = W.small(W.CONFIGS[6], B=2, H=4, HKV=2, Sq=16, Sk=24)
    assert wl.layout == "bshd"
    inp = W.make_inputs(wl)
    q, k, v = W.device_tensors(inp, torch, "cpu")
    assert q.shape == (2, 4, 16, 128) and k.shape == (2, 2, 24, 128)
    assert q.stride() == (16 * 4 * 128, 128, 4 * 128, 1)      # storage [B, S, H, D]
    assert k.stride() == (24 * 2 * 128, 128, 2 * 128, 1)
    np.testing.assert_array_equal(q.float().numpy(), inp.q)
    np.testing.assert_array_equal(v.float().numpy(), inp.v)
    c = W.device_tensors(W.make_inputs(W.small(wl, layout="bhsd")), torch, "cpu")
    assert c[0].is_contiguous() and torch.equal(c[0], q)


def test_block_mask_recipe():
    wl = W.CONFIGS[7]
    assert wl.mask == "band_random" and not wl.causal
    small = W.small(wl, B=1, H=4, HKV=2, Sq=1000, Sk=1300)
    a, b = W.make_inputs(small), W.make_inputs(small)
    np.testing.assert_array_equal(a.block_mask, b.block_mask)
    m = a.block_mask
    assert m.shape == (1, 2, 8, 21) and m.dtype == np.uint8
    for r in range(8):
        assert np.all(m[0, :, r, 0] == 1)                           # global block
        for c in range(max(0, 2 * r - 2), min(21, 2 * r + 2)):
            assert np.all(m[0, :, r, c] == 1)                       # local band
    assert 0.1 < float(m.mean()) < 0.6
    # the full-size mask: density near band + global + 15 % random
    full = W.make_inputs(W.small(wl, B=1, H=8, HKV=8, Sq=4096, Sk=4096)).block_mask
    assert 0.15 < float(full.mean()) < 0.3


def test_bench_counted_flops_match_oracle_masks():
    # bench.py's closed-form per-row counts against the oracle's own masks
    import importlib.util
    import os
    from oracle import block_visible, visible_mask
    spec = importlib.util.spec_from_file_location(
        "bench", os.path.join(os.path.dirname(os.path.dirname(__file__)), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    for causal, window in [(0, 0), (1, 0), (1, 150), (0, 300)]:
        wl = W.small(W.CONFIGS[7], B=2, H=4, HKV=2, Sq=700, Sk=900, causal=causal,
                     window=window)
        inp = W.make_inputs(wl)
        i = np.arange(wl.Sq)
        want = 0
        for b in range(wl.B):
            for h in range(wl.H):
                vis = visible_mask(i, wl.Sk, bool(causal), window)
                vis &= block_visible(inp.block_mask[0, h // 2], i, wl.Sk)
                want += int(vis.sum())
        assert bench.counted_flops(wl, inp.block_mask) == 4.0 * wl.D * want
        plain = int(visible_mask(i, wl.Sk, bool(causal), window).sum()) * wl.B * wl.H
        assert bench.counted_flops(wl) == 4.0 * wl.D * plain

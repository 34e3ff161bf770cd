"""Calls on two streams at once. Each call takes its workspace (the forward's
key-split partials, the backward's D_i and chunk partials) stream-ordered from
the library's memory pool on the caller's stream, and the persistent schedules
are uploaded synchronously, so calls in flight on different streams must not
disturb each other: every result of forward + backward pairs interleaved on two
non-default streams, with no synchronization between the streams, equals the
same calls run alone bit for bit (the kernels are deterministic)."""
import pytest

import workloads as W
from test_parity import to_device, wl_small

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = [
    # forced key splits in the forward; dK/dV row chunks in the backward
    wl_small("bf16", 1, 8, 2, 1100, 1100, 128, 1, 0, seed=61),
    # fp32: dQ key chunks and dK/dV row chunks, a persistent-capable small grid
    wl_small("f32", 1, 4, 1, 700, 2600, 64, 1, 0, seed=62),
]


def _run(fa, x, wl):
    q, k, v, do = x
    o, lse = fa.fwd(q, k, v, causal=bool(wl.causal), window=wl.window, scale=wl.scale(),
                    num_splits=3)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=bool(wl.causal), window=wl.window,
                        scale=wl.scale())
    return o, lse, dq, dk, dv


def test_two_streams_match_calls_alone():
    import attention_forward_online_fa_amd as fa
    torch.manual_seed(5)
    inputs = []
    for wl in CASES:
        q, k, v = to_device(W.make_inputs(wl))
        inputs.append((q, k, v, torch.randn_like(q)))
    print("[streams] calls alone", flush=True)
    alone = [_run(fa, x, wl) for x, wl in zip(inputs, CASES)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    got = [[], []]
    print("[streams] interleaved on two streams", flush=True)
    for _ in range(3):
        for i, (s, x, wl) in enumerate(zip(streams, inputs, CASES)):
            with torch.cuda.stream(s):
                got[i].append(_run(fa, x, wl))
    torch.cuda.synchronize()
    for i in range(len(CASES)):
        for rep, r in enumerate(got[i]):
            for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), r, alone[i]):
                assert torch.equal(a, b), f"case {i} call {rep}: {name} differs"

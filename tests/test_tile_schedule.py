"""CPU model of the bf16 kernel's key-tile loop (host-side logic only, no GPU).

The kernel walks the key tiles of a (query block, split) in pairs. Pairs whose
two tiles are visible to every row of the block, and whose copied tiles (the
next ones) hold a full tile of keys below Sk, run a step without skip, mask or
bounds decisions; the other pairs run the general step. This model restates
that split from the kernel's integer definitions and checks, over fixed and
random shapes, that the steps cover every tile once in order and that no
interior step sees a masked key or copies a partial tile (which would read
rows past the end of K and V)."""
import random

import pytest

BM = 128


def key_range(Sq, Sk, causal, window, q0, nsplit, split_len, split):
    lo, hi = 0, Sk
    if causal:
        hi = min(hi, q0 + BM)
    if window > 0:
        lo = max(lo, q0 - window + 1)
    if nsplit > 1:
        lo = max(lo, split * split_len)
        hi = min(hi, (split + 1) * split_len)
    return lo, hi


def schedule(n, u_lo, u_hi, full_hi):
    in2 = lambda t: t >= u_lo and t + 1 < u_hi and t + 2 < full_hi
    steps, t, done = [], 0, n == 0

    def gen2(t):
        steps.append(("general", t))
        if t + 1 >= n:
            return True
        steps.append(("general", t + 1))
        return t + 2 >= n

    while not done and not in2(t):
        done = gen2(t)
        t += 2
    while not done and in2(t):
        steps += [("interior", t), ("interior", t + 1)]
        t += 2
    while not done:
        done = gen2(t)
        t += 2
    return steps


def check_shape(Sq, Sk, causal, window, BN, nsplit, sched=None):
    sched = sched or schedule
    sk_tiles = (Sk + BN - 1) // BN
    ns = min(nsplit, sk_tiles)
    split_len = ((sk_tiles + ns - 1) // ns) * BN
    ns = (Sk + split_len - 1) // split_len
    n_interior = 0
    for q0 in range(0, Sq, BM):
        for split in range(ns):
            lo, hi = key_range(Sq, Sk, causal, window, q0, ns, split_len, split)
            t0 = (lo // BN) * BN
            n = (hi - t0 + BN - 1) // BN if hi > lo else 0
            full_hi = min(n, (Sk - t0) // BN)
            u_lo = u_hi = 0
            if q0 + BM <= Sq:
                u_hi = full_hi
                if causal:
                    u_hi = min(u_hi, max(0, (q0 - t0 + 1) // BN))
                if window > 0:
                    need = q0 + BM - window - t0
                    u_lo = (need + BN - 1) // BN if need > 0 else 0
            steps = sched(n, u_lo, u_hi, full_hi)
            assert [t for _, t in steps] == list(range(n))
            for kind, t in steps:
                if kind != "interior":
                    continue
                n_interior += 1
                kt = t0 + t * BN
                assert lo <= kt and kt + BN <= hi
                for i in (q0, q0 + BM - 1):   # the extreme rows bound every row
                    assert i < Sq
                    for j in (kt, kt + BN - 1):
                        assert not causal or j <= i
                        assert window == 0 or j >= i - window + 1
                assert t + 1 < n and kt + 2 * BN <= Sk
    return n_interior


FIXED = [
    # Sq, Sk, causal, window, BN, splits
    (4096, 4096, 1, 0, 64, 1), (4096, 4096, 0, 0, 64, 1), (8192, 65536, 0, 0, 32, 8),
    (200, 700, 0, 0, 64, 2), (260, 700, 1, 150, 64, 3), (16384, 16384, 1, 4096, 64, 1),
    (300, 300, 1, 0, 64, 1), (257, 190, 1, 0, 64, 1), (384, 500, 1, 100, 64, 1),
    (96, 1000, 0, 0, 32, 1), (200, 700, 0, 0, 32, 7),
]


@pytest.mark.parametrize("shape", FIXED, ids=["-".join(map(str, s)) for s in FIXED])
def test_schedule_fixed(shape):
    check_shape(*shape)


def test_schedule_random():
    rng = random.Random(20261202)
    total = 0
    for _ in range(300):
        total += check_shape(rng.randint(1, 1500), rng.randint(1, 1500), rng.randint(0, 1),
                             rng.choice([0, 0, 1, 17, 100, 700]), rng.choice([32, 64]),
                             rng.choice([1, 1, 2, 3, 7]))
    assert total > 0          # the interior path is exercised


def test_schedule_rejects_partial_copy():
    # A pair bound that ignores whether the copied tile is full lets an interior
    # step copy the partial last tile of a split: the model must catch that.
    def buggy(n, u_lo, u_hi, full_hi):
        return schedule(n, u_lo, min(u_hi, n - 1), n)
    with pytest.raises(AssertionError):
        check_shape(200, 700, 0, 0, 64, 2, sched=buggy)


def check_sparse(Sq, Sk, causal, window, BN, nsplit, rng, sched=None):
    """Block-sparse form: the workgroup visits a sorted subset of its range's
    key tiles (its mask's nonzero blocks); position t of that list is the
    tile at key list[t]. Without a causal or window mask the kernel takes the
    interior step on every list position whose tile, and the next one it
    copies, are full; only the last listed tile can be partial."""
    sched = sched or schedule
    sk_tiles = (Sk + BN - 1) // BN
    ns = min(nsplit, sk_tiles)
    split_len = ((sk_tiles + ns - 1) // ns) * BN
    ns = (Sk + split_len - 1) // split_len
    n_interior = 0
    for q0 in range(0, Sq, BM):
        for split in range(ns):
            lo, hi = key_range(Sq, Sk, causal, window, q0, ns, split_len, split)
            t0 = (lo // BN) * BN
            n_all = (hi - t0 + BN - 1) // BN if hi > lo else 0
            keep = [t for t in range(n_all) if rng.random() < 0.6]
            kts = [t0 + BN * t for t in keep]
            n = len(kts)
            full_hi = n - 1 if n > 0 and kts[-1] + BN > Sk else n
            u_lo = u_hi = 0
            if q0 + BM <= Sq and not causal and window <= 0:
                u_hi = full_hi
            steps = sched(n, u_lo, u_hi, full_hi)
            assert [t for _, t in steps] == list(range(n))
            for kind, t in steps:
                if kind != "interior":
                    continue
                n_interior += 1
                kt = kts[t]
                assert not causal and window == 0 and q0 + BM <= Sq
                assert lo <= kt and kt + BN <= min(hi, Sk)
                assert t + 1 < n and kts[t + 1] + BN <= Sk   # the copied tile is full
    return n_interior


def test_schedule_block_sparse_random():
    rng = random.Random(20261203)
    total = 0
    for _ in range(200):
        total += check_sparse(rng.randint(1, 1500), rng.randint(1, 1500), rng.randint(0, 1),
                              rng.choice([0, 0, 1, 100]), rng.choice([32, 64]),
                              rng.choice([1, 1, 2, 3]), rng)
    assert total > 0

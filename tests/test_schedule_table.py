"""Persistent-launch schedules (host computation in libfa.so; runs without a GPU).

For float32 causal or windowed problems with few query tiles the library runs
one persistent workgroup per slot over a list of key-split pieces. These tests
check the lists against an independent model of the work: every piece exactly
once, and the most loaded slot no worse than longest-first greedy placement.
"""
import heapq

import pytest

import attention_forward_online_fa_amd as fa

BM, BN, COST0 = 128, 32, 5     # query rows per tile, keys per tile (fp32), fixed cost in half tiles


def piece_tiles(q0, split, split_len, Sq, Sk, causal, window):
    # keys a query tile [q0, q0 + BM) visits in one split, from the masking rules
    lo, hi = split * split_len, min(Sk, split * split_len + split_len)
    last = min(q0 + BM, Sq) - 1
    if causal:
        hi = min(hi, last + 1)
    if window > 0:
        lo = max(lo, q0 - window + 1)
    return 0 if hi <= lo else (hi - (lo // BN) * BN + BN - 1) // BN


def model(B, H, HKV, Sq, Sk, ns, causal, window):
    sk_tiles = (Sk + BN - 1) // BN
    split_len = -(-sk_tiles // ns) * BN
    units, group = B * H * ns, H // HKV
    n_q = -(-Sq // BM)
    cost = []
    for item in range(n_q * units):
        qb, u = divmod(item, units)
        split = (u // group) % ns
        cost.append(2 * piece_tiles(qb * BM, split, split_len, Sq, Sk, causal, window) + COST0)
    return cost


def greedy_makespan(cost, nslot):
    h = [0] * nslot
    for c in sorted(cost, reverse=True):
        heapq.heappush(h, heapq.heappop(h) + c)
    return max(h)


CASES = [
    # B, H, HKV, Sq, Sk, D, causal, window, nslot
    (4, 8, 8, 1024, 1024, 64, 1, 0, 768),      # fp32 causal MHA workload
    (1, 4, 2, 300, 300, 64, 1, 0, 96),         # ragged, GQA
    (2, 2, 1, 1000, 1500, 128, 0, 256, 128),   # one-sided window, Sk > Sq
    (1, 16, 4, 2048, 2048, 128, 1, 512, 512),  # causal sliding window
    (1, 1, 1, 129, 129, 256, 1, 0, 7),
]


@pytest.mark.parametrize("case", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_schedule_covers_every_piece_once_and_balances(case):
    B, H, HKV, Sq, Sk, D, causal, window, nslot = case
    ns, off, items = fa.schedule_table(B, H, HKV, Sq, Sk, D, nslot, causal=causal, window=window)
    cost = model(B, H, HKV, Sq, Sk, ns, causal, window)
    assert len(off) == nslot + 1 and off[0] == 0 and off[-1] == len(items)
    assert all(a <= b for a, b in zip(off, off[1:]))
    assert sorted(items) == list(range(len(cost)))
    loads = [sum(cost[i] for i in items[off[s]:off[s + 1]]) for s in range(nslot)]
    assert max(loads) <= greedy_makespan(cost, nslot)
    # no slot can shed its cheapest piece to the least loaded slot and stay the maximum
    lo = min(loads)
    for s in range(nslot):
        if loads[s] == max(loads) and off[s + 1] > off[s]:
            c = min(cost[i] for i in items[off[s]:off[s + 1]])
            assert lo + c >= loads[s]


def test_split_count_cuts_the_longest_tile_to_the_average_load():
    # fp32 causal MHA workload on 768 slots: 4608 key tiles in all, 6 per slot,
    # longest query tile 32 tiles -> ceil(32 / (6 + 2.5)) = 4 splits
    ns, off, items = fa.schedule_table(4, 8, 8, 1024, 1024, 64, 768, causal=True)
    assert ns == 4


def test_schedule_table_argument_errors():
    with pytest.raises(fa.FaError):
        fa.schedule_table(1, 4, 3, 64, 64, 64, 8, causal=True)     # H % HKV != 0
    with pytest.raises(fa.FaError):
        fa.schedule_table(1, 4, 4, 64, 64, 64, 0, causal=True)     # no slot

"""CPU model of the few-token bucketing in csrc/k_decode.h (route_small): a
bitonic sort of the keys (e << 6 | t << 4 | k) over 64 lanes, absent entries
last, then runs of equal experts found by comparing each sorted entry with
the one before it and numbered by a prefix count. The model transcribes
those steps and checks them against the definition of the bucketing: entries
ordered by (expert, token), one run per distinct expert in ascending order,
each run's first slot and token count, and every (t, k)'s slot."""
import itertools
import random

import pytest


def bitonic_64(keys):
    """The kernel's network: lane-parallel compare-exchange with partner lane ^ stride."""
    v = list(keys)
    size = 2
    while size <= 64:
        stride = size >> 1
        while stride > 0:
            other = [v[lane ^ stride] for lane in range(64)]
            nv = []
            for lane in range(64):
                keep_min = ((lane & stride) == 0) == ((lane & size) == 0)
                nv.append(min(v[lane], other[lane]) if keep_min else max(v[lane], other[lane]))
            v = nv
            stride >>= 1
        size <<= 1
    return v


def model(flat, T, K):
    n = T * K
    keys = [0xFFFFFFFF] * 64
    for lane in range(n):
        t, k = divmod(lane, K)
        keys[lane] = (flat[lane] << 6) | (t << 4) | k
    key = bitonic_64(keys)
    ent = []
    slot_of = {}
    first = []
    for lane in range(64):
        has = lane < n
        e, t, k = key[lane] >> 6, (key[lane] >> 4) & 3, key[lane] & 15
        prev = key[lane - 1] if lane else key[lane]
        first.append(has and (lane == 0 or (prev >> 6) != (key[lane] >> 6)))
        if has:
            ent.append((e, t))
            slot_of[(t, k)] = lane
    runs = [lane for lane in range(64) if first[lane]]
    uniq = []
    for u, p in enumerate(runs):
        nxt = runs[u + 1] if u + 1 < len(runs) else n
        uniq.append((key[p] >> 6, p, nxt - p))
    return ent, slot_of, uniq


def definition(flat, T, K):
    entries = sorted((flat[t * K + k], t, k) for t in range(T) for k in range(K))
    ent = [(e, t) for e, t, _ in entries]
    slot_of = {(t, k): p for p, (e, t, k) in enumerate(entries)}
    uniq = []
    for p, (e, t, k) in enumerate(entries):
        if p == 0 or entries[p - 1][0] != e:
            uniq.append([e, p, 0])
        uniq[-1][2] += 1
    return ent, slot_of, [tuple(u) for u in uniq]


def routings():
    rng = random.Random(11)
    for T, K in [(1, 1), (1, 8), (2, 8), (3, 8), (4, 8), (4, 16), (2, 16), (3, 5), (4, 2)]:
        for E in (16, 256):
            if K > E:
                continue
            for _ in range(30):
                # correlated draws: tokens pick from a small pool, so experts repeat
                pool = rng.sample(range(E), min(E, rng.choice([K, K + 2, 2 * K, E])))
                flat = []
                for t in range(T):
                    flat += rng.sample(pool, K)
                yield T, K, flat
    # every token the same experts, in different orders; extremes of the index range
    yield 4, 16, [e for t in range(4) for e in (random.Random(t).sample(range(240, 256), 16))]
    yield 4, 8, [0, 255, 1, 254, 2, 253, 3, 252] * 4


@pytest.mark.parametrize("case", list(routings()))
def test_bitonic_bucketing_matches_the_definition(case):
    T, K, flat = case
    assert model(flat, T, K) == definition(flat, T, K)


def test_network_sorts_every_zero_one_input_of_a_sample():
    # 0-1 principle: a comparator network sorts every input iff it sorts every
    # 0-1 input; check a sample of 0-1 inputs and all single-one inputs
    rng = random.Random(3)
    cases = [[1 if i == j else 0 for i in range(64)] for j in range(64)]
    cases += [[rng.randint(0, 1) for _ in range(64)] for _ in range(2000)]
    for c in cases:
        assert bitonic_64(c) == sorted(c)

"""Pins of the oracle's ranking, selection and compaction against brute force.

The brute force below ranks by counting (an item's rank is the number of
items that beat it: larger key, or equal key and lower index), which is a
different formulation from the oracle's sort.
"""
import itertools
import math

import numpy as np
import pytest

import oracle

NAN_BITS = 0x7FC00000
INF_BITS = 0x7F800000


def brute_rank_range(keys, r_lo, r_hi, nonzero_only=False, include=None):
    n = len(keys)
    elig = [m for m in range(n) if (not nonzero_only) or keys[m] != 0]
    out = []
    for i in range(n):
        chosen = False
        if i in elig:
            rank = sum(1 for m in elig if keys[m] > keys[i] or (keys[m] == keys[i] and m < i))
            chosen = r_lo <= rank < r_hi
        if include is not None and include[i]:
            chosen = True
        if chosen:
            out.append(i)
    return out


def test_exhaustive_small():
    alphabet = [0, 1, 7, INF_BITS, NAN_BITS]
    for n in range(0, 5):
        for combo in itertools.product(alphabet, repeat=n):
            keys = np.array(combo, dtype=np.uint32)
            for r_lo in range(0, n + 1):
                for r_hi in range(r_lo, n + 2):
                    for nz in (False, True):
                        got = oracle.rank_range(keys, r_lo, r_hi, nonzero_only=nz).tolist()
                        assert got == brute_rank_range(list(combo), r_lo, r_hi, nz), (combo, r_lo, r_hi, nz)


def test_random_with_include():
    rng = np.random.default_rng(1)
    for trial in range(300):
        n = int(rng.integers(1, 65))
        keys = rng.integers(0, 6, size=n).astype(np.uint32) * np.uint32(rng.integers(1, 1 << 20))
        r_lo = int(rng.integers(0, n + 1))
        r_hi = int(rng.integers(r_lo, n + 3))
        inc = rng.random(n) < 0.2 if trial % 2 else None
        nz = bool(trial % 3 == 0)
        got = oracle.rank_range(keys, r_lo, r_hi, nonzero_only=nz, include=inc).tolist()
        assert got == brute_rank_range(keys.tolist(), r_lo, r_hi, nz, inc)


def test_count_invariant():
    rng = np.random.default_rng(2)
    for _ in range(50):
        n = int(rng.integers(1, 200))
        keys = rng.integers(0, 4, size=n).astype(np.uint32)
        r_lo = int(rng.integers(0, n + 1))
        r_hi = int(rng.integers(r_lo, n + 5))
        for nz in (False, True):
            eligible = int(np.count_nonzero(keys)) if nz else n
            sel = oracle.rank_range(keys, r_lo, r_hi, nonzero_only=nz)
            assert sel.size == max(0, min(r_hi, eligible) - r_lo)
            assert np.all(np.diff(sel) > 0)


def test_key_abs_orders_magnitude():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(4000) * np.exp(rng.standard_normal(4000) * 4)).astype(np.float32)
    k = oracle.key_abs(v)
    mags = [abs(float(x)) for x in v]
    for _ in range(2000):
        i, j = rng.integers(0, v.size, size=2)
        assert (k[i] > k[j]) == (mags[i] > mags[j])
        assert (k[i] == k[j]) == (mags[i] == mags[j])


def test_key_abs_special_values():
    v = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1.0, -1.0], dtype=np.float32)
    k = oracle.key_abs(v)
    assert k[0] == k[1] == 0
    assert k[2] == k[3] == INF_BITS
    assert k[4] > k[2]
    assert k[5] == k[6]
    # NaN ranks first, then the infinities (lower index first), then +-1, then zeros.
    assert oracle.rank_order(k).tolist() == [4, 2, 3, 5, 6, 0, 1]


def test_key_signed_orders_values():
    rng = np.random.default_rng(4)
    v = (rng.standard_normal(3000) * 10).astype(np.float32)
    v[:5] = [0.0, -0.0, -1e-30, 1e-30, -np.inf]
    k = oracle.key_signed(v)
    for _ in range(3000):
        i, j = rng.integers(0, v.size, size=2)
        if float(v[i]) != float(v[j]):
            assert (k[i] > k[j]) == (float(v[i]) > float(v[j]))


def test_cluster_max_and_expand():
    rng = np.random.default_rng(5)
    keys = rng.integers(0, 1000, size=96).astype(np.uint32)
    kappa = oracle.cluster_max_key(keys, 32)
    for c in range(3):
        assert kappa[c] == max(int(x) for x in keys[32 * c:32 * c + 32])
    rows = oracle.expand_clusters(np.array([0, 2]), 32)
    assert rows.tolist() == list(range(0, 32)) + list(range(64, 96))


def test_count_of():
    # percent -> count: floor(p*N/100) (SelectInfer Table 1 ratios on d_ff sizes)
    assert oracle.count_of(50, 8192) == 4096
    assert oracle.count_of(30, 8192) == 2457
    assert oracle.count_of(20, 8192) == 1638
    assert oracle.count_of(15, 4096) == 614 and oracle.count_of(35, 4096) == 1433
    assert oracle.count_of(15, 14336) == 2150 and oracle.count_of(35, 14336) == 5017
    assert oracle.count_of(40, 17408) == 6963
    assert math.floor(40 * 17408 / 100) == 6963

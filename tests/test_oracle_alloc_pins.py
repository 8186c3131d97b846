"""Pins of the salience and rank-allocation oracle (oracle/alloc.py) against closed forms, hand-worked
cases, invariants and a brute-force search over thresholds.

The method ("VarRate: Training-Free Variable-Rate KV Cache Compression for Long-Context LLMs", "Method"):
each token's rank follows its query salience and no token drops to rank zero.
"""
import math

import numpy as np
import pytest

from oracle import alloc as A


def _rand(rng, B, W, T, Hq, Hkv, d=16, scale=1.0):
    q = rng.standard_normal((B, W, Hq, d)) * scale
    k = rng.standard_normal((B, T, Hkv, d)) * scale
    return q, k


def test_salience_total_is_queries_times_heads():
    rng = np.random.default_rng(0)
    q, k = _rand(rng, 3, 8, 40, 4, 2)
    seq = [40, 5, 8]
    s = A.salience(q, k, seq, 10000.0)
    # every present query's probabilities sum to 1 per head; sequence 1 has only 5 of the 8 window positions
    np.testing.assert_allclose(s.sum(axis=1), [8 * 4, 5 * 4, 8 * 4], rtol=1e-12)
    assert np.all(s[1, 5:] == 0) and np.all(s >= 0)


def test_salience_single_query_is_its_attention_row():
    # W = 1: the salience is the softmax row of the last query; RoPE written here with complex numbers
    rng = np.random.default_rng(1)
    d, T = 8, 12
    q, k = _rand(rng, 1, 1, T, 2, 1, d=d)
    theta = 100.0
    freq = theta ** (-2.0 * np.arange(d // 2) / d)

    def rot(x, p):
        z = (x[: d // 2] + 1j * x[d // 2:]) * np.exp(1j * p * freq)
        return np.r_[z.real, z.imag]

    want = np.zeros(T)
    for h in range(2):
        qr = rot(q[0, 0, h], T - 1)
        sc = np.array([qr @ rot(k[0, t, 0], t) for t in range(T)]) / math.sqrt(d)
        p = np.exp(sc - sc.max())
        want += p / p.sum()
    np.testing.assert_allclose(A.salience(q, k, [T], theta)[0], want, rtol=1e-12)


def test_salience_uniform_keys_closed_form():
    # identical keys and theta = 0: each query spreads 1 / (pos + 1) over its causal range
    rng = np.random.default_rng(2)
    T, W, Hq = 10, 4, 3
    q = rng.standard_normal((1, W, Hq, 8))
    k = np.tile(rng.standard_normal((1, 1, 1, 8)), (1, T, 1, 1))
    s = A.salience(q, k, [T], 0.0)[0]
    want = np.zeros(T)
    for i in range(W):
        p = T - W + i
        want[: p + 1] += Hq / (p + 1)
    np.testing.assert_allclose(s, want, rtol=1e-12)


def test_salience_gqa_mapping():
    # two KV heads holding the same keys give what one KV head gives
    rng = np.random.default_rng(3)
    q, k = _rand(rng, 1, 4, 20, 4, 1)
    s1 = A.salience(q, k, [20], 500.0)
    s2 = A.salience(q, np.repeat(k, 2, axis=2), [20], 500.0)
    np.testing.assert_allclose(s1, s2, rtol=1e-12)


def test_alloc_hand_worked():
    # ladder 8/16/32, weights 1, 0.5, saliences 3, 2, 1, mean rank 16: budget 48, 24 at the base rank.  Steps by
    # gain: (t0, 8->16) 3, (t1, 8->16) 2, (t0, 16->32) 1.5 ...; costs 8, 8, 16: the third no longer fits.
    r = A.rank_alloc(np.array([[3, 2, 1]], np.float32), [3], [8, 16, 32], np.array([1, 0.5], np.float32), 16)
    assert r.tolist() == [[16, 16, 8]]
    # mean 24: budget 72, extra 48: 8 + 8 + 16 = 32, then (t2, 8->16) gain 1 and (t1, 16->32) gain 1 tie (cost 24):
    # 56 > 48, so the tie group is left out as a whole
    r = A.rank_alloc(np.array([[3, 2, 1]], np.float32), [3], [8, 16, 32], np.array([1, 0.5], np.float32), 24)
    assert r.tolist() == [[32, 16, 8]]


def test_alloc_extremes_and_padding():
    rng = np.random.default_rng(4)
    sal = rng.random((2, 50)).astype(np.float32)
    lad, w = [8, 16, 32, 64], np.array([4, 2, 1], np.float32)
    assert np.all(A.rank_alloc(sal, [50, 30], lad, w, 8)[0] == 8)
    full = A.rank_alloc(sal, [50, 30], lad, w, 64)
    assert np.all(full[0] == 64) and np.all(full[1, :30] == 64) and np.all(full[1, 30:] == 0)


def test_alloc_invariants_and_threshold_brute_force():
    rng = np.random.default_rng(5)
    lad = [8, 16, 32, 64]
    w = np.array([1.0, 0.6, 0.25], np.float32)
    for trial in range(30):
        T = int(rng.integers(1, 14))
        sal = rng.random((1, T)).astype(np.float32)
        if trial % 3 == 0:
            sal[0, : T // 2] = sal[0, 0]          # ties
        mean = float(rng.uniform(8, 64))
        r = A.rank_alloc(sal, [T], lad, w, mean)[0].astype(np.int64)
        bud = A.budget(mean, T)
        assert set(r.tolist()) <= set(lad) and r.sum() <= bud
        # monotone in salience
        for a in range(T):
            for b in range(T):
                if sal[0, a] > sal[0, b]:
                    assert r[a] >= r[b]
        # brute force: every threshold allocation {steps with gain >= lam}, lam over the gains and +inf; the
        # oracle's is the one with the smallest lam that fits
        gains = (sal[0][:, None] * w[None, :]).astype(np.float32)
        best = None
        for lam in sorted(set(gains.ravel().tolist()) | {math.inf}, reverse=True):
            steps = (gains >= np.float32(lam)).sum(axis=1)
            tot = int(np.array(lad)[steps].sum())
            if tot <= bud:
                best = np.array(lad)[steps]
            else:
                break
        assert np.array_equal(r, best), (trial, r, best)


def test_alloc_budget_floor():
    assert A.budget(20.8, 100) == 2080 and A.budget(20.85, 3) == 62

"""Pins of the Lagrangian budget allocation oracle (oracle/plan.py).

The method ("JoLT: Near-Lossless KV Cache Compression" thesis page, "How JoLT works"): one multiplier picks
every cell's ranks and residual width under a shared byte budget.  Everett's theorem fixes what such a choice
guarantees: an allocation that minimizes D + lam B cell by cell has the least total distortion among all
allocations that cost no more bytes.  Brute force over every allocation of small problems checks that, and
hand-worked cases, extremes and monotonicity check the rest.
"""
import itertools

import numpy as np
import pytest

from oracle import plan as PL


def _rand(rng, n_cells, n_opt):
    # options of increasing bytes and decreasing distortion, with some dominated options mixed in
    B = np.sort(rng.integers(1, 40, (n_cells, n_opt)), axis=1).astype(np.float64)
    D = np.sort(rng.random((n_cells, n_opt)) * 10, axis=1)[:, ::-1].copy()
    D[rng.random(D.shape) < 0.15] += 3.0
    return D, B


def test_hand_worked():
    # two cells, options (bytes, distortion): cell 0: (1, 9), (2, 4), (4, 1); cell 1: (1, 5), (3, 2)
    # crossings: cell 0: 5 (o0->o1), 1.5 (o1->o2), 8/3 (o0->o2); cell 1: 1.5
    D = np.array([[9.0, 4.0, 1.0], [5.0, 2.0, np.inf]])
    B = np.array([[1.0, 2.0, 4.0], [1.0, 3.0, 1e9]])
    assert PL.plan(D, B, 7)[0].tolist() == [2, 1]      # lam = 0: the best options fit (4 + 3)
    # budget 5: at lam = 1.5 cell 0 ties o1/o2 and cell 1 ties o0/o1, both take the cheaper (3 bytes); the tie
    # fill then gives cell 0 its o2 (5 bytes); cell 1's o1 would make 7
    ch, lam = PL.plan(D, B, 5)
    assert ch.tolist() == [2, 0] and lam == pytest.approx(1.5)
    ch, lam = PL.plan(D, B, 3)
    assert ch.tolist() == [1, 0] and lam == pytest.approx(1.5)
    ch, lam = PL.plan(D, B, 2)                          # 1.5 and 8/3 give 3 bytes; at 5 cell 0 ties o0/o1
    assert ch.tolist() == [0, 0] and lam == pytest.approx(5.0)
    assert PL.plan(D, B, 1.5) is None


def test_rounded_crossing_still_reaches_the_cheapest_options():
    # cell 0 switches at (13.4 - 10.3) / 24, a rounded value at which D + lam B of its two options need not be
    # equal in floating point; the choice must still fall back to the cheap option there, so that the budget
    # 105 (the cheapest options cost 101) has a solution.  Cell 2's two options cost the same: the one of less
    # distortion is its only sensible choice.
    D = np.array([[13.4, 10.3], [20.0, 19.7], [10.7, 2.9]])
    B = np.array([[13.0, 37.0], [32.0, 39.0], [56.0, 56.0]])
    ch, lam = PL.plan(D, B, 105)
    assert ch.tolist() == [0, 0, 1] and lam == (13.4 - 10.3) / 24
    assert PL.plan(D, B, 125)[0].tolist() == [1, 0, 1]
    assert PL.plan(D, B, 132)[0].tolist() == [1, 1, 1]


def test_everett_optimality_brute_force():
    rng = np.random.default_rng(1)
    for trial in range(40):
        nc, no = int(rng.integers(1, 5)), int(rng.integers(2, 5))
        D, B = _rand(rng, nc, no)
        cheapest = B.min(axis=1).sum()
        budget = float(rng.uniform(cheapest, B.max(axis=1).sum() + 3))
        ch, lam = PL.plan(D, B, budget)
        rows = np.arange(nc)
        used, dist = B[rows, ch].sum(), D[rows, ch].sum()
        assert used <= budget
        for alloc in itertools.product(range(no), repeat=nc):
            a = np.array(alloc)
            if B[rows, a].sum() <= used:
                assert D[rows, a].sum() >= dist - 1e-12, (trial, alloc)
        # and every cell's choice minimizes D + lam B
        v = D + lam * B
        # lam is a rounded crossing point: the two vertices it ties agree to a few ulps of the values
        assert np.all(v[rows, ch] <= v.min(axis=1) + 1e-12 * (1 + np.abs(v).max()))


def test_extremes_and_monotonicity():
    rng = np.random.default_rng(2)
    D, B = _rand(rng, 6, 5)
    rows = np.arange(6)
    best = np.array([min(range(5), key=lambda o: (D[c, o], B[c, o], o)) for c in range(6)])
    assert np.array_equal(PL.plan(D, B, 1e9)[0], best)
    cheap_total = B.min(axis=1).sum()
    ch, _ = PL.plan(D, B, cheap_total)
    assert B[rows, ch].sum() == cheap_total
    assert PL.plan(D, B, cheap_total - 0.5) is None
    prev = np.inf
    for budget in np.linspace(cheap_total, B.max(axis=1).sum(), 25):
        ch, _ = PL.plan(D, B, budget)
        dist = D[rows, ch].sum()
        assert dist <= prev + 1e-12
        prev = dist


def test_tail_energy():
    assert PL.tail_energy([5.0, 3.0, 1.0, 0.5], 2) == 1.5 and PL.tail_energy([1.0], 1) == 0.0

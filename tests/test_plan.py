"""kvc_plan_budget (host code of the library) against the Lagrangian allocation oracle: the same choices and
multiplier on random option tables, and on tables built from a spectrum (no GPU needed)."""
import numpy as np
import pytest

from oracle import plan as PL
from rank_bit_compressed_amd import kvc


def test_plan_matches_oracle_on_random_tables():
    rng = np.random.default_rng(3)
    for trial in range(200):
        nc, no = int(rng.integers(1, 9)), int(rng.integers(1, 7))
        B = np.sort(rng.integers(0, 60, (nc, no)), axis=1).astype(np.float64)
        D = np.round(np.sort(rng.random((nc, no)) * 20, axis=1)[:, ::-1], 1).copy()   # rounded: ties happen
        D[rng.random(D.shape) < 0.2] += 2.0
        budget = float(rng.integers(int(B.min(axis=1).sum()), int(B.max(axis=1).sum()) + 5))
        want = PL.plan(D, B, budget)
        ch, lam = kvc.plan_budget(D, B, budget)
        assert want is not None
        assert ch.tolist() == want[0].tolist() and lam == want[1], (trial, ch, want)


def test_plan_rejects_what_does_not_fit_and_bad_values():
    D = np.array([[3.0, 1.0]]); B = np.array([[2.0, 5.0]])
    with pytest.raises(kvc.KvcError):
        kvc.plan_budget(D, B, 1.0)
    with pytest.raises(kvc.KvcError):
        kvc.plan_budget(np.array([[np.nan, 1.0]]), B, 10.0)
    with pytest.raises(kvc.KvcError):
        kvc.plan_budget(D, np.array([[-1.0, 5.0]]), 10.0)


def test_plan_from_spectra_ranks_and_residual():
    # cells = (keys, values) of 4 layers; options = rank r in {16, 32, 48, 64} x residual {off, 2 bits}; per token
    # and head, INT4 codes r/2 + 4 bytes per 32-group, the residual 34 bytes; distortion: the spectrum's energy
    # past r, times 1 without the residual and 0.15 with it (a rotated 2-bit quantizer's relative error here)
    rng = np.random.default_rng(4)
    ranks, T_heads = [16, 32, 48, 64], 32768 * 8
    D, B = [], []
    for layer in range(4):
        for which in range(2):
            s2 = np.sort(rng.random(128) ** (3 + which + layer % 2))[::-1] * 1000
            d_row, b_row = [], []
            for r in ranks:
                for res in (0, 1):
                    d_row.append(PL.tail_energy(s2, r) * (0.15 if res else 1.0))
                    b_row.append(T_heads * (r // 2 + 4 * (r // 32 if r % 32 == 0 else r // 32 + 1) + 34 * res))
            D.append(d_row)
            B.append(b_row)
    D, B = np.array(D), np.array(B, dtype=np.float64)
    for frac in (0.25, 0.5, 0.8):
        budget = B.min(1).sum() + frac * (B.max(1).sum() - B.min(1).sum())
        want = PL.plan(D, B, budget)
        ch, lam = kvc.plan_budget(D, B, budget)
        assert ch.tolist() == want[0].tolist() and lam == want[1]
        assert B[np.arange(8), ch].sum() <= budget

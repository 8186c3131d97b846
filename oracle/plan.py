"""CPU oracle for the Lagrangian rank/bit allocation of a byte budget.

TEST INFRASTRUCTURE ONLY.  Only the tests import this module; the product library never does.  Plain Python
and numpy in fp64.

What is computed ("JoLT: Near-Lossless KV Cache Compression" thesis page, Abstract and "How JoLT works"; "A
JoLT for the KV cache", abstract): the keys and the values of each layer group are separate cells, and one
Lagrangian multiplier chooses every cell's ranks and residual bit width under a shared byte budget, before
anything is compressed.  Reading: each cell c has options o (a rank and a residual width, say) with a
distortion D[c][o] and a storage cost B[c][o].  For a multiplier lam >= 0 every cell takes the option that
minimizes D + lam B (ties: fewer bytes, then the lower option index).  The multiplier is the smallest lam whose
total bytes fit the budget.  The total only changes where some cell's choice does, at the crossing points
lam = (D[c][o1] - D[c][o2]) / (B[c][o2] - B[c][o1]); those and 0 are the candidates.  At that multiplier several
cells may tie between options (that is where they switch), and taking all of them at their cheapest can leave
budget unused: cell by cell, in order, a tied cell then takes its tied option of most bytes that still fits
(equal bytes: the lower index).  Every cell still minimizes D + lam B, so no allocation of at most the same
bytes has less total distortion (Everett's theorem).
"""
import numpy as np


def choose(D, B, lam):
    """Per-cell option minimizing D + lam B, ties to fewer bytes, then the lower index: int [n_cells]."""
    D = np.asarray(D, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    out = np.zeros(D.shape[0], dtype=np.int64)
    for c in range(D.shape[0]):
        best = None
        for o in range(D.shape[1]):
            key = (D[c, o] + lam * B[c, o], B[c, o], o)
            if best is None or key < best:
                best = key
        out[c] = best[2]
    return out


def candidates(D, B):
    """0 and every positive crossing point of two options of one cell, increasing."""
    D = np.asarray(D, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    lams = {0.0}
    for c in range(D.shape[0]):
        for o1 in range(D.shape[1]):
            for o2 in range(D.shape[1]):
                if B[c, o2] > B[c, o1] and D[c, o1] > D[c, o2]:
                    lams.add((D[c, o1] - D[c, o2]) / (B[c, o2] - B[c, o1]))
    return sorted(lams)


def plan(D, B, budget):
    """(choice int [n_cells], lam) of the smallest candidate lam whose choices fit the budget; None if even the
    cheapest options do not fit."""
    D = np.asarray(D, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    rows = np.arange(D.shape[0])
    for lam in candidates(D, B):
        ch = choose(D, B, lam)
        used = B[rows, ch].sum()
        if used > budget:
            continue
        for c in range(D.shape[0]):
            v = D[c] + lam * B[c]
            tied = [o for o in range(D.shape[1]) if v[o] == v[ch[c]]]
            for o in sorted(tied, key=lambda o: (-B[c, o], o)):
                if used - B[c, ch[c]] + B[c, o] <= budget:
                    used += B[c, o] - B[c, ch[c]]
                    ch[c] = o
                    break
        return ch, lam
    # at the largest crossing every cell already holds its cheapest option (ties go to fewer bytes)
    return None


def tail_energy(sigma2, r):
    """Energy of a spectrum (squared singular values, decreasing) beyond rank r."""
    s = np.asarray(sigma2, dtype=np.float64)
    return float(s[r:].sum())

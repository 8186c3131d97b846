"""CPU oracle for the Lagrangian rank/bit allocation of a byte budget.

TEST INFRASTRUCTURE ONLY.  Only the tests import this module; the product library never does.  Plain Python
and numpy in fp64.

What is computed ("JoLT: Near-Lossless KV Cache Compression" thesis page, Abstract and "How JoLT works"; "A
JoLT for the KV cache", abstract): the keys and the values of each layer group are separate cells, and one
Lagrangian multiplier chooses every cell's ranks and residual bit width under a shared byte budget, before
anything is compressed.  Reading: each cell c has options o (a rank and a residual width, say) with a
distortion D[c][o] and a storage cost B[c][o].  For a multiplier lam >= 0 every cell takes the option that
minimizes D + lam B (ties: fewer bytes).  As lam falls from infinity each cell walks up its lower convex hull of
(bytes, distortion) points, switching at its crossing multipliers (the breakpoints); the allocation uses the
smallest of 0 and all breakpoints whose choices fit the budget.  The choice at a multiplier is decided by
comparing it with the breakpoints themselves, not by evaluating D + lam B in floating point, so that rounding
cannot make the bytes non-monotone in lam.  At the chosen multiplier, cells sitting exactly on a breakpoint (a
tie between two vertices) then move on, cell by cell in order, while the bytes still fit.  Every cell's choice
minimizes D + lam B, so no allocation of at most the same bytes has less total distortion (Everett's theorem).
"""
import numpy as np


def hull(D_c, B_c):
    """One cell's Lagrangian path: (vertices, breakpoints).  From the cheapest option (fewest bytes, then least
    distortion, then lowest index), each step goes to the option of more bytes and less distortion with the
    largest crossing multiplier (D_v - D_p) / (B_p - B_v), the farthest of equal ones (most bytes, then the lowest
    index); breakpoints are kept non-increasing.  Choosing vertex k for multipliers in [lam_k, lam_(k-1)) is what
    minimizing D + lam B with ties to fewer bytes gives, decided by comparisons with these numbers only."""
    n = len(D_c)
    order = sorted(range(n), key=lambda o: (B_c[o], D_c[o], o))
    v = order[0]
    verts, lams = [v], []
    while True:
        best = None
        for p in range(n):
            if B_c[p] > B_c[v] and D_c[p] < D_c[v]:
                lam = (D_c[v] - D_c[p]) / (B_c[p] - B_c[v])
                key = (lam, B_c[p], -p)
                if best is None or key > best[0]:
                    best = (key, p)
        if best is None:
            return verts, lams
        lam, p = best[0][0], best[1]
        if lams and lam > lams[-1]:
            lam = lams[-1]
        verts.append(p)
        lams.append(lam)
        v = p


def walk(lams, lam):
    """Index of the vertex chosen at multiplier lam: every breakpoint strictly above lam is passed."""
    k = 0
    while k < len(lams) and lams[k] > lam:
        k += 1
    return k


def plan(D, B, budget):
    """(choice int [n_cells], lam) for the smallest of 0 and the cells' breakpoints whose choices fit; then the
    tie fill.  None if even the cheapest options do not fit."""
    D = np.asarray(D, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    nc = D.shape[0]
    hulls = [hull(list(D[c]), list(B[c])) for c in range(nc)]
    cands = sorted({0.0} | {l for _, ls in hulls for l in ls})
    for lam in cands:
        ks = [walk(ls, lam) for _, ls in hulls]
        used = sum(B[c, hulls[c][0][ks[c]]] for c in range(nc))
        if used > budget:
            continue
        for c in range(nc):  # tie fill: a cell on a breakpoint equal to lam moves on while the bytes fit
            verts, ls = hulls[c]
            while ks[c] < len(ls) and ls[ks[c]] == lam:
                extra = B[c, verts[ks[c] + 1]] - B[c, verts[ks[c]]]
                if used + extra > budget:
                    break
                used += extra
                ks[c] += 1
        return np.array([hulls[c][0][ks[c]] for c in range(nc)], dtype=np.int64), lam
    return None


def choose(D, B, lam):
    """Per-cell option at multiplier lam (no tie fill): int [n_cells]."""
    D = np.asarray(D, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    out = []
    for c in range(D.shape[0]):
        verts, ls = hull(list(D[c]), list(B[c]))
        out.append(verts[walk(ls, lam)])
    return np.array(out, dtype=np.int64)


def tail_energy(sigma2, r):
    """Energy of a spectrum (squared singular values, decreasing) beyond rank r."""
    s = np.asarray(sigma2, dtype=np.float64)
    return float(s[r:].sum())

"""CPU oracle for the partial Tucker form of a layer group's cache and its expansion into the up-projections
the block-shared decode reads.

TEST INFRASTRUCTURE ONLY.  Only the tests import this module; the product library never does.  Plain numpy in
fp64, with numpy's SVD as the one library step.

What is computed ("JoLT: Near-Lossless KV Cache Compression" thesis page, "How JoLT works" and "Key findings";
"A JoLT for the KV cache", abstract): the keys (or the values) of one sequence's layer group form a
fourth-order tensor X[t, i, h, l] (token, feature, head, layer).  A partial Tucker decomposition truncates only
the token and feature modes and keeps heads and layers whole:
    X ~ G x_1 U_t x_2 U_f,   X^[t, i, h, l] = sum_c sum_j U_t[t, c] U_f[i, j] G[c, j, h, l],
with U_t [T, r_t] and U_f [d, r_f] orthonormal and the core G [r_t, r_f, H, L].  Readings:
  * The factors are the leading left singular vectors of the token-mode and feature-mode unfoldings (the
    truncated higher-order SVD), and the core is X projected on them; the pages fix the form, not the fit.
  * Attention over the stored factors: token t's row U_t[t] is a latent shared by every head and layer of the
    group, and head h of layer l rebuilds its (pre-RoPE) key from it through W_hl = U_f G[:, :, h, l]^T
    ([d, r_t]): k = W_hl U_t[t].  That is the block-shared form (one latent per token, per-layer
    up-projections), with W_hl per sequence because the core is fitted per prefill cache.
  * The randomized token factor (FlashJoLT replaces the exact token-mode SVD with a randomized approximation;
    the pages name no scheme): randomized subspace iteration on the token-mode unfolding A = X_(1) [T, D] --
    the range finder of Halko, Martinsson and Tropp (2011) with q power iterations -- started from a Gaussian
    test matrix Omega [D, r_t] that the caller draws.  The sketch is as wide as the token rank (no
    oversampling and no closing small SVD): the partial Tucker form depends on U_t only through its span,
    since the core absorbs any rotation of it.  Every orthonormalisation is the Q factor of the QR
    decomposition with a positive diagonal R, which is unique for a full-rank argument.
    Pinned (tests/test_oracle_tucker_pins.py) by the uniqueness of that QR factor, exactness on planted rank, Halko,
    Martinsson and Tropp's deterministic error bound and the power iteration's principal-angle bound; no page
    prints a worked example to compare against.
"""
import numpy as np


def reconstruct(u_t, u_f, core):
    """X^[t, i, h, l] from the factors u_t [T, r_t], u_f [d, r_f] and core [r_t, r_f, H, L] (mode products)."""
    u_t = np.asarray(u_t, dtype=np.float64)
    u_f = np.asarray(u_f, dtype=np.float64)
    core = np.asarray(core, dtype=np.float64)
    y = np.tensordot(u_t, core, axes=(1, 0))                 # [T, r_f, H, L]: mode-1 product
    y = np.tensordot(u_f, y, axes=(1, 1))                    # [d, T, H, L]: mode-2 product
    return np.transpose(y, (1, 0, 2, 3))


def _leading(m, r):
    """Leading r left singular vectors of m, each with its entry of largest magnitude positive."""
    u, _, _ = np.linalg.svd(m, full_matrices=False)
    u = u[:, :r].copy()
    piv = u[np.argmax(np.abs(u), axis=0), np.arange(u.shape[1])]
    return u * np.where(piv < 0, -1.0, 1.0)


def unfold(x, mode):
    """Mode unfolding of a fourth-order tensor: rows indexed by that mode."""
    x = np.asarray(x, dtype=np.float64)
    return np.moveaxis(x, mode, 0).reshape(x.shape[mode], -1)


def hosvd(x, r_t, r_f):
    """Truncated partial HOSVD of x [T, d, H, L] on the token and feature modes -> (u_t, u_f, core)."""
    x = np.asarray(x, dtype=np.float64)
    u_t = _leading(unfold(x, 0), r_t)
    u_f = _leading(unfold(x, 1), r_f)
    core = np.tensordot(u_t.T, x, axes=(1, 0))               # [r_t, d, H, L]
    core = np.tensordot(u_f.T, core, axes=(1, 1))            # [r_f, r_t, H, L]
    return u_t, u_f, np.transpose(core, (1, 0, 2, 3))


def expand(u_f, core):
    """Block-shared up-projections from the feature factor and the core: w [L, r_t, H * d] with
    w[l, c, h * d + i] = (u_f core[:, :, h, l]^T)[i, c], so that the key of head h at layer l for latent u is
    w[l, :, h * d:(h + 1) * d]^T u."""
    u_f = np.asarray(u_f, dtype=np.float64)
    core = np.asarray(core, dtype=np.float64)
    d = u_f.shape[0]
    r_t, _, H, L = core.shape
    w = np.zeros((L, r_t, H * d))
    for l in range(L):
        for h in range(H):
            w[l, :, h * d:(h + 1) * d] = (u_f @ core[:, :, h, l].T).T
    return w


def to_bf16_bits(x):
    """bf16 bit patterns (uint16) of fp64 values rounded once to 8 significant bits, ties to even (normal
    range)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                                       # x = m 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(m * 256.0), e - 8)                  # exact in fp32
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def orth(y):
    """Q factor of the QR decomposition of y [n, k] (n >= k) with a positive diagonal R (numpy's QR, then the
    signs of Q's columns flipped where R's diagonal is negative): the unique such orthonormal basis of the
    column space when y has full column rank."""
    q, r = np.linalg.qr(np.asarray(y, dtype=np.float64))
    sgn = np.where(np.diag(r) < 0, -1.0, 1.0)
    return q * sgn


def randomized_range(a, omega, q):
    """Randomized subspace iteration on a [T, D] from omega [D, k]: Q = orth(a omega), then q times
    Z = orth(a^T Q), Q = orth(a Z).  Returns Q [T, k], an orthonormal basis of range((a a^T)^q a omega)."""
    a = np.asarray(a, dtype=np.float64)
    Q = orth(a @ np.asarray(omega, dtype=np.float64))
    for _ in range(q):
        Z = orth(a.T @ Q)
        Q = orth(a @ Z)
    return Q


def fit_randomized(x_tlhd, r_t, r_f, omega, q):
    """Partial Tucker factors of one sequence's layer group from x_tlhd [T, L, H, d] (token, layer, head,
    feature; the token-mode unfolding's columns are taken in that (l, h, i) order, which is also the row order
    of omega [L * H * d, r_t]): the randomized token factor u_t [T, r_t], the exact feature factor u_f [d, r_f]
    (leading left singular vectors of the feature-mode unfolding, largest-magnitude entry of each column
    positive) and the core projected on both, in the up-projection expansion's layout [L, H, r_t, r_f]."""
    x = np.asarray(x_tlhd, dtype=np.float64)
    T = x.shape[0]
    u_t = randomized_range(x.reshape(T, -1), omega, q)
    xs = np.transpose(x, (0, 3, 2, 1))                       # [T, d, H, L], the convention of hosvd
    u_f = _leading(unfold(xs, 1), r_f)
    core = np.tensordot(u_t.T, xs, axes=(1, 0))              # [r_t, d, H, L]
    core = np.tensordot(u_f.T, core, axes=(1, 1))            # [r_f, r_t, H, L]
    return u_t, u_f, np.transpose(core, (3, 2, 1, 0))        # [L, H, r_t, r_f]


def core_to_hosvd_layout(core_lhcj):
    """core [L, H, r_t, r_f] (the expansion's layout) -> [r_t, r_f, H, L] (reconstruct's)."""
    return np.transpose(np.asarray(core_lhcj), (2, 3, 1, 0))

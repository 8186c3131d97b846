"""CPU oracle for per-head basis fitting (the prefill step that produces the bases the decode reads).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's CPU-baseline leg import this
module; the product library never does.  Plain numpy in fp64; the singular value decomposition is
LAPACK's (numpy.linalg.svd), used as one library step.

What is computed (page titles and sections):
  - "JoLT: Near-Lossless KV Cache Compression" (thesis page), "Key findings": a per-head SVD of the cache
    beats every 4-D format that compresses the head or layer axis, and keys are decomposed before RoPE.
  - "A JoLT for the KV cache" (index page), abstract: the feature mode of the partial Tucker
    decomposition is truncated (the head and layer modes are kept).
  Reading: for KV head h, the rows of X_h are the head's pre-RoPE vectors (keys, or values) of every
  cached token, t < seq_len[b] of every sequence b.  The basis B_h (d x r) is the r right singular
  vectors of X_h with the largest singular values, in decreasing order; the latent of a token is then
  c = B_h^T k and its reconstruction B_h c.  No mean is removed (an SVD, not a PCA: the decode adds no
  mean term back).  Singular vectors are defined up to sign; the convention here makes the entry of
  largest magnitude of each column positive (the first such entry on a tie).
"""
import numpy as np


def sign_canonical(basis):
    """Flip each column of basis [..., d, r] so that its entry of largest magnitude is positive."""
    b = np.array(basis, dtype=np.float64, copy=True)
    idx = np.argmax(np.abs(b), axis=-2)                          # [..., r], first maximum on ties
    piv = np.take_along_axis(b, idx[..., None, :], axis=-2)      # [..., 1, r]
    return np.where(piv < 0, -b, b)


def head_rows(x, seq_len, h):
    """The rows of X_h: x[b, t, h, :] for t < seq_len[b], sequences in order, fp64 [N, d]."""
    x = np.asarray(x)
    rows = [np.asarray(x[b, :int(n), h, :], dtype=np.float64) for b, n in enumerate(seq_len)]
    return np.concatenate(rows, axis=0) if rows else np.zeros((0, x.shape[-1]))


def fit_basis(x, seq_len, rank):
    """Per-head SVD basis.

    x: [B, max_T, Hkv, d] pre-RoPE keys or values; seq_len: [B] tokens used per sequence (0..max_T);
    rank: r in 1..d.
    Returns (basis [Hkv, d, r] fp64, sign-canonical; sigma2 [Hkv, d] fp64, the squared singular values
    in decreasing order, i.e. the eigenvalues of X_h^T X_h, zero-padded when X_h has fewer than d rows).
    A head with no rows gets the first r coordinate axes (every direction is a singular vector then).
    """
    x = np.asarray(x)
    B, max_T, Hkv, d = x.shape
    if not 1 <= rank <= d:
        raise ValueError("rank must lie in 1..d")
    basis = np.zeros((Hkv, d, rank))
    sigma2 = np.zeros((Hkv, d))
    for h in range(Hkv):
        X = head_rows(x, seq_len, h)
        if X.shape[0] == 0:
            basis[h] = np.eye(d)[:, :rank]
            continue
        _, s, vt = np.linalg.svd(X, full_matrices=False)   # s decreasing; rows of vt are right singular vectors
        k = s.shape[0]
        sigma2[h, :k] = s * s
        if k >= rank:
            basis[h] = vt[:rank].T
        else:
            # fewer rows than r: complete the basis with an orthonormal set orthogonal to the row space
            q, _ = np.linalg.qr(np.concatenate([vt.T, np.eye(d)], axis=1))
            basis[h] = q[:, :rank]
    return sign_canonical(basis), sigma2


def truncation_energy(x, seq_len, basis):
    """sum over heads' rows of |k - B B^T k|^2 per head: [Hkv] fp64 (Eckart-Young: the sum of the
    squared singular values beyond the rank, when basis holds the leading right singular vectors)."""
    x = np.asarray(x)
    Hkv = x.shape[2]
    out = np.zeros(Hkv)
    for h in range(Hkv):
        X = head_rows(x, seq_len, h)
        Bh = np.asarray(basis[h], dtype=np.float64)
        R = X - (X @ Bh) @ Bh.T
        out[h] = float(np.sum(R * R))
    return out

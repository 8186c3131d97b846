"""Pins of the basis-fitting oracle (oracle/fit.py) against what the mathematics fixes.

The oracle computes the per-head SVD basis ("JoLT: Near-Lossless KV Cache Compression", "Key findings":
per-head SVD, pre-RoPE).  These checks do not re-call its SVD on the same data: they plant a known
decomposition (closed form), check Eckart-Young, equivariance and masking properties, and find the
leading directions of a tiny case by brute-force search over the sphere.
"""
import numpy as np
import pytest

from oracle import fit as F


def _orth(rng, n, k):
    q, r = np.linalg.qr(rng.standard_normal((n, k)))
    return q * np.sign(np.diag(r))


def _planted(rng, N, d, sig):
    U = _orth(rng, N, d)
    V = _orth(rng, d, d)
    return (U * sig) @ V.T, V


def test_planted_decomposition_recovered():
    rng = np.random.default_rng(1)
    N, d, r = 400, 128, 24
    sig = 10.0 * 2.0 ** (-np.arange(d) / 10.0)           # distinct, decreasing
    X, V = _planted(rng, N, d, sig)
    basis, s2 = F.fit_basis(X[None, :, None, :], [N], r)
    np.testing.assert_allclose(basis[0], F.sign_canonical(V[:, :r]), atol=1e-9)
    np.testing.assert_allclose(s2[0], sig ** 2, rtol=1e-10)
    # left singular vectors (a transposed operand) would not even have the right shape; the leading
    # right singular vector, not the trailing one, comes first
    assert abs(basis[0][:, 0] @ V[:, 0]) > 1 - 1e-12


def test_eckart_young_truncation_energy():
    rng = np.random.default_rng(2)
    N, d, r = 300, 64, 9
    sig = np.linspace(5.0, 0.1, d)
    X, _ = _planted(rng, N, d, sig)
    basis, _ = F.fit_basis(X[None, :, None, :], [N], r)
    e = F.truncation_energy(X[None, :, None, :], [N], basis)
    assert e[0] == pytest.approx(float(np.sum(sig[r:] ** 2)), rel=1e-10)
    # any other orthonormal r-frame leaves more energy
    other = _orth(rng, d, r)
    assert F.truncation_energy(X[None, :, None, :], [N], other[None])[0] > e[0] * 1.01


def test_uncentered_mean_direction_leads():
    # rows = a common direction mu plus small isotropic noise: an SVD puts mu first; a PCA (mean removed)
    # would put a noise direction first
    rng = np.random.default_rng(3)
    N, d = 500, 32
    mu = rng.standard_normal(d); mu /= np.linalg.norm(mu)
    X = 3.0 * mu[None, :] + 0.05 * rng.standard_normal((N, d))
    basis, _ = F.fit_basis(X[None, :, None, :], [N], 2)
    assert abs(basis[0][:, 0] @ mu) > 0.999


def test_masking_and_sequence_split():
    rng = np.random.default_rng(4)
    d, r = 16, 5
    lens = [7, 0, 20, 13]
    rows = rng.standard_normal((sum(lens), d)) * np.linspace(3, 0.2, d)
    x = np.full((4, 24, 1, d), 1e6)                       # padding beyond seq_len must be ignored
    o = 0
    for b, n in enumerate(lens):
        x[b, :n, 0] = rows[o:o + n]
        o += n
    b1, s1 = F.fit_basis(x, lens, r)
    b2, s2 = F.fit_basis(rows[None, :, None, :], [len(rows)], r)
    np.testing.assert_allclose(b1, b2, atol=1e-12)
    np.testing.assert_allclose(s1, s2, rtol=1e-12)
    # token order does not matter
    perm = rng.permutation(len(rows))
    b3, _ = F.fit_basis(rows[perm][None, :, None, :], [len(rows)], r)
    np.testing.assert_allclose(b3, b2, atol=1e-10)


def test_rotation_equivariance_and_head_independence():
    rng = np.random.default_rng(5)
    N, d, r = 200, 32, 6
    x = rng.standard_normal((1, N, 2, d)) * np.linspace(4, 0.3, d)
    Q = _orth(rng, d, d)
    xr = x.copy()
    xr[0, :, 0] = x[0, :, 0] @ Q.T                       # head 0 rotated: k' = Q k
    b, _ = F.fit_basis(x, [N], r)
    br, _ = F.fit_basis(xr, [N], r)
    np.testing.assert_allclose(np.abs(np.sum(br[0] * (Q @ b[0]), axis=0)), 1.0, atol=1e-9)
    np.testing.assert_allclose(br[1], b[1], atol=1e-12)   # head 1 untouched


def test_coordinate_axes():
    d, r = 12, 4
    scales = np.array([0.5, 7.0, 1.0, 3.0, 0.1, 5.0, 0.2, 2.0, 0.3, 4.0, 0.4, 6.0])
    X = np.diag(scales)                                   # orthogonal columns with distinct norms
    basis, s2 = F.fit_basis(X[None, :, None, :], [d], r)
    order = np.argsort(-scales)[:r]
    np.testing.assert_allclose(basis[0], np.eye(d)[:, order], atol=1e-12)
    np.testing.assert_allclose(s2[0], np.sort(scales ** 2)[::-1], rtol=1e-12)


def test_fewer_rows_than_rank_and_empty_head():
    rng = np.random.default_rng(6)
    d, r = 16, 6
    x = np.zeros((1, 8, 2, d))
    x[0, :3, 0] = rng.standard_normal((3, d))
    basis, s2 = F.fit_basis(x, [3], r)
    np.testing.assert_allclose(basis[0].T @ basis[0], np.eye(r), atol=1e-12)
    # the row space lies inside the span of the basis
    R = x[0, :3, 0]
    np.testing.assert_allclose(R @ basis[0] @ basis[0].T, R, atol=1e-12)
    assert np.all(s2[0, 3:] == 0)
    # head 1 has only zero rows: a zero Gram matrix, any frame is exact; the oracle returns the axes
    assert np.all(s2[1] == 0)
    np.testing.assert_allclose(np.abs(basis[1]).sum(axis=0), 1.0)
    np.testing.assert_allclose(basis[1].T @ basis[1], np.eye(r), atol=1e-12)


def test_brute_force_leading_directions_tiny():
    # d = 3: the first singular vector maximizes |X b| over the unit sphere, the second maximizes it on the
    # great circle orthogonal to the first.  A dense search, no decomposition.
    rng = np.random.default_rng(7)
    X = rng.standard_normal((6, 3)) * np.array([3.0, 1.5, 0.5])
    basis, s2 = F.fit_basis(X[None, :, None, :], [6], 2)
    th = np.linspace(0, np.pi, 721)
    ph = np.linspace(0, 2 * np.pi, 1441)
    T, P = np.meshgrid(th, ph, indexing="ij")
    pts = np.stack([np.sin(T) * np.cos(P), np.sin(T) * np.sin(P), np.cos(T)], -1).reshape(-1, 3)
    val = np.sum((pts @ X.T) ** 2, axis=1)
    b0 = pts[np.argmax(val)]
    assert abs(b0 @ basis[0][:, 0]) > 1 - 1e-4
    assert np.max(val) == pytest.approx(s2[0, 0], rel=1e-4)
    e1 = np.cross(b0, [1.0, 0.0, 0.0]); e1 /= np.linalg.norm(e1)
    e2 = np.cross(b0, e1)
    a = np.linspace(0, np.pi, 20001)
    circ = np.cos(a)[:, None] * e1 + np.sin(a)[:, None] * e2
    b1 = circ[np.argmax(np.sum((circ @ X.T) ** 2, axis=1))]
    assert abs(b1 @ basis[0][:, 1]) > 1 - 1e-4


def test_sign_convention():
    b = np.array([[0.1, -0.7], [-0.9, 0.7], [0.2, 0.1]])
    c = F.sign_canonical(b)
    np.testing.assert_allclose(c[:, 0], [-0.1, 0.9, -0.2])   # largest |entry| (-0.9) made positive
    np.testing.assert_allclose(c[:, 1], [0.7, -0.7, -0.1])   # tie: the first one (-0.7) made positive

"""Pins of the partial Tucker oracle (oracle/tucker.py): planted decompositions, the matrix special case
(Eckart-Young), the truncated HOSVD error bounds, the gauge freedom of the factors, and the expansion into
up-projections checked against the mode products by an independent route.

The form ("JoLT: Near-Lossless KV Cache Compression" thesis page, "How JoLT works"): token and feature modes
truncated, heads and layers kept whole.
"""
import numpy as np
import pytest

from oracle import tucker as TK


def _orth(rng, n, r):
    q, _ = np.linalg.qr(rng.standard_normal((n, r)))
    return q


def _planted(rng, T=40, d=12, H=3, L=2, r_t=5, r_f=4):
    u_t, u_f = _orth(rng, T, r_t), _orth(rng, d, r_f)
    core = rng.standard_normal((r_t, r_f, H, L)) * 3
    return u_t, u_f, core


def test_reconstruct_elementwise_brute_force():
    rng = np.random.default_rng(0)
    u_t, u_f, core = _planted(rng, T=7, d=5, H=2, L=3, r_t=3, r_f=2)
    x = TK.reconstruct(u_t, u_f, core)
    assert x.shape == (7, 5, 2, 3)
    for t, i, h, l in [(0, 0, 0, 0), (6, 4, 1, 2), (3, 2, 0, 1), (5, 1, 1, 0)]:
        want = sum(u_t[t, c] * u_f[i, j] * core[c, j, h, l] for c in range(3) for j in range(2))
        assert abs(x[t, i, h, l] - want) < 1e-12


def test_planted_decomposition_is_recovered():
    rng = np.random.default_rng(1)
    u_t, u_f, core = _planted(rng)
    x = TK.reconstruct(u_t, u_f, core)
    gt, gf, gc = TK.hosvd(x, 5, 4)
    assert np.allclose(TK.reconstruct(gt, gf, gc), x, atol=1e-10)
    # the same subspaces (projectors), orthonormal factors
    assert np.allclose(gt @ gt.T, u_t @ u_t.T, atol=1e-10)
    assert np.allclose(gf @ gf.T, u_f @ u_f.T, atol=1e-10)
    assert np.allclose(gt.T @ gt, np.eye(5), atol=1e-12) and np.allclose(gf.T @ gf, np.eye(4), atol=1e-12)


def test_full_ranks_are_exact_and_matrix_case_is_eckart_young():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((9, 6, 2, 2))
    gt, gf, gc = TK.hosvd(x, 9, 6)
    assert np.allclose(TK.reconstruct(gt, gf, gc), x, atol=1e-12)
    # one head, one layer, the feature mode kept whole: the best rank-r approximation of the T x d matrix
    m = rng.standard_normal((30, 8))
    s = np.linalg.svd(m, compute_uv=False)
    for r in (1, 3, 7):
        gt, gf, gc = TK.hosvd(m[:, :, None, None], r, 8)
        err = np.sum((TK.reconstruct(gt, gf, gc)[:, :, 0, 0] - m) ** 2)
        assert abs(err - np.sum(s[r:] ** 2)) < 1e-9
        # the token mode kept whole instead: the tail of the feature-mode spectrum (the same singular values)
        gt, gf, gc = TK.hosvd(m[:, :, None, None], 30, r)
        err = np.sum((TK.reconstruct(gt, gf, gc)[:, :, 0, 0] - m) ** 2)
        assert abs(err - np.sum(s[r:] ** 2)) < 1e-9


def test_truncated_hosvd_error_bounds():
    # De Lathauwer, De Moor and Vandewalle (2000): the error of the truncated HOSVD lies between the larger of
    # the two modes' discarded energies and their sum
    rng = np.random.default_rng(3)
    u_t, u_f, core = _planted(rng, T=50, d=16, H=2, L=3, r_t=10, r_f=8)
    x = TK.reconstruct(u_t, u_f, core) + 0.3 * rng.standard_normal((50, 16, 2, 3))
    for r_t, r_f in ((4, 3), (10, 8), (12, 16), (50, 5)):
        gt, gf, gc = TK.hosvd(x, r_t, r_f)
        err = np.sum((TK.reconstruct(gt, gf, gc) - x) ** 2)
        e1 = np.sum(np.linalg.svd(TK.unfold(x, 0), compute_uv=False)[r_t:] ** 2)
        e2 = np.sum(np.linalg.svd(TK.unfold(x, 1), compute_uv=False)[r_f:] ** 2)
        assert max(e1, e2) - 1e-9 <= err <= e1 + e2 + 1e-9, (r_t, r_f, err, e1, e2)


def test_unfoldings_hold_the_right_fibres():
    x = np.arange(2 * 3 * 4 * 5, dtype=np.float64).reshape(2, 3, 4, 5)
    u0, u1 = TK.unfold(x, 0), TK.unfold(x, 1)
    assert u0.shape == (2, 60) and u1.shape == (3, 40)
    assert set(u1[2]) == set(x[:, 2].ravel()) and set(u0[1]) == set(x[1].ravel())


def test_gauge_freedom():
    # rotating a factor and counter-rotating the core leaves the tensor unchanged
    rng = np.random.default_rng(4)
    u_t, u_f, core = _planted(rng)
    q, p = _orth(rng, 5, 5), _orth(rng, 4, 4)
    core2 = np.einsum("ac,bj,cjhl->abhl", q.T, p.T, core)
    assert np.allclose(TK.reconstruct(u_t @ q, u_f @ p, core2), TK.reconstruct(u_t, u_f, core), atol=1e-12)


def test_expand_rebuilds_every_key_through_the_latent():
    # k(t, h, l) = W[l][:, h d:(h+1) d]^T u_t[t] must equal the mode products, for non-square shapes in which a
    # transposed operand could not line up
    rng = np.random.default_rng(5)
    T, d, H, L, r_t, r_f = 11, 6, 3, 2, 5, 4
    u_t, u_f, core = _planted(rng, T, d, H, L, r_t, r_f)
    w = TK.expand(u_f, core)
    assert w.shape == (L, r_t, H * d)
    x = TK.reconstruct(u_t, u_f, core)
    for l in range(L):
        for h in range(H):
            k = u_t @ w[l, :, h * d:(h + 1) * d]                   # [T, d]
            assert np.allclose(k, x[:, :, h, l], atol=1e-12)
    # the feature factor the identity: the up-projection is the core slice itself
    core_i = rng.standard_normal((r_t, d, H, L))
    wi = TK.expand(np.eye(d), core_i)
    for l in range(L):
        for h in range(H):
            assert np.array_equal(wi[l, :, h * d:(h + 1) * d], core_i[:, :, h, l])


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7 (bf16 keeps 7 stored fraction bits): to even, 1.0; and
    # 1 + 3 2^-8 rounds up to 1 + 2^-6
    vals = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -2.5, 1 + 2.0 ** -8 + 2.0 ** -30, 3.0e-3])
    bits = TK.to_bf16_bits(vals)
    assert bits.tolist()[:4] == [0x3F80, 0x3F80, 0x3F82, 0xC020]
    assert bits[4] == 0x3F81
    back = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert abs(back[5] - 3.0e-3) <= 2.0 ** -8 * 3.0e-3              # the unit roundoff of 8 significant bits


# ---------------------------------------------------------------- randomized token factor (FlashJoLT reading)

def _svd_matrix(rng, T, D, sig):
    """A = U diag(sig) V^T with random orthonormal U [T, n], V [D, n], n = len(sig)."""
    n = len(sig)
    return _orth(rng, T, n) @ np.diag(sig) @ _orth(rng, D, n).T


def test_orth_is_the_qr_factor_with_positive_diagonal():
    # Q orthonormal, Q^T y upper triangular with a positive diagonal (the definition), and equal to classical
    # Gram-Schmidt in fp64 on a well-conditioned y (an independent route to the same unique factor)
    rng = np.random.default_rng(20)
    y = rng.standard_normal((50, 7))
    q = TK.orth(y)
    r = q.T @ y
    assert np.allclose(q.T @ q, np.eye(7), atol=1e-13)
    assert np.allclose(np.tril(r, -1), 0, atol=1e-12) and (np.diag(r) > 0).all()
    assert np.allclose(q @ r, y, atol=1e-12)
    gs = np.zeros_like(y)
    for j in range(7):
        v = y[:, j] - gs[:, :j] @ (gs[:, :j].T @ y[:, j])
        gs[:, j] = v / np.linalg.norm(v)
    assert np.allclose(q, gs, atol=1e-12)


@pytest.mark.parametrize("q", [0, 1, 3])
def test_randomized_range_is_exact_on_planted_rank(q):
    # rank(A) = k = sketch width: the range is recovered exactly whatever q
    rng = np.random.default_rng(21)
    a = _svd_matrix(rng, 200, 60, np.linspace(5.0, 0.5, 8))
    u = np.linalg.svd(a, full_matrices=False)[0][:, :8]
    Q = TK.randomized_range(a, rng.standard_normal((60, 8)), q)
    assert np.allclose(Q.T @ Q, np.eye(8), atol=1e-12)
    assert np.allclose(Q @ Q.T, u @ u.T, atol=1e-9)


@pytest.mark.parametrize("q", [0, 1, 2])
def test_randomized_range_within_the_deterministic_bound(q):
    # Halko, Martinsson & Tropp (2011), Theorem 9.1 (Frobenius form), for the sketch width k = target rank: with
    # Omega_1 = V_1^T Omega (k x k, invertible almost surely) and Omega_2 = V_2^T Omega,
    #   |(I - QQ^T) B|_F^2 <= |S_2|_F^2 + |S_2 Omega_2 Omega_1^-1|_F^2
    # for B with singular values S; applied to B = (A A^T)^q A, singular values sigma^(2q+1), whose sketch the
    # power scheme computes.  A slowly decaying spectrum, five draws of Omega.
    rng = np.random.default_rng(22)
    T, D, k = 300, 80, 10
    sig = 4.0 * (1.0 + np.arange(D)) ** -0.6
    U, V = _orth(rng, T, D), _orth(rng, D, D)
    a = U @ np.diag(sig) @ V.T
    s_q = sig ** (2 * q + 1)
    b = U @ np.diag(s_q) @ V.T
    for _ in range(5):
        om = rng.standard_normal((D, k))
        Q = TK.randomized_range(a, om, q)
        err2 = np.sum(((np.eye(T) - Q @ Q.T) @ b) ** 2)
        o1, o2 = V[:, :k].T @ om, V[:, k:].T @ om
        bound2 = np.sum(s_q[k:] ** 2) + np.sum((np.diag(s_q[k:]) @ o2 @ np.linalg.inv(o1)) ** 2)
        assert err2 <= bound2 * (1 + 1e-9), (err2, bound2)
        assert err2 >= np.sum(s_q[k:] ** 2) * (1 - 1e-9)     # never better than the optimal rank-k subspace


def test_power_iterations_converge_to_the_leading_subspace():
    # a gap sigma_{k+1} / sigma_k = 0.5: the largest principal angle between range(Q) and the leading k left
    # singular vectors obeys tan(theta) <= |S_2^(2q+1) Omega_2 Omega_1^-1 S_1^-(2q+1)|_2 and shrinks with q
    rng = np.random.default_rng(23)
    T, D, k = 250, 60, 6
    sig = np.concatenate([np.linspace(4.0, 2.0, k), 1.0 * 0.97 ** np.arange(D - k)])
    U, V = _orth(rng, T, D), _orth(rng, D, D)
    a = U @ np.diag(sig) @ V.T
    om = rng.standard_normal((D, k))
    o1, o2 = V[:, :k].T @ om, V[:, k:].T @ om
    prev = None
    for q in range(5):
        Q = TK.randomized_range(a, om, q)
        sin_max = np.linalg.norm(Q - U[:, :k] @ (U[:, :k].T @ Q), 2)   # |(I - U_k U_k^T) Q|_2
        e = 2 * q + 1
        tan_b = np.linalg.norm(np.diag(sig[k:] ** e) @ o2 @ np.linalg.inv(o1) @ np.diag(sig[:k] ** -e), 2)
        assert sin_max <= tan_b / np.sqrt(1 + tan_b ** 2) + 1e-10
        if prev is not None:
            assert sin_max < prev
        prev = sin_max
    assert prev < 1e-2


def test_unfolding_column_order_pairs_with_omega_rows():
    # permuting the unfolding's columns and Omega's rows alike changes nothing
    rng = np.random.default_rng(24)
    a = rng.standard_normal((90, 40))
    om = rng.standard_normal((40, 5))
    perm = rng.permutation(40)
    assert np.allclose(TK.randomized_range(a, om, 1), TK.randomized_range(a[:, perm], om[perm], 1), atol=1e-12)


def test_fit_randomized_on_a_planted_group():
    # a planted partial Tucker tensor (token rank 5, feature rank 4) in the [T, L, H, d] layout: exact
    # reconstruction, the feature factor of the exact HOSVD, and the core equal to the projection computed
    # element by element
    rng = np.random.default_rng(25)
    T, L, H, d, r_t, r_f = 40, 2, 3, 12, 5, 4
    u_t, u_f, core = _planted(rng, T=T, d=d, H=H, L=L, r_t=r_t, r_f=r_f)
    xs = TK.reconstruct(u_t, u_f, core)                    # [T, d, H, L]
    x = np.transpose(xs, (0, 3, 2, 1))                     # [T, L, H, d]
    om = rng.standard_normal((L * H * d, r_t))
    gt, gf, gc = TK.fit_randomized(x, r_t, r_f, om, 1)
    assert gc.shape == (L, H, r_t, r_f)
    assert np.allclose(TK.reconstruct(gt, gf, TK.core_to_hosvd_layout(gc)), xs, atol=1e-10)
    assert np.allclose(gf, TK.hosvd(xs, r_t, r_f)[1], atol=1e-10)
    assert np.allclose(gt @ gt.T, u_t @ u_t.T, atol=1e-9)
    for l, h, c, j in [(0, 0, 0, 0), (1, 2, 4, 3), (0, 1, 2, 1), (1, 0, 3, 2)]:
        want = sum(gt[t, c] * gf[i, j] * x[t, l, h, i] for t in range(T) for i in range(d))
        assert abs(gc[l, h, c, j] - want) < 1e-10

"""Pins of the oracle's inverse roots, scaling and iterations (CPU only).

Each check compares the oracle with something other than itself: closed forms
(diagonal and scaled-identity inputs, Q diag(lambda) Q^T built from its
factors), the defining identity X^p A = I, scalar recurrences evaluated on the
eigenvalues, exact polynomial reproduction and the product counts the pages
state.
"""

import numpy as np
import pytest

import oracle
import synthetic


def rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


@pytest.mark.parametrize("p", [2, 4])
def test_eigh_root_diagonal_and_identity(p):
    lam = np.array([3.0, 1.0, 0.25, 1e-3, 7.5])
    X = oracle.inverse_root_eigh(np.diag(lam), p)
    assert np.allclose(X, np.diag(lam ** (-1.0 / p)), rtol=1e-14, atol=0)
    c = 0.37
    Y = oracle.inverse_root_eigh(c * np.eye(6), p)
    assert np.allclose(Y, c ** (-1.0 / p) * np.eye(6), rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("p", [2, 4])
def test_eigh_root_closed_form_spd(p):
    A, lam, Q = synthetic.spd_stack(11, 3, 48, 1e-6, 1.0, return_factors=True)
    for i in range(3):
        X = oracle.inverse_root_eigh(A[i], p)
        want = (Q[i] * lam[i] ** (-1.0 / p)) @ Q[i].T
        assert rel(X, want) < 1e-9
        # defining identity, symmetry, positive definiteness
        assert oracle.residual(X, A[i], p) < 1e-9
        assert np.allclose(X, X.T, atol=1e-12 * np.abs(X).max())
        assert np.linalg.eigvalsh(X).min() > 0


def test_eigh_root_eps_added_once():
    # rank-deficient PSD factor: eigenvalues (lambda + eps)^(-1/4), eps only once
    gen = np.random.default_rng(3)
    G = gen.standard_normal((12, 5))
    L = G @ G.T
    eps = 1e-3
    lam, Q = np.linalg.eigh(L)
    lam = np.clip(lam, 0, None)
    want = (Q * (lam + eps) ** -0.25) @ Q.T
    assert rel(oracle.inverse_root_eigh(L, 4, eps), want) < 1e-10


def test_frobenius_bounds_lambda_max():
    A, lam, _ = synthetic.spd_stack(5, 4, 64, 1e-6, 1.0, return_factors=True)
    for i in range(4):
        s = oracle.frobenius_scale(A[i])
        assert s >= lam[i].max() * (1 - 1e-12)
        assert np.isclose(s, np.sqrt(np.sum(lam[i] ** 2)), rtol=1e-12)
    assert np.isclose(oracle.frobenius_scale(np.zeros((3, 3)), 0.5), 0.5 * np.sqrt(3))


def test_power_iteration_bounds_and_exactness():
    # exact on a diagonal input when a start vector is the top eigenvector
    D = np.diag([3.0, 1.0, 0.5, 0.25])
    V0 = np.array([[0.0, 1.0, 1.0, 0.0], [1.0, 0.0, 0.0, 0.0]])
    rho, j, rq = oracle.power_iteration(D, V0, 10, half_operands=False)
    assert rho == 3.0 and j == 1
    # Rayleigh quotients never exceed lambda_max; they approach it with a gap
    A, lam, _ = synthetic.spd_stack(7, 3, 96, 1e-4, 1.0, return_factors=True)
    V0 = synthetic.pi_start_vectors(1, 16, 96)
    for i in range(3):
        lmax = lam[i].max()
        rho, _, rq = oracle.power_iteration(A[i], V0, 10, half_operands=False)
        assert (rq <= lmax * (1 + 1e-12)).all()
        rho200, _, _ = oracle.power_iteration(A[i], V0, 400, half_operands=False)
        assert abs(rho200 - lmax) / lmax < 1e-6
        # half-precision operands: a Rayleigh quotient of the rounded matrix
        Ah = A[i].astype(np.float16).astype(np.float64)
        rhoh, _, _ = oracle.power_iteration(A[i], V0, 10, half_operands=True)
        assert rhoh <= np.linalg.eigvalsh(Ah).max() * (1 + 1e-12)
        assert abs(rhoh - lmax) / lmax < 0.2


def test_power_iteration_half_branch_hand_rounded():
    """The half-precision branch on a 3 x 3 case rounded by hand.

    IEEE half keeps 11 significant bits, so x in [2^e, 2^(e+1)) rounds to a
    multiple of 2^(e-10), ties to even.  The matrix entries:
      0.1 in [2^-4, 2^-3): 0.1 * 2^14 = 1638.4 -> 1638 / 2^14 = 819 / 8192;
      0.3 in [2^-2, 2^-1): 0.3 * 2^12 = 1228.8 -> 1229 / 4096;
      1, 0.5 and 0.25 are exact.
    Start vector (1, 2, 3) / sqrt(14) = (0.26726, 0.53452, 0.80178):
      0.26726 * 2^12 = 1094.70 -> 1095 / 4096;
      0.53452 * 2^11 = 1094.70 -> 1095 / 2048;
      0.80178 * 2^11 = 1642.05 -> 1642 / 2048 = 821 / 1024.
    One product with the rounded matrix, normalised, gives
    (0.44530, 0.74214, 0.50093), rounded in turn:
      0.44530 * 2^12 = 1823.95 -> 1824 / 4096 = 57 / 128;
      0.74214 * 2^11 = 1519.90 -> 1520 / 2048 = 95 / 128;
      0.50093 * 2^11 = 1025.91 -> 1026 / 2048 = 513 / 1024.
    The Rayleigh quotient of that rounded vector with the rounded matrix is
    the oracle's answer.  Without the roundings it differs by 2e-5, so a
    rounding skipped or taken in another place fails the 1e-13 check."""
    A = np.array([[1.0, 0.1, 0.0], [0.1, 0.5, 0.3], [0.0, 0.3, 0.25]])
    Am = np.array([[1.0, 819 / 8192, 0.0], [819 / 8192, 0.5, 1229 / 4096], [0.0, 1229 / 4096, 0.25]])
    v0 = np.array([1095 / 4096, 1095 / 2048, 821 / 1024])
    v1 = Am @ v0
    v1 = v1 / np.linalg.norm(v1)
    assert np.allclose(v1, [0.44530, 0.74214, 0.50093], atol=5e-6)  # the values rounded above
    v1h = np.array([57 / 128, 95 / 128, 513 / 1024])
    w = Am @ v1h
    want = float(v1h @ w / (v1h @ v1h))
    rho, j, rq = oracle.power_iteration(A, np.array([[1.0, 2.0, 3.0]]), 1, half_operands=True)
    assert j == 0 and abs(rho - want) <= 1e-13 * want
    rho_full, _, _ = oracle.power_iteration(A, np.array([[1.0, 2.0, 3.0]]), 1, half_operands=False)
    assert abs(rho_full - want) > 1e-5 * want


@pytest.mark.parametrize("p", [2, 4])
def test_cn_scalar_and_matrix(p):
    a = np.logspace(-6, 0, 25)
    x = oracle.cn_scalar(a, p, 40)
    assert np.allclose(x, a ** (-1.0 / p), rtol=1e-12)
    A, lam, Q = synthetic.spd_stack(12, 2, 32, 1e-4, 1.0, return_factors=True)
    s = oracle.frobenius_scale(A[0])
    for k in (3, 9, 30):
        Xk = oracle.cn_matrix(A[0] / s, p, k)
        want = (Q[0] * oracle.cn_scalar(lam[0] / s, p, k)) @ Q[0].T
        assert rel(Xk, want) < 1e-9
    assert rel(oracle.cn_matrix(A[0] / s, p, 30) * s ** (-1.0 / p),
               oracle.inverse_root_eigh(A[0], p)) < 1e-9


def test_ndb_scalar_matrix_and_count():
    a = np.logspace(-8, 0, 30)
    y, z = oracle.ndb_scalar(a, 40)
    assert np.allclose(y, np.sqrt(a), rtol=1e-12) and np.allclose(z, 1 / np.sqrt(a), rtol=1e-12)
    A, lam, Q = synthetic.spd_stack(13, 2, 32, 1e-4, 1.0, return_factors=True)
    s = oracle.frobenius_scale(A[0])
    for k in (1, 4, 25):
        cnt = [0]
        Y, Z = oracle.ndb_matrix(A[0] / s, k, cnt)
        ys, zs = oracle.ndb_scalar(lam[0] / s, k)
        assert rel(Y, (Q[0] * ys) @ Q[0].T) < 1e-9
        assert rel(Z, (Q[0] * zs) @ Q[0].T) < 1e-9
        # three products per iteration, the first two cheaper
        assert cnt[0] == 3 * k - 2
    cnt = [0]
    X = oracle.ndb_inverse_root_matrix(A[0] / s, 4, 25, 20, cnt)
    assert cnt[0] == (3 * 25 - 2) + (3 * 20 - 2)
    assert rel(X * s ** -0.25, (Q[0] * lam[0] ** -0.25) @ Q[0].T) < 1e-9
    X2 = oracle.ndb_inverse_root_matrix(A[0] / s, 2, 25)
    assert rel(X2 * s ** -0.5, (Q[0] * lam[0] ** -0.5) @ Q[0].T) < 1e-9


def test_chebyshev_scalar_closed_form():
    c = np.array([0.3, -1.2, 0.7, 0.05, 2.0])
    th = np.linspace(0, np.pi, 37)
    t = np.cos(th)
    want = sum(ck * np.cos(k * th) for k, ck in enumerate(c))
    assert np.allclose(oracle.chebyshev_scalar(c, t), want, atol=1e-13)


def test_chebyshev_fit_reproduces_polynomials():
    eps = 0.01
    d = 6
    # f given in x through t = 2 (x - eps) - 1: f = T_3(t) + 0.5 T_1(t) - 0.25
    def f(x):
        t = 2.0 * (x - eps) - 1.0
        return 4 * t ** 3 - 3 * t + 0.5 * t - 0.25
    c = oracle.chebyshev_coefficients(4, d, eps, f=f)
    want = np.zeros(d + 1)
    want[0], want[1], want[3] = -0.25, 0.5, 1.0
    assert np.allclose(c, want, atol=1e-14)


def test_chebyshev_fit_accuracy_smooth_case():
    # x^(-1/4) on [0.1, 1.1] is analytic inside the Bernstein ellipse through the
    # singularity at t = -1.2 (rho = 1.2 + sqrt(0.44) ~ 1.86): the fit error
    # falls geometrically, like rho^(-d)
    eps, p = 0.1, 4
    x = np.linspace(0.0, 1.0, 1001)
    f = (x + eps) ** (-1.0 / p)
    err = {}
    for d in (16, 32):
        c = oracle.chebyshev_coefficients(p, d, eps)
        err[d] = np.max(np.abs(oracle.chebyshev_scalar(c, 2 * x - 1) - f) / f)
    rho = 1.2 + np.sqrt(1.2 ** 2 - 1)
    assert err[16] < 10 * rho ** -16
    assert err[32] < 10 * rho ** -32


def test_clenshaw_matrix_equals_polynomial_and_counts():
    A, lam, Q = synthetic.spd_stack(14, 1, 40, 1e-3, 1.0, return_factors=True)
    s = oracle.frobenius_scale(A[0])
    As = A[0] / s
    S = 2 * As - np.eye(40)
    for d in (2, 5, 16):
        c = oracle.chebyshev_coefficients(4, d, 1e-3)
        cnt = [0]
        P = oracle.clenshaw_matrix(S, c, cnt)
        assert cnt[0] == d - 1
        want = (Q[0] * oracle.chebyshev_scalar(c, 2 * lam[0] / s - 1)) @ Q[0].T
        assert rel(P, want) < 1e-10
        assert rel(oracle.chebyshev_matrix_eigh(As, c), want) < 1e-10
    # the coefficients of t^2 = (T_0 + T_2)/2 give S^2 exactly
    P2 = oracle.clenshaw_matrix(S, np.array([0.5, 0.0, 0.5]))
    assert np.allclose(P2, S @ S, atol=1e-14)


def test_iteration_exact_root_matches_matrix_iterations():
    A = synthetic.spd_stack(15, 1, 24, 1e-3, 1.0)[0]
    s = oracle.frobenius_scale(A)
    Xcn = oracle.iteration_exact_root(A, 4, "cn", s, iters=6)
    assert rel(Xcn, oracle.cn_matrix(A / s, 4, 6) * s ** -0.25) < 1e-10
    Xndb = oracle.iteration_exact_root(A, 4, "ndb", s, iters=5, iters2=4)
    assert rel(Xndb, oracle.ndb_inverse_root_matrix(A / s, 4, 5, 4) * s ** -0.25) < 1e-10
    c = oracle.chebyshev_coefficients(4, 9, 1e-3)
    Xch = oracle.iteration_exact_root(A, 4, "chebyshev", s, coeffs=c)
    assert rel(Xch, oracle.clenshaw_matrix(2 * A / s - np.eye(24), c) * s ** -0.25) < 1e-10

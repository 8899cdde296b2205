"""Pins of the oracle's statistics, preconditioning, grafting and full step.

The direction is checked against a brute-force Kronecker construction (the
(m n) x (m n) matrix ((L + eps I) (x) (R + eps I))^(-1/4) applied to the
row-major vec of G, via scipy's Schur-Pade fractional power), against the
step-1 closed form through the SVD of G, and the grafting against its norm
invariant and the Adam step-1 closed form.
"""

import numpy as np
import pytest
import scipy.linalg

import oracle
import synthetic


def rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


def test_stats_integer_sums_and_ema_weights():
    gen = np.random.default_rng(0)
    G = [gen.integers(-3, 4, size=(5, 7)).astype(np.float64) for _ in range(3)]
    L, R = np.zeros((5, 5)), np.zeros((7, 7))
    for g in G:
        L, R = oracle.update_stats(L, R, g, 1.0)
    # exact integer arithmetic: explicit double sums
    for i in range(5):
        for j in range(5):
            assert L[i, j] == sum(g[i, k] * g[j, k] for g in G for k in range(7))
    for i in range(7):
        for j in range(7):
            assert R[i, j] == sum(g[k, i] * g[k, j] for g in G for k in range(5))
    # EMA with a constant gradient: L_t = (1 - beta2^t) G G^T
    b2 = 0.9
    L, R = np.zeros((5, 5)), np.zeros((7, 7))
    for _ in range(4):
        L, R = oracle.update_stats(L, R, G[0], b2)
    assert np.allclose(L, (1 - b2 ** 4) * G[0] @ G[0].T, rtol=1e-13)


# Rectangular blocks have rank-deficient factors: eps = 1e-12 would make the
# (m n)-sized Kronecker matrix too ill-conditioned for the brute-force route
# itself, so they take a large eps; square blocks take the tiny one.
@pytest.mark.parametrize("m,n,eps", [(3, 5, 1e-2), (4, 6, 1e-2), (6, 4, 0.5), (4, 4, 1e-12), (5, 5, 1e-12)])
def test_direction_matches_bruteforce_kronecker(m, n, eps):
    gen = np.random.default_rng(m * 10 + n)
    shapes = [(m, n)]
    opt = oracle.ShampooOracle(shapes, [max(m, n)], beta2=1.0, eps=eps, graft="sgd", lr=0.1)
    W = [np.zeros((m, n))]
    Gs = [gen.standard_normal((m, n)) for _ in range(2)]
    Lsum, Rsum = np.zeros((m, m)), np.zeros((n, n))
    for G in Gs:
        D, _ = opt.step(W, [G])
        Lsum += G @ G.T
        Rsum += G.T @ G
        K = np.kron(Lsum + eps * np.eye(m), Rsum + eps * np.eye(n))
        Kr = np.real(scipy.linalg.fractional_matrix_power(K, -0.25))
        want = (Kr @ G.reshape(-1)).reshape(m, n)
        assert rel(D[0], want) < 1e-7


def test_step1_polar_closed_form_and_sgd_graft():
    gen = np.random.default_rng(4)
    n = 16
    G = gen.standard_normal((n, n))
    U, sig, Vt = np.linalg.svd(G)
    for beta2, eps in ((1.0, 1e-12), (0.999, 1e-12), (1.0, 0.3)):
        opt = oracle.ShampooOracle([(n, n)], [n], beta2=beta2, eps=eps, graft="sgd", lr=0.1)
        W = [np.zeros((n, n))]
        D, Dg = opt.step(W, [G])
        w = 1.0 if beta2 == 1.0 else 1.0 - beta2
        want = (U * (sig / np.sqrt(w * sig ** 2 + eps))) @ Vt
        assert rel(D[0], want) < 1e-8
        # grafted to the SGD step length
        assert np.isclose(np.linalg.norm(Dg[0]), np.linalg.norm(G), rtol=1e-13)
        assert np.allclose(W[0], -0.1 * Dg[0], rtol=0, atol=1e-15)


def test_blocks_are_independent_shampoos():
    gen = np.random.default_rng(5)
    shapes = [(7, 10)]
    B = 4
    opt = oracle.ShampooOracle(shapes, [B], beta2=1.0, eps=1e-3, graft="sgd")
    G = gen.standard_normal((7, 10))
    D, _ = opt.step([np.zeros((7, 10))], [G])
    t = oracle.plan_blocks(shapes, [B])
    for b in range(t.shape[0]):
        rs, cs = oracle.block_slices(t, b)
        g = G[rs, cs]
        mm, nn = g.shape
        K = np.kron(g @ g.T + 1e-3 * np.eye(mm), g.T @ g + 1e-3 * np.eye(nn))
        Kr = np.real(scipy.linalg.fractional_matrix_power(K, -0.25))
        assert rel(D[0][rs, cs], (Kr @ g.reshape(-1)).reshape(mm, nn)) < 1e-7


def test_adam_graft_step1_and_norm_invariant():
    gen = np.random.default_rng(6)
    shapes = [(6, 9), (9, 4)]
    opt = oracle.ShampooOracle(shapes, [8, 8], beta2=0.999, eps=1e-12, graft="adam", lr=1e-3)
    W = [np.zeros(s) for s in shapes]
    G = [gen.standard_normal(s) for s in shapes]
    D, Dg = opt.step(W, G)
    for p in range(2):
        delta1 = G[p] / (np.abs(G[p]) + 1e-8)  # Adam's first step: m_hat = G, v_hat = G^2
        assert np.isclose(np.linalg.norm(Dg[p]), np.linalg.norm(delta1), rtol=1e-12)
        assert np.allclose(Dg[p] / np.linalg.norm(Dg[p]), D[p] / np.linalg.norm(D[p]), atol=1e-14)
        assert np.allclose(W[p], -1e-3 * Dg[p], atol=1e-18)


def test_adam_graft_constant_gradient_every_step():
    """A constant gradient G gives m_t = (1 - beta1^t) G and v_t = (1 - beta2^t)
    G^2, so the bias-corrected direction is G / (|G| + eps_g) at every t.  A
    state that is not carried between steps, or a bias correction taken at a
    fixed t, leaves m_hat != G from t = 2 on."""
    gen = np.random.default_rng(9)
    G = gen.standard_normal((4, 6))
    want = G / (np.abs(G) + 1e-8)
    state = {"m": np.zeros((4, 6)), "v": np.zeros((4, 6))}
    for t in range(1, 6):
        d = oracle.graft_direction("adam", G, state, t, beta1=0.9, beta2=0.999, eps_g=1e-8)
        assert np.allclose(d, want, rtol=1e-12, atol=0)
    # through the step: the grafted norm is ||G / (|G| + eps_g)|| at every step
    opt = oracle.ShampooOracle([(4, 6)], [8], beta2=0.999, eps=1e-12, graft="adam", lr=1e-3)
    W = [np.zeros((4, 6))]
    for t in range(5):
        _, Dg = opt.step(W, [G])
        assert np.isclose(np.linalg.norm(Dg[0]), np.linalg.norm(want), rtol=1e-12)


def test_adam_graft_two_steps_hand_computed():
    """Two steps with different gradients, beta1 = 1/2, beta2 = 3/4, eps_g = 0:
    m_1 = G_1/2 = (1, -1/2), v_1 = G_1^2/4 = (1, 1/4);
    m_2 = m_1/2 + G_2/2 = (5/2, 5/4), v_2 = 3 v_1/4 + G_2^2/4 = (19/4, 39/16);
    m_hat = m_2 / (1 - 1/4) = (10/3, 5/3), v_hat = v_2 / (1 - 9/16) = (76/7, 39/7);
    Delta_2 = m_hat / sqrt(v_hat)."""
    G1, G2 = np.array([[2.0, -1.0]]), np.array([[4.0, 3.0]])
    state = {"m": np.zeros((1, 2)), "v": np.zeros((1, 2))}
    d1 = oracle.graft_direction("adam", G1, state, 1, beta1=0.5, beta2=0.75, eps_g=0.0)
    assert np.allclose(d1, [[1.0, -1.0]], rtol=1e-15)
    d2 = oracle.graft_direction("adam", G2, state, 2, beta1=0.5, beta2=0.75, eps_g=0.0)
    want = np.array([[(10 / 3) / np.sqrt(76 / 7), (5 / 3) / np.sqrt(39 / 7)]])
    assert np.allclose(d2, want, rtol=1e-14, atol=0)
    assert np.allclose(state["m"], [[2.5, 1.25]], rtol=1e-15) and np.allclose(state["v"], [[4.75, 2.4375]], rtol=1e-15)
    # the same two steps through the oracle's step: the grafted step has
    # ||Delta_2|| as its norm and D's direction
    opt = oracle.ShampooOracle([(1, 2)], [2], beta2=0.999, eps=1e-12, graft="adam", lr=1.0, beta1=0.5,
                               graft_beta2=0.75, eps_g=0.0)
    W = [np.zeros((1, 2))]
    opt.step(W, [G1])
    D, Dg = opt.step(W, [G2])
    assert np.isclose(np.linalg.norm(Dg[0]), np.linalg.norm(want), rtol=1e-13)
    assert np.allclose(Dg[0] / np.linalg.norm(Dg[0]), D[0] / np.linalg.norm(D[0]), atol=1e-14)


def test_momentum_graft_two_steps():
    gen = np.random.default_rng(7)
    shapes = [(5, 8)]
    opt = oracle.ShampooOracle(shapes, [8], beta2=0.999, eps=1e-12, graft="momentum", lr=0.1, momentum=0.9)
    W = [np.zeros((5, 8))]
    G1, G2 = gen.standard_normal((5, 8)), gen.standard_normal((5, 8))
    _, Dg1 = opt.step(W, [G1])
    assert np.isclose(np.linalg.norm(Dg1[0]), np.linalg.norm(G1), rtol=1e-12)
    _, Dg2 = opt.step(W, [G2])
    M = 0.9 * Dg1[0] + Dg2[0]
    assert np.allclose(W[0], -0.1 * Dg1[0] - 0.1 * M, atol=1e-14)


def test_blockwise_graft_and_no_graft():
    """Block-wise grafting: each block's D_g has the norm of its slice of
    Delta and D's direction; with one block per parameter it is the
    layer-wise graft.  Graft "none" steps along D itself."""
    gen = np.random.default_rng(8)
    shapes = [(10, 7), (5, 12)]
    G = [gen.standard_normal(s) for s in shapes]
    for graft in ("sgd", "adam"):
        opt = oracle.ShampooOracle(shapes, [4, 4], beta2=0.9, eps=1e-6, graft=graft, lr=0.1, graft_blockwise=True)
        W = [np.zeros(s) for s in shapes]
        D, Dg = opt.step(W, G)
        for b in range(opt.table.shape[0]):
            p = int(opt.table[b, 0])
            rs, cs = oracle.block_slices(opt.table, b)
            delta = G[p] if graft == "sgd" else G[p] / (np.abs(G[p]) + 1e-8)
            assert np.isclose(np.linalg.norm(Dg[p][rs, cs]), np.linalg.norm(delta[rs, cs]), rtol=1e-12)
            u, v = Dg[p][rs, cs].ravel(), D[p][rs, cs].ravel()
            assert np.isclose(u @ v, np.linalg.norm(u) * np.linalg.norm(v), rtol=1e-12)
        for p in range(2):
            assert np.allclose(W[p], -0.1 * Dg[p], atol=1e-15)
    # one block per parameter: block-wise = layer-wise
    one = [oracle.ShampooOracle(shapes, [16, 16], beta2=0.9, eps=1e-6, graft="sgd", lr=0.1, graft_blockwise=bw)
           for bw in (False, True)]
    Ws = [[np.zeros(s) for s in shapes] for _ in one]
    for o, W in zip(one, Ws):
        o.step(W, G)
    for p in range(2):
        np.testing.assert_array_equal(Ws[0][p], Ws[1][p])
    # graft "none": W <- W - lr D
    opt = oracle.ShampooOracle(shapes, [4, 4], beta2=0.9, eps=1e-6, graft="none", lr=0.1)
    W = [np.zeros(s) for s in shapes]
    D, Dg = opt.step(W, G)
    for p in range(2):
        np.testing.assert_array_equal(Dg[p], D[p])
        assert np.allclose(W[p], -0.1 * D[p], atol=1e-15)


def test_chebyshev_step_tends_to_shifted_root():
    # The fit approximates (x + eps)^(-1/4) on the Frobenius-scaled spectrum x of
    # L + eps I: with a large degree the step tends to
    # ((L + eps I)/s + eps I)^(-1/4) s^(-1/4) on each side.
    gen = np.random.default_rng(8)
    n, eps = 12, 1e-2
    G = gen.standard_normal((n, n)) + 3 * np.eye(n)
    o_cheb = oracle.ShampooOracle([(n, n)], [n], beta2=1.0, eps=eps, root="chebyshev", cheb_degree=60)
    D, _ = o_cheb.step([np.zeros((n, n))], [G])

    def side(F):
        A = F + eps * np.eye(n)
        s = np.linalg.norm(A)
        lam, Q = np.linalg.eigh(A)
        return (Q * (lam / s + eps) ** -0.25) @ Q.T * s ** -0.25

    want = side(G @ G.T) @ G @ side(G.T @ G)
    assert rel(D[0], want) < 1e-4


def test_zero_gradient_gives_zero_step():
    opt = oracle.ShampooOracle([(4, 4)], [4], beta2=1.0, eps=1e-12, graft="sgd")
    W = [np.ones((4, 4))]
    D, Dg = opt.step(W, [np.zeros((4, 4))])
    assert not np.any(D[0]) and not np.any(Dg[0]) and np.all(W[0] == 1.0)


def test_oracle_and_product_share_nothing():
    import os
    import re
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    for d, pat in (("oracle", r"matrix_inverse_roots_amd"), ("matrix_inverse_roots_amd", r"\boracle\b")):
        for dirpath, _, files in os.walk(os.path.join(root, d)):
            for f in files:
                if f.endswith((".py", ".hip", ".h", ".hpp", ".cpp", ".c")):
                    src = open(os.path.join(dirpath, f)).read()
                    assert not re.search(r"^\s*(from|import)\s+" + pat, src, re.M), (f, pat)
                    assert "#include" not in src or not re.search(r'#include\s+"[^"]*' + pat, src)

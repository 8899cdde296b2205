"""Inverse p-th roots of SPD blocks: limit oracle and literal iterations.

Oracle; test infrastructure only.  float64 numpy throughout.

* Limit oracle ([DASH] "B.1 Regularization (dampening) for EVD"; [NOTES]
  "Spreading the preconditioners across GPUs"): eigendecompose L + eps*I once,
  lift the eigenvalues to at least eps, and return Q diag(lambda^(-1/p)) Q^T.
  eps is added exactly once (the B.1 section warns against adding it twice).
* Scaling ([DASH] "3. Inverse Root Methods", "Matrix scaling" and
  "Power-Iteration"): divide by the Frobenius norm, or by the largest Rayleigh
  quotient over a set of power-iteration start vectors run in half precision.
* Coupled Newton ([NOTES] "Roots on idle CPUs, partial preconditioners for
  large layers, and grafting": the coupled iteration of Guo-Higham and
  Iannazzo).  X_0 = I, M_0 = A_s; T = ((p+1) I - M)/p; X <- X T; M <- T^p M.
  X tends to A_s^(-1/p).
* Newton-DB ([DASH] "3. Inverse Root Methods", "Newton-DB": three products per
  iteration, the first iteration two cheaper, the fourth root by chaining two
  calls).  Y_0 = A_s, Z_0 = I; T = (3 I - Z Y)/2; Y <- Y T; Z <- T Z.  Y tends
  to A_s^(1/2) and Z to A_s^(-1/2).  The fourth root feeds the first call's Y
  (spectrum inside (0, 1]) to the second call and returns its Z.
* Chebyshev ([DASH] "A.1/A.2 Chebyshev polynomials"): coefficients fitted once
  on [eps, 1 + eps] for x^(-1/p); the scaled matrix (spectrum in [0, 1]) is
  mapped to [-1, 1] by S = 2 A_s - I and the series is summed by Clenshaw's
  recurrence started at B_d, B_(d-1) and stopped at B_1 (d - 1 products).

Readings taken where the pages are silent (each listed in the design notes):
the Chebyshev fit uses N = 4(d + 1) first-kind nodes and the discrete Chebyshev
transform; the power iteration runs ``iters`` products with column
normalisation, then one more product for the Rayleigh quotients, picking the
largest (lowest index on ties) with no safety factor.
"""

import numpy as np


def _sym(A):
    return 0.5 * (A + A.T)


def regularize(A, eps):
    """A + eps * I."""
    A = np.asarray(A, dtype=np.float64)
    return A + eps * np.eye(A.shape[0])


def frobenius_scale(A, eps=0.0):
    """s = ||A + eps I||_F  ([DASH] "3. Inverse Root Methods", "Matrix scaling")."""
    return float(np.linalg.norm(regularize(A, eps), "fro"))


def _round_half(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def _normalize_cols(V):
    n = np.sqrt(np.sum(V * V, axis=0))
    n = np.where(n > 0, n, 1.0)
    return V / n


def power_iteration(Af, V0, iters, half_operands=True):
    """Multi-start power iteration on a (pre-scaled) symmetric matrix.

    Af: [b, b] symmetric; V0: [k, b] start vectors (one per row).  Each of the
    ``iters`` steps normalises every column of V and multiplies by Af; a final
    product gives the Rayleigh quotients v_j^T Af v_j / v_j^T v_j of the
    normalised vectors.  With ``half_operands`` the matrix and the vectors are
    rounded to IEEE half before every product (the pages' half-precision
    multi-power-iteration), products and sums being exact float64 here.

    Returns (largest Rayleigh quotient, index of the start vector giving it,
    all Rayleigh quotients).
    """
    Af = np.asarray(Af, dtype=np.float64)
    Am = _round_half(Af) if half_operands else Af
    V = np.asarray(V0, dtype=np.float64).T.copy()
    for _ in range(iters):
        Vn = _normalize_cols(V)
        if half_operands:
            Vn = _round_half(Vn)
        V = Am @ Vn
    Vn = _normalize_cols(V)
    if half_operands:
        Vn = _round_half(Vn)
    W = Am @ Vn
    num = np.sum(Vn * W, axis=0)
    den = np.sum(Vn * Vn, axis=0)
    rq = np.where(den > 0, num / np.where(den > 0, den, 1.0), 0.0)
    j = int(np.argmax(rq))  # argmax returns the lowest index among ties
    return float(rq[j]), j, rq


def inverse_root_eigh(A, p, eps=0.0):
    """Limit oracle: (A + eps I)^(-1/p) by symmetric eigendecomposition.

    Eigenvalues are lifted to at least eps (no second shift).  With eps = 0 a
    non-positive eigenvalue gives an infinite root, which is the caller's
    problem: the synthetic inputs are SPD.
    """
    lam, Q = np.linalg.eigh(_sym(regularize(A, eps)))
    lam = np.maximum(lam, eps)
    with np.errstate(divide="ignore"):
        d = lam ** (-1.0 / p)
    return (Q * d) @ Q.T


def residual(X, A, p):
    """||X^p A - I||_F / sqrt(b): how well X inverts the p-th root of A."""
    X = np.asarray(X, dtype=np.float64)
    A = np.asarray(A, dtype=np.float64)
    b = A.shape[0]
    return float(np.linalg.norm(np.linalg.matrix_power(X, p) @ A - np.eye(b), "fro") / np.sqrt(b))


# ----------------------------------------------------------------------------
# Coupled Newton
# ----------------------------------------------------------------------------

def cn_matrix(As, p, iters):
    """Coupled Newton for As^(-1/p), float64 matrix recurrence, fixed count."""
    As = np.asarray(As, dtype=np.float64)
    b = As.shape[0]
    I = np.eye(b)
    X = I.copy()
    M = As.copy()
    for _ in range(iters):
        T = ((p + 1) * I - M) / p
        X = X @ T
        M = np.linalg.matrix_power(T, p) @ M
    return X


def cn_scalar(a, p, iters):
    """The same recurrence on scalars (eigenvalues): x tends to a^(-1/p)."""
    a = np.asarray(a, dtype=np.float64)
    x = np.ones_like(a)
    m = a.copy()
    for _ in range(iters):
        t = ((p + 1) - m) / p
        x = x * t
        m = t ** p * m
    return x


# ----------------------------------------------------------------------------
# Newton-DB (Denman-Beavers in its coupled Newton-Schulz form)
# ----------------------------------------------------------------------------

def ndb_matrix(As, iters, count=None):
    """Coupled iteration for As^(1/2) (Y) and As^(-1/2) (Z), fixed count.

    The first iteration starts from Z_0 = I, so T_0 = (3 I - As)/2 needs no
    product, Y_1 = As T_0 costs one and Z_1 = T_0 none: the pages' "first
    iteration saves two products".  Later iterations cost three.  ``count``, if
    given, is a one-element list incremented per matrix product.
    """
    As = np.asarray(As, dtype=np.float64)
    b = As.shape[0]
    I = np.eye(b)
    if iters <= 0:
        return As.copy(), I.copy()
    T = (3.0 * I - As) / 2.0
    Y = As @ T
    Z = T
    if count is not None:
        count[0] += 1
    for _ in range(iters - 1):
        T = (3.0 * I - Z @ Y) / 2.0
        Y = Y @ T
        Z = T @ Z
        if count is not None:
            count[0] += 3
    return Y, Z


def ndb_scalar(a, iters):
    """The Newton-DB recurrence on scalars: y -> sqrt(a), z -> 1/sqrt(a)."""
    a = np.asarray(a, dtype=np.float64)
    y = a.copy()
    z = np.ones_like(a)
    for _ in range(iters):
        t = (3.0 - z * y) / 2.0
        y, z = y * t, t * z
    return y, z


def ndb_inverse_root_matrix(As, p, iters1, iters2=0, count=None):
    """As^(-1/p) for p in {2, 4} by one or two chained Newton-DB calls."""
    Y, Z = ndb_matrix(As, iters1, count)
    if p == 2:
        return Z
    if p == 4:
        _, Z2 = ndb_matrix(Y, iters2, count)
        return Z2
    raise ValueError("Newton-DB gives p = 2 or p = 4 only")


# ----------------------------------------------------------------------------
# Chebyshev
# ----------------------------------------------------------------------------

def chebyshev_coefficients(p, d, eps, npoints=None, f=None):
    """Coefficients c_0..c_d of the degree-d first-kind Chebyshev fit.

    The fit is on x in [eps, 1 + eps] through t = 2 (x - eps) - 1 in [-1, 1],
    using N first-kind nodes t_j = cos(pi (j + 1/2) / N) and the discrete
    Chebyshev transform c_k = (2/N) sum_j f(x_j) T_k(t_j), with c_0 halved.
    For N > d this is the least-squares fit at the nodes.  f defaults to
    x^(-1/p).
    """
    N = 4 * (d + 1) if npoints is None else int(npoints)
    if N <= d:
        raise ValueError("need more nodes than the degree")
    j = np.arange(N, dtype=np.float64)
    theta = np.pi * (j + 0.5) / N
    t = np.cos(theta)
    x = (t + 1.0) / 2.0 + eps
    fx = x ** (-1.0 / p) if f is None else np.asarray(f(x), dtype=np.float64)
    c = np.empty(d + 1, dtype=np.float64)
    for k in range(d + 1):
        c[k] = (2.0 / N) * np.sum(fx * np.cos(k * theta))
    c[0] *= 0.5
    return c


def chebyshev_scalar(c, t):
    """sum_k c_k T_k(t) by the three-term recurrence of the T_k (no Clenshaw)."""
    t = np.asarray(t, dtype=np.float64)
    Tkm1 = np.ones_like(t)
    total = c[0] * Tkm1
    if len(c) == 1:
        return total
    Tk = t.copy()
    total = total + c[1] * Tk
    for k in range(2, len(c)):
        Tkm1, Tk = Tk, 2.0 * t * Tk - Tkm1
        total = total + c[k] * Tk
    return total


def chebyshev_matrix_eigh(As, c):
    """Polynomial oracle: Q diag(sum_k c_k T_k(2 lambda - 1)) Q^T for As = Q diag(lambda) Q^T."""
    lam, Q = np.linalg.eigh(_sym(np.asarray(As, dtype=np.float64)))
    return (Q * chebyshev_scalar(c, 2.0 * lam - 1.0)) @ Q.T


def clenshaw_matrix(S, c, count=None):
    """Clenshaw's recurrence on a matrix argument S, with d - 1 products.

    B_d = c_d I; B_(d-1) = c_(d-1) I + 2 c_d S; B_k = c_k I + 2 S B_(k+1) - B_(k+2)
    for k = d-2 .. 1; result c_0 I + S B_1 - B_2.  ``count`` counts products.
    """
    S = np.asarray(S, dtype=np.float64)
    b = S.shape[0]
    I = np.eye(b)
    d = len(c) - 1
    if d == 0:
        return c[0] * I
    if d == 1:
        return c[0] * I + c[1] * S
    Bk2 = c[d] * I                       # B_d
    Bk1 = c[d - 1] * I + 2.0 * c[d] * S  # B_(d-1)
    for k in range(d - 2, 0, -1):
        Bk = c[k] * I + 2.0 * (S @ Bk1) - Bk2
        if count is not None:
            count[0] += 1
        Bk2, Bk1 = Bk1, Bk
    out = c[0] * I + S @ Bk1 - Bk2
    if count is not None:
        count[0] += 1
    return out


# ----------------------------------------------------------------------------
# Iteration-exact oracle (diagnostic)
# ----------------------------------------------------------------------------

def iteration_exact_root(A, p, method, s, eps=0.0, iters=0, iters2=0, coeffs=None):
    """What the fixed-count iteration gives in exact arithmetic.

    Every iterate is a polynomial in A_s = (A + eps I)/s, so the k-th iterate
    is Q phi_k(Lambda/s) Q^T with phi_k the scalar recurrence.  The result is
    multiplied by s^(-1/p) as the solvers do.  ``s`` is whatever scale the
    solver used (Frobenius or power iteration).
    """
    lam, Q = np.linalg.eigh(_sym(regularize(A, eps)))
    a = lam / s
    if method == "cn":
        phi = cn_scalar(a, p, iters)
    elif method == "ndb":
        y, z = ndb_scalar(a, iters)
        if p == 2:
            phi = z
        elif p == 4:
            _, phi = ndb_scalar(y, iters2)
        else:
            raise ValueError("Newton-DB gives p = 2 or p = 4 only")
    elif method == "chebyshev":
        phi = chebyshev_scalar(coeffs, 2.0 * a - 1.0)
    else:
        raise ValueError(method)
    return (Q * phi) @ Q.T * s ** (-1.0 / p)

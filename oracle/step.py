"""One block-diagonal Shampoo step, literally, per parameter and per block.

Oracle; test infrastructure only.  float64 numpy throughout.

* Statistics ([DASH] "2. Preliminaries on Shampoo"; [NOTES] "The geometric mean
  of the two bounds is the Kronecker bound"): L <- beta2 L + (1 - beta2) G G^T
  and R <- beta2 R + (1 - beta2) G^T G; with beta2 = 1 the factors are plain
  sums over steps, L <- L + G G^T (the notes' sum over s <= t).  No bias
  correction: it would only rescale D by a scalar, which grafting removes.
* Direction ([NOTES] "AdaGrad's regret argument goes through with the
  Kronecker preconditioner"): with S = L^(1/4) (x) R^(1/4) the step is
  S^(-1) vec(G), i.e. D = (L + eps I)^(-1/4) G (R + eps I)^(-1/4) per block.
* Grafting ([3DS] "Hyperparameters": layer-wise grafting onto SGD; [DASH]
  "2. Preliminaries on Shampoo": rescale to Adam's update norm; [NOTES]
  "Grafting corrects Shampoo's eigenvalues": only the scale sets a step's
  length): per parameter, D_g = (||Delta||_F / ||D||_F) D, 0 when D = 0.
  SGD: Delta = G, W <- W - lr D_g.  SGD-momentum ([3DS] "How to use":
  lr = 0.1, momentum = 0.9): Delta = G, M <- mu M + D_g, W <- W - lr M.
  Adam: m <- beta1 m + (1 - beta1) G, v <- beta2 v + (1 - beta2) G^2, bias
  corrected, Delta = m_hat / (sqrt(v_hat) + eps_g), W <- W - lr D_g.
  Options beyond the layer-wise default: block-wise grafting ([DASH] "2.
  Preliminaries on Shampoo" speaks of block-wise Adam grafting) takes the two
  norms over each block's slice of D and Delta; graft "none" steps along D
  itself, W <- W - lr D.

Order inside a step: statistics with G_t first, then roots, then D from G_t.
"""

import numpy as np

from .blocks import plan_blocks, block_slices, reshape_2d
from .roots import (
    inverse_root_eigh,
    frobenius_scale,
    chebyshev_coefficients,
    chebyshev_matrix_eigh,
)


def update_stats(L, R, G, beta2):
    """One statistics update of a block's factors (returns new L, R)."""
    G = np.asarray(G, dtype=np.float64)
    if beta2 == 1.0:
        return L + G @ G.T, R + G.T @ G
    return beta2 * L + (1.0 - beta2) * (G @ G.T), beta2 * R + (1.0 - beta2) * (G.T @ G)


def precondition(Lr, G, Rr):
    """D = Lr G Rr for one block (Lr, Rr the inverse roots of its factors)."""
    return np.asarray(Lr, dtype=np.float64) @ np.asarray(G, dtype=np.float64) @ np.asarray(Rr, dtype=np.float64)


def graft_direction(kind, G, state, t, beta1=0.9, beta2=0.999, eps_g=1e-8):
    """The grafting direction Delta of one parameter (updates Adam's state).

    kind: "sgd" and "momentum" use Delta = G; "adam" uses the bias-corrected
    Adam direction.  ``state`` is a dict holding "m" and "v" for Adam.
    """
    G = np.asarray(G, dtype=np.float64)
    if kind in ("sgd", "momentum"):
        return G
    if kind == "adam":
        state["m"] = beta1 * state["m"] + (1.0 - beta1) * G
        state["v"] = beta2 * state["v"] + (1.0 - beta2) * G * G
        mhat = state["m"] / (1.0 - beta1 ** t)
        vhat = state["v"] / (1.0 - beta2 ** t)
        return mhat / (np.sqrt(vhat) + eps_g)
    raise ValueError(kind)


class ShampooOracle:
    """Literal block-diagonal Shampoo on a list of parameters (float64).

    root: "eigh" (limit of coupled Newton and Newton-DB) or "chebyshev" (the
    fitted polynomial evaluated exactly on the eigenvalues of the Frobenius
    scaled factor).  Parameters are given in their 2-D view (dim 0 kept).
    """

    def __init__(self, shapes, block_sizes, beta2=1.0, eps=1e-12, p=4,
                 root="eigh", cheb_degree=16, cheb_points=None,
                 graft="sgd", lr=0.1, momentum=0.9, beta1=0.9, graft_beta2=0.999,
                 eps_g=1e-8, graft_blockwise=False):
        self.shapes = [reshape_2d(s) for s in shapes]
        self.table = plan_blocks(self.shapes, block_sizes)
        self.beta2, self.eps, self.p = float(beta2), float(eps), int(p)
        self.root = root
        self.coeffs = (chebyshev_coefficients(p, cheb_degree, eps, cheb_points)
                       if root == "chebyshev" else None)
        self.graft, self.lr, self.momentum = graft, float(lr), float(momentum)
        self.beta1, self.graft_beta2, self.eps_g = float(beta1), float(graft_beta2), float(eps_g)
        self.graft_blockwise = bool(graft_blockwise)
        self.t = 0
        self.L = []
        self.R = []
        for b in range(self.table.shape[0]):
            rows, cols = int(self.table[b, 5]), int(self.table[b, 6])
            self.L.append(np.zeros((rows, rows)))
            self.R.append(np.zeros((cols, cols)))
        self.state = [{"m": np.zeros(s), "v": np.zeros(s), "mom": np.zeros(s)} for s in self.shapes]

    def _root(self, A):
        if self.root == "eigh":
            return inverse_root_eigh(A, self.p, self.eps)
        if self.root == "chebyshev":
            Ae = A + self.eps * np.eye(A.shape[0])
            s = frobenius_scale(Ae)
            if s == 0.0:
                return np.zeros_like(A)
            return chebyshev_matrix_eigh(Ae / s, self.coeffs) * s ** (-1.0 / self.p)
        raise ValueError(self.root)

    def step(self, W, G):
        """One step.  W: list of 2-D float64 arrays (updated in place); G: list
        of 2-D gradients.  Returns (D, Dg): the ungrafted and grafted
        directions per parameter."""
        self.t += 1
        G = [np.asarray(g, dtype=np.float64).reshape(s) for g, s in zip(G, self.shapes)]
        D = [np.zeros(s) for s in self.shapes]
        for b in range(self.table.shape[0]):
            p = int(self.table[b, 0])
            rs, cs = block_slices(self.table, b)
            Gb = G[p][rs, cs]
            self.L[b], self.R[b] = update_stats(self.L[b], self.R[b], Gb, self.beta2)
            Lr = self._root(self.L[b])
            Rr = self._root(self.R[b])
            D[p][rs, cs] = precondition(Lr, Gb, Rr)
        Dg = []
        for p, s in enumerate(self.shapes):
            if self.graft == "none":
                dg = D[p].copy()
            else:
                delta = graft_direction(self.graft, G[p], self.state[p], self.t,
                                        beta1=self.beta1, beta2=self.graft_beta2, eps_g=self.eps_g)
                dg = np.zeros(s)
                if self.graft_blockwise:
                    groups = [block_slices(self.table, b) for b in range(self.table.shape[0])
                              if int(self.table[b, 0]) == p]
                else:
                    groups = [(slice(None), slice(None))]
                for rs, cs in groups:
                    nD = np.linalg.norm(D[p][rs, cs])
                    nd = np.linalg.norm(delta[rs, cs])
                    if nD > 0:
                        dg[rs, cs] = D[p][rs, cs] * (nd / nD)
            Dg.append(dg)
            if self.graft == "momentum":
                self.state[p]["mom"] = self.momentum * self.state[p]["mom"] + dg
                W[p] -= self.lr * self.state[p]["mom"]
            else:
                W[p] -= self.lr * dg
        return D, Dg

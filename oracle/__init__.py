"""CPU float64 oracle for the block-diagonal Shampoo preconditioner step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``matrix_inverse_roots_amd``) never imports it, and this package imports
nothing from the product path: the two share no kernels, headers, helpers,
tables or constant generators.

Everything here is plain numpy/scipy in float64, written as literal per-block
loops on the *unpadded* block slices, so that a reader can check each step
against the pages by eye.

Sources cited in this package (titles of the pages; sections as named there):

* [DIST]   "A Distributed Data-Parallel PyTorch Implementation of the Distributed
           Shampoo Optimizer for Training Neural Networks At-Scale" (abstract).
* [DASH]   "DASH: Faster Shampoo via Batched Block Preconditioning and Efficient
           Inverse-Root Solvers", source-linked AI summary: sections
           "2. Preliminaries on Shampoo", "3. Inverse Root Methods",
           "4. Blocking Strategy", "A.1/A.2 Chebyshev polynomials",
           "A.3 Numerical Precision", "B.1 Regularization (dampening) for EVD",
           "D. DASH for Computer Vision".
* [3DS]    "3D-Shampoo optimizer" README: "How to use", "Hyperparameters".
* [NOTES]  "Shampoo" notes: paragraphs "The geometric mean of the two bounds is
           the Kronecker bound", "AdaGrad's regret argument goes through with the
           Kronecker preconditioner", "Roots on idle CPUs, partial preconditioners
           ... and grafting", "Spreading the preconditioners across GPUs",
           "Grafting corrects Shampoo's eigenvalues".

Parity status: every public function is pinned by a ``-m "not gpu"`` test
against a closed form, an invariant, a brute-force construction or a value the
pages print; none is "parity unpinned".
"""

from .blocks import reshape_2d, plan_blocks, pack_blocks, unpack_blocks, block_slices
from .roots import (
    regularize,
    frobenius_scale,
    power_iteration,
    inverse_root_eigh,
    cn_matrix,
    cn_scalar,
    ndb_matrix,
    ndb_scalar,
    ndb_inverse_root_matrix,
    chebyshev_coefficients,
    chebyshev_scalar,
    chebyshev_matrix_eigh,
    clenshaw_matrix,
    residual,
    iteration_exact_root,
)
from .step import (
    update_stats,
    precondition,
    graft_direction,
    ShampooOracle,
)

__all__ = [
    "reshape_2d", "plan_blocks", "pack_blocks", "unpack_blocks", "block_slices",
    "regularize", "frobenius_scale", "power_iteration", "inverse_root_eigh",
    "cn_matrix", "cn_scalar", "ndb_matrix", "ndb_scalar", "ndb_inverse_root_matrix",
    "chebyshev_coefficients", "chebyshev_scalar", "chebyshev_matrix_eigh",
    "clenshaw_matrix", "residual", "iteration_exact_root",
    "update_stats", "precondition", "graft_direction", "ShampooOracle",
]

"""Non-finite fallback of shampoo_step (flag only / keep the previous root /
recompute in float64).

A reliable failure: statistics in float64 with beta2 = 0 (L_t = G_t G_t^T,
positive definite as stored), step 1 with a well-conditioned gradient
(Gram spectrum in [0.1, 1]), step 2 with Gram spectrum in [1e-8, 1], and a
Newton-DB chain with half-precision products, which diverges on the second
(half precision cannot resolve that spectrum).  The float64 recomputation
is checked against the oracle's eigendecomposition root of the same
float64 statistics.
"""

import numpy as np
import pytest

import oracle
import synthetic
from helpers import rel_fro, to_dev, log

pytestmark = pytest.mark.gpu

B, NPARAM = 512, 2


@pytest.fixture(scope="module")
def mir():
    import matrix_inverse_roots_amd as m
    return m


def two_steps(mir, fallback):
    import torch
    W = [torch.zeros(B, B, dtype=torch.float32, device="cuda") for _ in range(NPARAM)]
    ro = mir.RootOpts(method="ndb", scaling="power", iters=28, iters2=17, compute="f16", pi_vectors=16,
                      pi_iters=10)
    opt = mir.Shampoo(W, block_size=B, beta2=0.0, eps=1e-12, root=ro, graft="sgd", lr=1e-3,
                      stats_dtype=torch.float64, fallback=fallback)
    st = opt.stacks[0]
    g1 = synthetic.gram_spectrum_grads(31, NPARAM, B, 0.1, 1.0)
    opt.step([to_dev(g) for g in g1])
    torch.cuda.synchronize()
    assert int(st.flags.sum().item()) == 0, "step 1 (well conditioned) must not be flagged"
    roots1 = st.roots.clone()
    g2 = synthetic.gram_spectrum_grads(32, NPARAM, B, 1e-8, 1.0)
    opt.step([to_dev(g) for g in g2])
    torch.cuda.synchronize()
    return W, st, roots1


def test_fallback_none_lets_the_failure_through(mir):
    W, st, _ = two_steps(mir, "none")
    fl = st.flags.cpu().numpy()
    log(f"fallback none: flags {fl.tolist()}")
    assert (fl & mir.FLAG_NONFINITE).any()
    assert not all(np.isfinite(w.cpu().numpy()).all() for w in W)


def test_fallback_keep_previous_root(mir):
    W, st, roots1 = two_steps(mir, "keep")
    fl = st.flags.cpu().numpy()
    log(f"fallback keep: flags {fl.tolist()}")
    bad = (fl & mir.FLAG_NONFINITE) != 0
    assert bad.any()
    assert ((fl & mir.FLAG_KEPT_PREVIOUS) != 0).tolist() == bad.tolist()
    r1, r2 = roots1.cpu().numpy(), st.roots.cpu().numpy()
    for f in range(2 * NPARAM):
        if bad[f]:
            np.testing.assert_array_equal(r2[f], r1[f])
        else:
            assert np.isfinite(r2[f]).all()
    assert all(np.isfinite(w.cpu().numpy()).all() for w in W)


def test_fallback_recompute_in_float64(mir):
    W, st, _ = two_steps(mir, "f64")
    fl = st.flags.cpu().numpy()
    log(f"fallback f64: flags {fl.tolist()}")
    bad = (fl & mir.FLAG_NONFINITE) != 0
    assert bad.any()
    assert ((fl & mir.FLAG_RECOMPUTED_F64) != 0).tolist() == bad.tolist()
    assert not (fl & mir.FLAG_KEPT_PREVIOUS).any()
    L = st.LR.cpu().numpy()
    R = st.roots.cpu().numpy()
    worst = 0.0
    for f in np.nonzero(bad)[0]:
        ref = oracle.inverse_root_eigh(L[f], 4, 1e-12)
        worst = max(worst, rel_fro(R[f], ref))
    log(f"recomputed factors {int(bad.sum())}: worst rel err vs oracle {worst:.2e}")
    assert worst < 1e-4
    assert all(np.isfinite(w.cpu().numpy()).all() for w in W)


def test_fallback_workspace_and_validation(mir):
    import torch
    W = [torch.zeros(256, 256, device="cuda")]
    base = mir.Shampoo(W, block_size=256, fallback="none").stacks[0].ws.numel()
    keep = mir.Shampoo(W, block_size=256, fallback="keep").stacks[0].ws.numel()
    f64 = mir.Shampoo(W, block_size=256, fallback="f64").stacks[0].ws.numel()
    assert base < keep < f64
    with pytest.raises(ValueError):
        mir.Shampoo(W, block_size=256, fallback="retry")

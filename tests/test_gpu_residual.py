"""Device solver residual ||X^p A_s - I||_F / sqrt(v) and the residual flag.

The residual the library computes on the device is compared with the
oracle's residual (oracle.residual, float64 on the host) of the very roots
the library returned.  The chains are stopped early (few iterations or a
low Chebyshev degree) so that the residual is far above the rounding noise
of either side and the comparison pins the formula: the power, the
regularised input, the valid region and the sqrt(v) normalisation.

The flag drives shampoo_step's fallback: with float64 statistics and a
float32 chain, the step-1 factors of a square Gaussian block (condition
number about 1e6, which float32 cannot resolve) come back finite but
inaccurate, are flagged RESIDUAL and are recomputed in float64, and the
parameters then match the oracle to the stated 1e-4.
"""

import numpy as np
import pytest

import oracle
import synthetic
from helpers import rel_fro, to_dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mir():
    import matrix_inverse_roots_amd as m
    return m


def roots_with_residual(mir, A, p, valid=None, **kw):
    import torch
    inp = to_dev(A)
    out = torch.empty_like(inp)
    n, B = A.shape[0], A.shape[1]
    res = torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")
    flags = torch.zeros(n, dtype=torch.int32, device="cuda")
    vd = None if valid is None else to_dev(np.asarray(valid, dtype=np.int32))
    opts = mir.RootOpts(residual_out=res, **kw)
    if opts.scaling == "power":
        opts.pi_start = to_dev(synthetic.pi_start_vectors(5, opts.pi_vectors, B))
    mir.shampoo_inverse_root(inp, out, p, opts, valid=vd, flags=flags)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), res.cpu().numpy().astype(np.float64), flags.cpu().numpy()


@pytest.mark.parametrize("method,p,compute,kw", [
    ("cn", 4, "f32", dict(iters=4)),
    ("cn", 2, "f64", dict(iters=3)),
    ("cn", 8, "f32", dict(iters=5)),
    ("ndb", 4, "f32", dict(iters=3, iters2=2)),
    ("ndb", 2, "f64", dict(iters=3)),
    ("ndb", 4, "f16", dict(iters=3, iters2=2)),
    ("chebyshev", 3, "f32", dict(cheb_degree=4)),
    ("chebyshev", 4, "f64", dict(cheb_degree=3, cheb_eval="ps")),
])
def test_residual_matches_oracle_on_returned_roots(mir, method, p, compute, kw):
    """Unconverged chains (residual 1e-3 .. 1) on padded and unpadded
    matrices: the device residual equals the oracle's residual of the
    returned root against the regularised input over the valid region."""
    B, n, eps = 128, 6, 1e-3
    A = synthetic.spd_stack(40 + p, n, B, 1e-2, 1.0)
    valid = [128, 100, 128, 64, 7, 128]
    for i, v in enumerate(valid):
        A[i, v:, :] = 0.0
        A[i, :, v:] = 0.0
    dt = np.float64 if compute == "f64" else np.float32
    X, res, fl = roots_with_residual(mir, A.astype(dt), p, valid=valid, method=method, compute=compute, eps=eps, **kw)
    worst, far = 0.0, 0
    for i, v in enumerate(valid):
        Ai = A[i, :v, :v].astype(dt).astype(np.float64) + eps * np.eye(v)
        want = oracle.residual(X[i, :v, :v], Ai, p)
        log(f"{method} p={p} {compute} matrix {i} (valid {v}): device residual {res[i]:.4e}, oracle {want:.4e}")
        if want > 1e-4:
            # far from converged: the residual is not rounding noise
            worst = max(worst, abs(res[i] - want) / want)
            far += 1
        else:
            # converged (a 7 x 7 matrix has few eigenvalues to resolve):
            # both sides at rounding level
            assert abs(res[i] - want) < (1e-12 if compute == "f64" else 1e-5)
    assert far >= 4
    # float32 or half chains compute the residual in float32 from the unscaled
    # iterate; the returned root is that iterate rounded once more after scaling
    assert worst < (1e-6 if compute == "f64" else 1e-3)
    assert not (fl & mir.FLAG_RESIDUAL).any()  # no bound given: no flag


def test_residual_of_converged_float64_roots_and_bound(mir):
    """Converged float64 coupled Newton: residuals at rounding level, below
    a bound of 1e-10 (no flag); the same call with a bound of 1e-16 flags
    every matrix, and the roots are written either way."""
    A = synthetic.spd_stack(9, 4, 256, 1e-3, 1.0)
    X, res, fl = roots_with_residual(mir, A, 4, method="cn", iters=30, compute="f64", residual_bound=1e-10)
    log(f"converged float64 residuals {res.tolist()}")
    assert (res < 1e-10).all() and not (fl & mir.FLAG_RESIDUAL).any()
    for i in range(4):
        assert rel_fro(X[i], oracle.inverse_root_eigh(A[i], 4)) < 1e-10
    X2, res2, fl2 = roots_with_residual(mir, A, 4, method="cn", iters=30, compute="f64", residual_bound=1e-16)
    assert ((fl2 & mir.FLAG_RESIDUAL) != 0).all()
    np.testing.assert_array_equal(X2, X)
    np.testing.assert_array_equal(res2, res)


def test_residual_flags_nonfinite_and_skips_zero_scale(mir):
    """An indefinite matrix (eigenvalue -0.3: the coupled Newton iterates
    diverge) has a non-finite residual and is flagged RESIDUAL and NONFINITE;
    an all-zero matrix (zero scale) is left to ZERO_SCALE."""
    A, lam, Q = synthetic.spd_stack(12, 3, 64, 1e-2, 1.0, return_factors=True)
    lam = lam.copy()
    lam[1, 0] = -0.3
    A[1] = (Q[1] * lam[1]) @ Q[1].T
    A[2] = 0.0
    X, res, fl = roots_with_residual(mir, A.astype(np.float32), 4, method="cn", iters=20, residual_bound=1e-2)
    log(f"residuals {res.tolist()}, flags {fl.tolist()}")
    assert fl[0] == 0 and res[0] < 1e-2
    assert fl[1] & mir.FLAG_RESIDUAL and fl[1] & mir.FLAG_NONFINITE and not np.isfinite(res[1])
    assert fl[2] == mir.FLAG_ZERO_SCALE


def test_step_residual_fallback_single_matrix_ten_steps(mir):
    """The 256 x 128 single-parameter workload (two 128-blocks, N(0,1)
    gradients from seed 0, beta2 = 1, eps = 1e-12, SGD lr 0.1, coupled Newton
    30) with float64 statistics, a float32 chain, residual bound 1e-4 and the
    float64 fallback: the step-1 factors (condition number about 1e6) are
    flagged RESIDUAL and recomputed in float64; from step 2 on the factors
    are sums of Gram matrices (condition number about 34) and the float32
    roots pass the bound.  Every step matches the oracle to 1e-4."""
    import torch
    shape = (256, 128)
    grads = synthetic.gaussian_grads(0, [shape], 10, 1.0)
    W = [torch.zeros(shape, dtype=torch.float32, device="cuda")]
    opt = mir.Shampoo(W, block_size=128, beta2=1.0, eps=1e-12,
                      root=mir.RootOpts(method="cn", iters=30, compute="f32", residual_bound=1e-4),
                      graft="sgd", lr=0.1, stats_dtype=torch.float64, fallback="f64", residuals=True)
    orc = oracle.ShampooOracle([shape], [128], beta2=1.0, eps=1e-12, graft="sgd", lr=0.1)
    Wo = [np.zeros(shape)]
    st = opt.stacks[0]
    for t in range(10):
        st.flags.zero_()
        opt.step([to_dev(grads[t][0])])
        orc.step(Wo, [grads[t][0].astype(np.float64)])
        torch.cuda.synchronize()
        fl = st.flags.cpu().numpy()
        res = st.residuals.cpu().numpy()
        e = rel_fro(W[0].cpu().numpy(), Wo[0])
        log(f"step {t + 1}: rel err {e:.2e}, residuals {np.array2string(res, precision=2)}, flags {fl.tolist()}")
        if t == 0:
            assert (fl == (mir.FLAG_RESIDUAL | mir.FLAG_RECOMPUTED_F64)).all()
        assert not (fl & (mir.FLAG_NONFINITE | mir.FLAG_KEPT_PREVIOUS)).any()
        assert e < 1e-4


def test_step_residual_keep_previous(mir):
    """Fallback "keep" with a residual bound no root can meet (1e-12): every
    factor is flagged RESIDUAL and keeps its previous root (zeros at step 1),
    so the direction, and the step, is zero."""
    import torch
    shape = (128, 128)
    g = synthetic.gaussian_grads(3, [shape], 1, 1.0)[0][0]
    W = [torch.zeros(shape, dtype=torch.float32, device="cuda")]
    opt = mir.Shampoo(W, block_size=128, beta2=1.0, eps=1e-3,
                      root=mir.RootOpts(method="cn", iters=20, residual_bound=1e-12), graft="sgd", lr=0.1,
                      fallback="keep", residuals=True)
    opt.step([to_dev(g)])
    torch.cuda.synchronize()
    st = opt.stacks[0]
    fl = st.flags.cpu().numpy()
    assert (fl == (mir.FLAG_RESIDUAL | mir.FLAG_KEPT_PREVIOUS)).all()
    assert not st.roots.any().item()
    assert not W[0].any().item()
    assert np.isfinite(st.residuals.cpu().numpy()).all()


@pytest.mark.parametrize("group", [True, False])
def test_step_residuals_grouped_and_padded(mir, group):
    """Ragged blocks: the residual of every factor, grouped by side or
    computed at the block size, equals the oracle's residual of the stored
    root against the stored statistics plus eps, over the valid size."""
    import torch
    shapes = [(300, 130), (64, 64), (5, 200)]
    grads = synthetic.gaussian_grads(21, shapes, 1, 0.1)[0]
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=128, beta2=0.999, eps=1e-3,
                      root=mir.RootOpts(method="cn", iters=6, compute="f64"), graft="sgd", lr=0.1,
                      stats_dtype=torch.float64, residuals=True, group_factors=group)
    opt.step([to_dev(g) for g in grads])
    torch.cuda.synchronize()
    st = opt.stacks[0]
    L, R, res = st.LR.cpu().numpy(), st.roots.cpu().numpy(), st.residuals.cpu().numpy()
    nb = st.nblk
    for f in range(2 * nb):
        blk = st.table[f % nb]
        v = int(blk[5] if f < nb else blk[6])
        want = oracle.residual(R[f, :v, :v], L[f, :v, :v] + 1e-3 * np.eye(v), 4)
        assert abs(res[f] - want) <= 1e-6 * want + 1e-12, (f, v, res[f], want)

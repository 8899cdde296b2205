"""Edge cases: the largest batch one call accepts, an empty stack,
a large block side, identity inputs (whose root is exactly I), a rank-one
statistic regularised by eps (condition number 1 + ||g||^2 / eps), and
parameters of one element, one row or one column."""

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


def root(mir, A, p=4, valid=None, **kw):
    import torch
    inp = to_dev(A)
    out = torch.empty_like(inp)
    flags = torch.zeros(A.shape[0], dtype=torch.int32, device="cuda")
    vd = None if valid is None else to_dev(np.asarray(valid, dtype=np.int32))
    mir.shampoo_inverse_root(inp, out, p, mir.RootOpts(**kw), valid=vd, flags=flags)
    torch.cuda.synchronize()
    return out, flags


def test_largest_batch_65535_matrices(mir):
    import torch
    n, B = 65535, 64
    base = synthetic.spd_stack(41, 16, B, 1e-2, 1.0).astype(np.float32)
    A = np.ascontiguousarray(np.tile(base, (n // 16 + 1, 1, 1))[:n])
    out, fl = root(mir, A, method="cn", iters=20)
    assert int((fl != 0).sum().item()) == 0
    for i in (0, 1, 15, 32768, n - 2, n - 1):
        X = out[i].cpu().numpy().astype(np.float64)
        assert rel_fro(X, oracle.inverse_root_eigh(A[i].astype(np.float64), 4)) < 1e-4, i
    # identical inputs give identical roots wherever they sit in the batch
    assert torch.equal(out[0], out[16]) and torch.equal(out[5], out[n - 1 - ((n - 1 - 5) % 16)])
    log(f"{n} matrices of {B}: all finite, sampled roots within 1e-4")


def test_block_side_2048(mir):
    A = synthetic.spd_stack(42, 2, 2048, 1e-2, 1.0).astype(np.float32)
    for method in ("cn", "ndb"):
        out, fl = root(mir, A, method=method, iters=20, iters2=14)
        assert not fl.any().item()
        X = out.cpu().numpy().astype(np.float64)
        worst = max(rel_fro(X[i], oracle.inverse_root_eigh(A[i].astype(np.float64), 4)) for i in range(2))
        log(f"B = 2048 {method}: worst {worst:.2e}")
        assert worst < 1e-4


@pytest.mark.parametrize("method", ["cn", "ndb"])
def test_identity_input(mir, method):
    B = 256
    A = np.stack([np.eye(B, dtype=np.float32)] * 3)
    for compute in ("f32", "f64"):
        out, fl = root(mir, A, method=method, iters=12, iters2=10, compute=compute)
        assert not fl.any().item()
        err = float((out.cpu().double() - torch_eye(B)).abs().max())
        log(f"identity {method} {compute}: max |X - I| {err:.1e}")
        assert err < (1e-5 if compute == "f32" else 1e-12)


def torch_eye(B):
    import torch
    return torch.eye(B, dtype=torch.float64)


def test_rank_one_statistic_with_eps(mir):
    """Rank-one statistic g g^T in float64 (exactly positive semidefinite to
    float64 rounding).  Rounded to float32 it would pick up eigenvalues of
    order -1e-6: the iterations then compute (A + eps I)^(-1/4) exactly while
    the eigendecomposition limit lifts eigenvalues below eps to eps, and the
    two part by about 5e-5 -- a property of that input, not of either side."""
    B, eps = 128, 1e-3
    gen = np.random.default_rng(43)
    g = gen.standard_normal((2, B, 1))
    A = g @ np.swapaxes(g, 1, 2)                          # rank one; eps regularises
    out, fl = root(mir, A, method="cn", iters=40, compute="f64", eps=eps)
    assert not fl.any().item()
    X = out.cpu().numpy()
    for i in range(2):
        ref = oracle.inverse_root_eigh(A[i], 4, eps)
        e = rel_fro(X[i], ref)
        r = oracle.residual(X[i], A[i] + eps * np.eye(B), 4)
        log(f"rank one + eps, factor {i}: rel err {e:.2e}, residual {r:.2e}")
        assert e < 1e-9


def test_empty_stack(mir):
    """A stack of no matrices: every call succeeds and writes nothing (the
    output tensor next to it keeps its bytes)."""
    import torch
    inp = torch.empty((0, 128, 128), dtype=torch.float32, device="cuda")
    out = torch.empty_like(inp)
    for kw in (dict(method="cn", iters=10), dict(method="ndb", iters=5, iters2=4), dict(method="cn", iters=10, tol=1e-4),
               dict(method="chebyshev", cheb_degree=8), dict(method="cn", iters=10, compute="f16")):
        mir.shampoo_inverse_root(inp, out, 4, mir.RootOpts(**kw))
    guard = torch.full((4,), 7.0, device="cuda")
    torch.cuda.synchronize()
    assert torch.equal(guard, torch.full((4,), 7.0, device="cuda"))


def test_degenerate_parameter_shapes(mir):
    """Parameters of one element, one row and one column (blocks of side 64
    with a single valid row or column; rank-one factors regularised by eps),
    on the float64 path: within 1e-4 of the oracle over two steps."""
    import torch
    shapes = [(1, 1), (1, 300), (300, 1), (2, 3)]
    grads = synthetic.gaussian_grads(43, shapes, 2, 0.1)
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=256, beta2=0.999, eps=1e-3,
                      root=mir.RootOpts(method="cn", iters=30, compute="f64"), graft="sgd", lr=0.1,
                      stats_dtype=torch.float64)
    orc = oracle.ShampooOracle(shapes, [256] * len(shapes), beta2=0.999, eps=1e-3, graft="sgd", lr=0.1)
    Wo = [np.zeros(s) for s in shapes]
    for t in range(2):
        opt.step([to_dev(g) for g in grads[t]])
        orc.step(Wo, [g.astype(np.float64) for g in grads[t]])
        torch.cuda.synchronize()
        errs = [rel_fro(w.cpu().numpy(), wo) for w, wo in zip(W, Wo)]
        log(f"degenerate shapes step {t + 1}: {['%.1e' % e for e in errs]}")
        assert max(errs) < 1e-4
    assert sum(int(f.sum().item()) for f in opt.flags()) == 0

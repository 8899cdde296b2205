"""GPU parity at the full workload sizes.

* 1024 SPD blocks 512 x 512 with lambda in [1e-8, 1] (the benchmark input),
  Newton-DB 28 + 17 with power-iteration scaling, in the launch configuration
  the benchmark times: the float64 chain against the oracle on every one of
  the 1024 blocks, to the stated 1e-4.  Float32 and half-precision products
  are diagnostics there (float32 cannot resolve condition number 1e8): their
  non-finite blocks must be flagged, and finite float32 blocks must match on
  the eigen-directions float32 resolves.
* The 12-layer decoder set (151 M parameters, 144 blocks of 1024): all
  parameters stepped on the GPU, the oracle run on sampled parameters (grafting
  is per parameter and blocks are independent, so a sampled parameter's
  result does not depend on the others).
* The 53-matrix bottleneck set with Chebyshev roots: all stepped, a spread
  of parameters checked.
* The half-precision variants of the first two: every non-finite block
  flagged; the decoder set's half-product coupled Newton within 2e-2.
"""

import numpy as np
import pytest

import oracle
import synthetic
from helpers import rel_fro, to_dev, bf16_tensor, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mir():
    import matrix_inverse_roots_amd as m
    return m


def all_blocks_vs_oracle(X, A64):
    """Relative Frobenius error of every block against the oracle's eigh root,
    the blocks spread over the host's cores (one BLAS thread each)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    import threadpoolctl

    def one(i):
        return rel_fro(X[i], oracle.inverse_root_eigh(A64[i], 4))

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpoolctl.threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        return np.array(list(ex.map(one, range(A64.shape[0]))))


def test_spd_stack_1024x512_newton_db_full_size(mir):
    import torch
    n, B = 1024, 512
    A64 = synthetic.spd_stack(3, n, B, 1e-8, 1.0)
    V0 = to_dev(synthetic.pi_start_vectors(3, 16, B))
    sample = [0, 1, 255, 511, 512, 777, 1022, 1023]
    # float64 chain
    inp = to_dev(A64)
    out = torch.empty_like(inp)
    flags = torch.zeros(n, dtype=torch.int32, device="cuda")
    opts = mir.RootOpts(method="ndb", scaling="power", compute="f64", iters=28, iters2=17, pi_vectors=16,
                        pi_iters=10, pi_start=V0)
    mir.shampoo_inverse_root(inp, out, 4, opts, flags=flags)
    torch.cuda.synchronize()
    assert int(flags.sum().item()) == 0
    X = out.cpu().numpy()
    del inp, out
    errs = all_blocks_vs_oracle(X, A64)
    del X
    worst = int(np.argmax(errs))
    log(f"1024 x 512^2 f64 NDB: all {n} blocks vs the oracle, worst rel err {errs[worst]:.2e} (block {worst}), "
        f"median {np.median(errs):.2e}")
    assert errs.max() < 1e-4
    # float32 chain: non-finite blocks must be flagged, finite ones checked on
    # the eigen-directions float32 can resolve
    A32 = A64.astype(np.float32)
    del A64
    inp = to_dev(A32)
    out = torch.empty_like(inp)
    flags.zero_()
    mir.shampoo_inverse_root(inp, out, 4, mir.RootOpts(**{**opts.__dict__, "compute": "f32"}), flags=flags)
    torch.cuda.synchronize()
    fl = flags.cpu().numpy()
    finite = torch.isfinite(out).flatten(1).all(1).cpu().numpy()
    assert ((~finite) <= ((fl & mir.FLAG_NONFINITE) != 0)).all()
    log(f"1024 x 512^2 f32 NDB: {int((~finite).sum())} of {n} blocks non-finite, all flagged")
    for i in sample:
        if not finite[i]:
            continue
        lam, Q = np.linalg.eigh(A32[i].astype(np.float64))
        keep = lam >= 1e-4 * lam.max()
        Qk = Q[:, keep]
        Xi = out[i].cpu().numpy().astype(np.float64)
        assert rel_fro(Qk.T @ Xi @ Qk, np.diag(lam[keep] ** -0.25)) < 1e-3
    # half-precision products (the stack's fp16 variant): [DASH] reports that
    # Newton-DB does not converge in FP16; every non-finite block is flagged
    flags.zero_()
    mir.shampoo_inverse_root(inp, out, 4, mir.RootOpts(**{**opts.__dict__, "compute": "f16"}), flags=flags)
    torch.cuda.synchronize()
    fl = flags.cpu().numpy()
    finite = torch.isfinite(out).flatten(1).all(1).cpu().numpy()
    assert ((~finite) <= ((fl & mir.FLAG_NONFINITE) != 0)).all()
    log(f"1024 x 512^2 f16 NDB: {int((~finite).sum())} of {n} blocks non-finite, all flagged")


def _decoder_run(mir, compute, stats64, sample, fallback="none", **root_kw):
    import torch
    shapes = synthetic.decoder_shapes()
    grads = synthetic.gaussian_grads(4, shapes, 3, 0.02, dtype="bf16")
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=1024, beta2=0.999, eps=1e-12,
                      root=mir.RootOpts(method="cn", iters=34, compute=compute, **root_kw),
                      graft="adam", lr=1e-3, grad_dtype=torch.bfloat16, fallback=fallback,
                      stats_dtype=torch.float64 if stats64 else torch.float32)
    sshapes = [shapes[i] for i in sample]
    orc = oracle.ShampooOracle(sshapes, [1024] * len(sample), beta2=0.999, eps=1e-12, graft="adam", lr=1e-3)
    Wo = [np.zeros(s) for s in sshapes]
    errs = []
    for t in range(3):
        for f in opt.flags():
            f.zero_()
        opt.step([bf16_tensor(g) for g in grads[t]])
        orc.step(Wo, [synthetic.bf16_bits_to_f32(grads[t][i]).astype(np.float64) for i in sample])
        torch.cuda.synchronize()
        e = max(rel_fro(W[i].cpu().numpy(), Wo[k]) for k, i in enumerate(sample))
        fl = torch.cat(opt.flags()).cpu().numpy()
        log(f"decoder set ({compute}, stats {'f64' if stats64 else 'f32'}, {root_kw}) step {t + 1}: sampled rel err "
            f"{e:.2e}, flags {np.unique(fl).tolist()} ({int((fl != 0).sum())} factors)")
        if fallback == "none":
            assert not fl.any()
        else:
            assert not (fl & (mir.FLAG_NONFINITE | mir.FLAG_KEPT_PREVIOUS)).any()
        errs.append(e)
    return errs


def test_decoder_set_full_size_f64(mir):
    """Float64 statistics, chain and products: the stated 1e-4 on every one
    of the 48 parameters (the oracle's 288 eigh roots per step)."""
    errs = _decoder_run(mir, "f64", True, sample=list(range(48)))
    assert all(e < 1e-4 for e in errs)


@pytest.mark.parametrize("scaling", ["frobenius", "power"])
def test_decoder_set_full_size_f32_chain_residual_checked(mir, scaling):
    """Float64 statistics, a float32 coupled Newton chain (after Frobenius or
    power-iteration scaling) stopping at ||M - I||_F <= 1e-4, its device
    residual checked against 1e-4 and the float64 recomputation as fallback
    (step 1's factors fail the check): the stated 1e-4."""
    errs = _decoder_run(mir, "f32", True, sample=[0, 1, 2, 3, 46, 47], fallback="f64", tol=1e-4,
                        residual_bound=1e-4, scaling=scaling)
    assert all(e < 1e-4 for e in errs)


def test_decoder_set_full_size_f32_diagnostic(mir):
    """Float32 diagnostic, not a parity test: float32 statistics of the
    step-1 single-Gram factors (condition number about 4e6) cannot reach
    1e-4 (measured 3.0e-2, 2.5e-2, 2.2e-2); fixed ceiling 5e-2."""
    errs = _decoder_run(mir, "f32", False, sample=[0, 3, 45])
    assert all(e < 5e-2 for e in errs)


@pytest.mark.parametrize("tol,scaling,pdt", [(0.0, "frobenius", None), (0.1, "frobenius", None), (0.1, "power", None),
                                             (0.1, "power", "bf16")])
def test_decoder_set_full_size_cn_half_products(mir, tol, scaling, pdt):
    """The decoder set with coupled Newton on half-precision products and the
    float64 fallback, as the benchmark's half-product steps run it (34
    iterations, or stopping once the half copy of M is within 0.1 of I in
    Frobenius norm; Frobenius or power-iteration scaling; preconditioning
    products in float32 or bfloat16): step 1's single-Gram factors diverge
    in half precision
    and are recomputed in float64; steps 2 and 3 converge in half precision
    on every factor; sampled parameters within the half-precision bar."""
    import torch
    shapes = synthetic.decoder_shapes()
    grads = synthetic.gaussian_grads(4, shapes, 3, 0.02, dtype="bf16")
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=1024, beta2=0.999, eps=1e-12,
                      root=mir.RootOpts(method="cn", iters=34, compute="f16", tol=tol, scaling=scaling),
                      graft="adam", lr=1e-3, grad_dtype=torch.bfloat16, fallback="f64",
                      precondition_dtype=torch.bfloat16 if pdt == "bf16" else None)
    sample = [0, 1, 2, 3, 46, 47]
    sshapes = [shapes[i] for i in sample]
    orc = oracle.ShampooOracle(sshapes, [1024] * len(sample), beta2=0.999, eps=1e-12, graft="adam", lr=1e-3)
    Wo = [np.zeros(s) for s in sshapes]
    for t in range(3):
        for f in opt.flags():
            f.zero_()
        opt.step([bf16_tensor(g) for g in grads[t]])
        orc.step(Wo, [synthetic.bf16_bits_to_f32(grads[t][i]).astype(np.float64) for i in sample])
        torch.cuda.synchronize()
        fl = torch.cat(opt.flags()).cpu().numpy()
        e = max(rel_fro(W[i].cpu().numpy(), Wo[k]) for k, i in enumerate(sample))
        log(f"decoder set (half products, tol {tol}, {scaling}, precondition {pdt or 'f32'}) step {t + 1}: "
            f"sampled rel err {e:.2e}, "
            f"flags {np.unique(fl).tolist()}")
        if t == 0:
            assert (fl == (mir.FLAG_NONFINITE | mir.FLAG_RECOMPUTED_F64)).all()
        else:
            assert not fl.any()
        assert e < 2e-2


@pytest.mark.parametrize("cheb_eval", ["clenshaw", "ps"])
def test_bottleneck_set_full_size_chebyshev(mir, cheb_eval):
    """The bottleneck-50 set (53 parameters, blocks of 256 and 1024 with
    ragged edges, Chebyshev degree 16 summed by Clenshaw's recurrence or the
    Paterson-Stockmeyer split, momentum grafting): every parameter within
    the stated 1e-4 of the oracle's exact polynomial at each of 3 steps."""
    import torch
    shapes = synthetic.bottleneck50_shapes()
    bsz = synthetic.bottleneck50_block_sizes(shapes)
    grads = synthetic.gaussian_grads(5, shapes, 3, 0.1)
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=lambda m, n: 1024 if max(m, n) >= 2048 else 256, beta2=0.999, eps=1e-12,
                      root=mir.RootOpts(method="chebyshev", cheb_degree=16, cheb_eval=cheb_eval), graft="momentum",
                      lr=0.1, momentum=0.9)
    sample = list(range(len(shapes)))   # all 53 parameters
    sshapes = [shapes[i] for i in sample]
    orc = oracle.ShampooOracle(sshapes, [bsz[i] for i in sample], beta2=0.999, eps=1e-12, root="chebyshev",
                               cheb_degree=16, graft="momentum", lr=0.1, momentum=0.9)
    Wo = [np.zeros(s) for s in sshapes]
    for t in range(3):
        opt.step([to_dev(g) for g in grads[t]])
        orc.step(Wo, [grads[t][i].astype(np.float64) for i in sample])
        torch.cuda.synchronize()
        e = max(rel_fro(W[i].cpu().numpy(), Wo[k]) for k, i in enumerate(sample))
        log(f"bottleneck set step {t + 1}: sampled rel err {e:.2e}")
        assert e < 1e-4
    assert sum(int(f.sum().item()) for f in opt.flags()) == 0

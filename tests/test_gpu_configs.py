"""GPU parity at the full workload sizes, checked on sampled outputs.

* 1024 SPD blocks 512 x 512 with lambda in [1e-8, 1] (the benchmark input),
  Newton-DB 28 + 17 with power-iteration scaling, in the launch configuration
  the benchmark times: float64 to 1e-4 on sampled blocks; float32 blocks are
  either flagged non-finite or match on the eigen-directions float32 resolves.
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
from helpers import rel_fro, to_dev, bf16_tensor, log, f32_direction_floor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mir():
    import matrix_inverse_roots_amd as m
    return m


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
    X = out[sample].cpu().numpy()
    del inp, out
    worst = max(rel_fro(X[k], oracle.inverse_root_eigh(A64[i], 4)) for k, i in enumerate(sample))
    log(f"1024 x 512^2 f64 NDB: worst sampled rel err {worst:.2e}")
    assert worst < 1e-4
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


def _decoder_run(mir, compute, stats64, sample):
    import torch
    shapes = synthetic.decoder_shapes()
    grads = synthetic.gaussian_grads(4, shapes, 3, 0.02, dtype="bf16")
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=1024, beta2=0.999, eps=1e-12, root=mir.RootOpts(method="cn", iters=34, compute=compute),
                      graft="adam", lr=1e-3, grad_dtype=torch.bfloat16,
                      stats_dtype=torch.float64 if stats64 else torch.float32)
    sshapes = [shapes[i] for i in sample]
    orc = oracle.ShampooOracle(sshapes, [1024] * len(sample), beta2=0.999, eps=1e-12, graft="adam", lr=1e-3)
    Wo = [np.zeros(s) for s in sshapes]
    errs = []
    tol = 1e-4
    for t in range(3):
        opt.step([bf16_tensor(g) for g in grads[t]])
        orc.step(Wo, [synthetic.bf16_bits_to_f32(grads[t][i]).astype(np.float64) for i in sample])
        if not stats64:
            for b in range(orc.table.shape[0]):
                tol = max(tol, 4 * f32_direction_floor(orc.L[b], orc.R[b], eps=1e-12))
        torch.cuda.synchronize()
        e = max(rel_fro(W[i].cpu().numpy(), Wo[k]) for k, i in enumerate(sample))
        nflag = sum(int(f.sum().item()) for f in opt.flags())
        log(f"decoder set ({compute}, stats {'f64' if stats64 else 'f32'}) step {t + 1}: sampled rel err {e:.2e} "
            f"(tolerance {tol:.2e}), flags {nflag}")
        assert nflag == 0
        errs.append((e, tol))
    return errs


def test_decoder_set_full_size_f64(mir):
    errs = _decoder_run(mir, "f64", True, sample=[0, 1, 2, 3, 46, 47])
    assert all(e < t for e, t in errs)


def test_decoder_set_full_size_f32(mir):
    errs = _decoder_run(mir, "f32", False, sample=[0, 3, 45])
    assert all(e < t for e, t in errs)


def test_decoder_set_full_size_cn_half_products(mir):
    """The decoder set with coupled Newton on half-precision products and the
    float64 fallback, as the benchmark's half-product step runs it: step 1's
    single-Gram factors diverge in half precision and are recomputed in
    float64; steps 2 and 3 converge in half precision on every factor;
    sampled parameters within the half-precision bar."""
    import torch
    shapes = synthetic.decoder_shapes()
    grads = synthetic.gaussian_grads(4, shapes, 3, 0.02, dtype="bf16")
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=1024, beta2=0.999, eps=1e-12, root=mir.RootOpts(method="cn", iters=34, compute="f16"),
                      graft="adam", lr=1e-3, grad_dtype=torch.bfloat16, fallback="f64")
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
        log(f"decoder set (half products) step {t + 1}: sampled rel err {e:.2e}, flags {np.unique(fl).tolist()}")
        if t == 0:
            assert (fl == (mir.FLAG_NONFINITE | mir.FLAG_RECOMPUTED_F64)).all()
        else:
            assert not fl.any()
        assert e < 2e-2


@pytest.mark.parametrize("cheb_eval", ["clenshaw", "ps"])
def test_bottleneck_set_full_size_chebyshev(mir, cheb_eval):
    import torch
    shapes = synthetic.bottleneck50_shapes()
    bsz = synthetic.bottleneck50_block_sizes(shapes)
    grads = synthetic.gaussian_grads(5, shapes, 3, 0.1)
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=lambda m, n: 1024 if max(m, n) >= 2048 else 256, beta2=0.999, eps=1e-12,
                      root=mir.RootOpts(method="chebyshev", cheb_degree=16, cheb_eval=cheb_eval), graft="momentum",
                      lr=0.1, momentum=0.9)
    sample = [0, 1, 2, 3, 14, 24, 40, 41, 48, 51, 52]
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

"""GPU parity of packing, statistics, preconditioning and the full step
against the CPU float64 oracle (bit-exact where the arithmetic is exact)."""

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


SHAPES = [(300, 130), (64, 64), (5, 700), (128, 128)]


@pytest.mark.parametrize("dt", ["f32", "bf16", "f64"])
def test_pack_unpack_bit_exact(mir, dt):
    import torch
    B = 128
    gen = np.random.default_rng(1)
    mats32 = [gen.standard_normal(s).astype(np.float32) for s in SHAPES]
    table = mir.shampoo_plan_blocks(SHAPES, [B] * len(SHAPES))
    tdev = mir.table_to_device(table)
    if dt == "bf16":
        bits = [synthetic.f32_to_bf16_bits(m) for m in mats32]
        dmats = [bf16_tensor(b) for b in bits]
        host = [synthetic.bf16_bits_to_f32(b) for b in bits]
        tdt = torch.bfloat16
    elif dt == "f64":
        host = [m.astype(np.float64) for m in mats32]
        dmats = [to_dev(m) for m in host]
        tdt = torch.float64
    else:
        host = mats32
        dmats = [to_dev(m) for m in mats32]
        tdt = torch.float32
    nblk = table.shape[0]
    st = torch.full((nblk, B, B), 7.0, dtype=tdt, device="cuda")
    stt = torch.full((nblk, B, B), 7.0, dtype=tdt, device="cuda")
    mir.shampoo_pack_blocks(dmats, tdev, B, st, stt)
    torch.cuda.synchronize()
    want = oracle.pack_blocks([h.astype(np.float64) for h in host], table.astype(np.int64), B)
    got = st.float().cpu().numpy().astype(np.float64)
    gott = stt.float().cpu().numpy().astype(np.float64)
    assert np.array_equal(got, want)
    assert np.array_equal(gott, np.swapaxes(want, 1, 2))
    if dt == "f32":
        outs = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in SHAPES]
        mir.shampoo_unpack_blocks(st, tdev, B, outs)
        torch.cuda.synchronize()
        for o, h in zip(outs, host):
            assert np.array_equal(o.cpu().numpy(), h)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("B", [128, 192])
def test_stats_integer_gradients_bit_exact(mir, dt, B):
    import torch
    gen = np.random.default_rng(B)
    nblk = 3
    # small integers: every product and partial sum is exact in float32
    G = [gen.integers(-4, 5, size=(B, B)).astype(np.float32) for _ in range(2)]
    LR = torch.zeros((2 * nblk, B, B), dtype=torch.float32, device="cuda")
    Lo = [np.zeros((B, B)) for _ in range(nblk)]
    Ro = [np.zeros((B, B)) for _ in range(nblk)]
    for g in G:
        stack = np.stack([np.roll(g, i, axis=0) for i in range(nblk)])
        if dt == "bf16":
            gs = bf16_tensor(synthetic.f32_to_bf16_bits(stack))
            gts = bf16_tensor(synthetic.f32_to_bf16_bits(np.ascontiguousarray(np.swapaxes(stack, 1, 2))))
        else:
            gs = to_dev(stack)
            gts = to_dev(np.ascontiguousarray(np.swapaxes(stack, 1, 2)))
        mir.shampoo_update_stats(gs, gts, LR, 1.0)
        for i in range(nblk):
            Lo[i], Ro[i] = oracle.update_stats(Lo[i], Ro[i], stack[i], 1.0)
    torch.cuda.synchronize()
    got = LR.cpu().numpy().astype(np.float64)
    for i in range(nblk):
        assert np.array_equal(got[i], Lo[i])
        assert np.array_equal(got[nblk + i], Ro[i])


def test_stats_ema_gaussian(mir):
    import torch
    B, nblk, b2 = 256, 4, 0.999
    gen = np.random.default_rng(2)
    LR = torch.zeros((2 * nblk, B, B), dtype=torch.float32, device="cuda")
    Lo = [np.zeros((B, B)) for _ in range(nblk)]
    Ro = [np.zeros((B, B)) for _ in range(nblk)]
    for _ in range(3):
        st = (gen.standard_normal((nblk, B, B)) * 0.02).astype(np.float32)
        mir.shampoo_update_stats(to_dev(st), to_dev(np.ascontiguousarray(np.swapaxes(st, 1, 2))), LR, b2)
        for i in range(nblk):
            Lo[i], Ro[i] = oracle.update_stats(Lo[i], Ro[i], st[i], b2)
    torch.cuda.synchronize()
    got = LR.cpu().numpy()
    # float32 dot products of length K accumulated in one register: |error|
    # <= K u32 |x||y| per entry (K = 256: 1.5e-5)
    for i in range(nblk):
        assert rel_fro(got[i], Lo[i]) < B * 2.0 ** -24 and rel_fro(got[nblk + i], Ro[i]) < B * 2.0 ** -24
        assert np.array_equal(got[i], got[i].T)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_stats_kernels_bit_identical(mir, dt):
    """Gaussian gradients, EMA statistics: a 192-side stack runs on the
    64-tile kernel, the same blocks zero-padded to 256 on the persistent
    128-tile kernel (bf16 operands into float32 for dt = bf16); the k order
    is the same and the padding adds exact zeros, so the valid regions agree
    bit for bit, and the padding stays zero."""
    import torch
    nblk, v, b2 = 3, 192, 0.999
    gen = np.random.default_rng(7)
    outs = []
    for B in (v, 256):
        LR = torch.zeros((2 * nblk, B, B), dtype=torch.float32, device="cuda")
        g2 = np.random.default_rng(7)
        for _ in range(2):
            st = np.zeros((nblk, B, B), dtype=np.float32)
            st[:, :v, :v] = (g2.standard_normal((nblk, v, v)) * 0.02).astype(np.float32)
            stt = np.ascontiguousarray(np.swapaxes(st, 1, 2))
            if dt == "bf16":
                gs = bf16_tensor(synthetic.f32_to_bf16_bits(st))
                gts = bf16_tensor(synthetic.f32_to_bf16_bits(stt))
            else:
                gs, gts = to_dev(st), to_dev(stt)
            mir.shampoo_update_stats(gs, gts, LR, b2)
        torch.cuda.synchronize()
        outs.append(LR.cpu().numpy())
    small, big = outs
    np.testing.assert_array_equal(small, big[:, :v, :v])
    assert not big[:, v:, :].any() and not big[:, :, v:].any()
    del gen


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_precondition_vs_oracle(mir, dt):
    import torch
    B, nblk = 256, 3
    gen = np.random.default_rng(4)
    roots = np.concatenate([synthetic.spd_stack(30, nblk, B, 0.1, 1.0),
                            synthetic.spd_stack(31, nblk, B, 0.1, 1.0)]).astype(np.float32)
    G = gen.standard_normal((nblk, B, B)).astype(np.float32)
    if dt == "bf16":
        bits = synthetic.f32_to_bf16_bits(G)
        gdev = bf16_tensor(bits)
        G = synthetic.bf16_bits_to_f32(bits)
    else:
        gdev = to_dev(G)
    D = torch.empty((nblk, B, B), dtype=torch.float32, device="cuda")
    mir.shampoo_precondition(to_dev(roots), gdev, D)
    torch.cuda.synchronize()
    Dh = D.cpu().numpy()
    for i in range(nblk):
        ref = oracle.precondition(roots[i].astype(np.float64), G[i], roots[nblk + i].astype(np.float64))
        assert rel_fro(Dh[i], ref) < 1e-5


@pytest.mark.parametrize("gdt", ["f32", "bf16"])
def test_float64_statistics_and_direction(mir, gdt):
    """float64 statistics (gradients widened exactly) and float64 roots in the
    preconditioning products: sums of exact float64 products of length K
    accumulate at most K u64 relative error."""
    import torch
    B, nblk, b2 = 256, 3, 0.999
    gen = np.random.default_rng(5)
    LR = torch.zeros((2 * nblk, B, B), dtype=torch.float64, device="cuda")
    Lo = [np.zeros((B, B)) for _ in range(nblk)]
    Ro = [np.zeros((B, B)) for _ in range(nblk)]
    for _ in range(2):
        st = (gen.standard_normal((nblk, B, B)) * 0.02).astype(np.float32)
        stt = np.ascontiguousarray(np.swapaxes(st, 1, 2))
        if gdt == "bf16":
            bits, bitst = synthetic.f32_to_bf16_bits(st), synthetic.f32_to_bf16_bits(stt)
            mir.shampoo_update_stats(bf16_tensor(bits), bf16_tensor(bitst), LR, b2)
            st = synthetic.bf16_bits_to_f32(bits)
        else:
            mir.shampoo_update_stats(to_dev(st), to_dev(stt), LR, b2)
        for i in range(nblk):
            Lo[i], Ro[i] = oracle.update_stats(Lo[i], Ro[i], st[i], b2)
    torch.cuda.synchronize()
    got = LR.cpu().numpy()
    for i in range(nblk):
        assert rel_fro(got[i], Lo[i]) < 1e-13 and rel_fro(got[nblk + i], Ro[i]) < 1e-13
    roots = np.concatenate([synthetic.spd_stack(32, nblk, B, 0.1, 1.0), synthetic.spd_stack(33, nblk, B, 0.1, 1.0)])
    D = torch.empty((nblk, B, B), dtype=torch.float32, device="cuda")
    gdev = to_dev(st) if gdt == "f32" else bf16_tensor(synthetic.f32_to_bf16_bits(st))
    mir.shampoo_precondition(to_dev(roots), gdev, D)
    torch.cuda.synchronize()
    Dh = D.cpu().numpy()
    for i in range(nblk):
        ref = oracle.precondition(roots[i], st[i].astype(np.float64), roots[nblk + i])
        # the float64 products end in one rounding to float32
        assert rel_fro(Dh[i], ref) < 2 ** -23


def run_steps(mir, shapes, block_sizes, grads, steps, hp, root_kw, oracle_root="eigh", grad_bf16=False,
              cheb_degree=16, check_every=True, stats64=False, allow_flags=False):
    """Run the GPU optimizer and the oracle side by side; return the worst
    parameter relative error after each checked step.  ``stats64`` keeps
    statistics, roots and preconditioning products in float64."""
    import torch
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=(lambda m, n: block_sizes[(m, n)]) if isinstance(block_sizes, dict) else block_sizes,
                      root=mir.RootOpts(**root_kw), grad_dtype=torch.bfloat16 if grad_bf16 else torch.float32,
                      stats_dtype=torch.float64 if stats64 else torch.float32, **hp)
    bs_list = [block_sizes[s] for s in shapes] if isinstance(block_sizes, dict) else [block_sizes] * len(shapes)
    orc = oracle.ShampooOracle(shapes, bs_list, beta2=hp["beta2"], eps=hp["eps"], root=oracle_root,
                               cheb_degree=cheb_degree, graft=hp["graft"], lr=hp["lr"],
                               momentum=hp.get("momentum", 0.9))
    Wo = [np.zeros(s) for s in shapes]
    errs = []
    for t in range(steps):
        gs = grads[t]
        if grad_bf16:
            dg = [bf16_tensor(g) for g in gs]
            hg = [synthetic.bf16_bits_to_f32(g).astype(np.float64) for g in gs]
        else:
            dg = [to_dev(g) for g in gs]
            hg = [g.astype(np.float64) for g in gs]
        opt.step(dg)
        orc.step(Wo, hg)
        if check_every or t == steps - 1:
            torch.cuda.synchronize()
            e = max(rel_fro(w.cpu().numpy(), wo) for w, wo in zip(W, Wo))
            fl = sum(int(f.sum().item()) for f in opt.flags())
            errs.append(e)
            log(f"step {t + 1}: worst parameter rel err {e:.2e}, flags {fl}")
            assert allow_flags or fl == 0
    return errs


def test_single_matrix_ten_steps(mir):
    """One 256 x 128 float32 parameter, block 128 (2 blocks), N(0,1) gradients
    from seed 0, 10 steps, beta2 = 1, eps = 1e-12, SGD grafting lr 0.1;
    coupled Newton 30 iterations.  The step-1 factors of a square Gaussian
    block have condition numbers up to 1e6; the float64 path (statistics,
    chain and products) meets the stated 1e-4 at every step."""
    grads = synthetic.gaussian_grads(0, [(256, 128)], 10, 1.0)
    errs = run_steps(mir, [(256, 128)], 128, grads, 10,
                     dict(beta2=1.0, eps=1e-12, graft="sgd", lr=0.1), dict(method="cn", iters=30, compute="f64"),
                     stats64=True)
    assert all(e < 1e-4 for e in errs)


def test_single_matrix_ten_steps_f32_diagnostic(mir):
    """Float32 diagnostic, not a parity test: the same ten steps with float32
    statistics and chain.  Float32 rounding of the step-1 factors (condition
    number 1e6) already moves the direction by about 5e-4, so this path misses
    the stated 1e-4 (measured 6.3e-4 at step 1, 2.0e-4 at step 10); a fixed
    ceiling of 1e-3 guards against regressions."""
    grads = synthetic.gaussian_grads(0, [(256, 128)], 10, 1.0)
    errs = run_steps(mir, [(256, 128)], 128, grads, 10,
                     dict(beta2=1.0, eps=1e-12, graft="sgd", lr=0.1), dict(method="cn", iters=30, compute="f32"))
    log(f"single parameter, float32 diagnostic, error per step: {errs}")
    assert all(e < 1e-3 for e in errs)


@pytest.mark.parametrize("tol", [0.0, 1e-4])
def test_ragged_blocks_momentum_and_ndb(mir, tol):
    """Ragged blocks (grouped roots), Newton-DB with power scaling, momentum
    grafting, float32; with a tolerance each group's calls stop at
    convergence.  eps = 1e-3 bounds the factors' condition numbers, and the
    float32 path meets the stated 1e-4."""
    shapes = [(300, 130), (64, 64), (5, 200)]
    grads = synthetic.gaussian_grads(21, shapes, 3, 0.1)
    errs = run_steps(mir, shapes, 128, grads, 3,
                     dict(beta2=0.999, eps=1e-3, graft="momentum", lr=0.1, momentum=0.9),
                     dict(method="ndb", scaling="power", iters=24, iters2=16, tol=tol))
    assert all(e < 1e-4 for e in errs)


def test_ragged_blocks_half_products_tolerance(mir):
    """Ragged blocks rooted in groups by factor side (64 to 512), coupled
    Newton on half products stopping at ||M - I||_F <= 0.05 (the half copy
    of M), Adam grafting: within the half-precision bar 2e-2 of the oracle
    at every step (eps = 1e-3 bounds the factors' condition numbers)."""
    shapes = [(600, 300), (64, 200), (300, 130), (5, 40)]
    grads = synthetic.gaussian_grads(29, shapes, 3, 0.1)
    errs = run_steps(mir, shapes, 512, grads, 3, dict(beta2=0.999, eps=1e-3, graft="adam", lr=0.01),
                     dict(method="cn", iters=34, compute="f16", tol=0.05))
    log(f"ragged blocks, half products with a tolerance: error per step {errs}")
    assert all(e < 2e-2 for e in errs)


@pytest.mark.parametrize("shapes,B", [([(300, 130), (64, 64), (5, 200)], 128), ([(512, 256), (256, 768)], 256)])
def test_bfloat16_preconditioning(mir, shapes, B):
    """Preconditioning on bfloat16 matrix cores (roots and G R^{-1/4} rounded
    to bfloat16, float32 accumulation) within the bfloat16 bar 2e-2 of the
    oracle, on ragged blocks (extents, tile lists of 64-tiles) and on full
    blocks (the persistent 128-tile kernel); eps = 1e-3 bounds the factors'
    condition numbers, gradients bfloat16 N(0, 0.1^2), Adam grafting."""
    import torch
    grads = synthetic.gaussian_grads(23, shapes, 3, 0.1, dtype="bf16")
    errs = run_steps(mir, shapes, B, grads, 3,
                     dict(beta2=0.999, eps=1e-3, graft="adam", lr=0.01, precondition_dtype=torch.bfloat16),
                     dict(method="cn", iters=30), grad_bf16=True)
    log(f"bfloat16 preconditioning, B {B}: error per step {errs}")
    assert all(e < 2e-2 for e in errs)


def test_decoder_layer_adam_bf16(mir):
    """One decoder layer of the d_model 1024 / MLP 4096 set (QKV, out, MLP up,
    MLP down), bfloat16 gradients N(0, 0.02^2), beta2 = 0.999, eps = 1e-12,
    Adam grafting lr 1e-3, block 1024, 3 steps; coupled Newton 34 iterations
    with statistics, chain and products in float64: the stated 1e-4."""
    shapes = synthetic.decoder_shapes(layers=1)
    grads = synthetic.gaussian_grads(4, shapes, 3, 0.02, dtype="bf16")
    errs = run_steps(mir, shapes, 1024, grads, 3, dict(beta2=0.999, eps=1e-12, graft="adam", lr=1e-3),
                     dict(method="cn", iters=34, compute="f64"), grad_bf16=True, check_every=True, stats64=True)
    assert all(e < 1e-4 for e in errs)


def test_decoder_layer_adam_bf16_f32_diagnostic(mir):
    """Float32 diagnostic, not a parity test: the decoder layer with float32
    statistics and chain.  The step-1 factors are single Gram matrices of
    square Gaussian blocks (condition number about 4 B^2 = 4e6), beyond what
    float32 statistics resolve, so this path misses 1e-4 (measured 3.1e-2);
    fixed ceiling 5e-2."""
    shapes = synthetic.decoder_shapes(layers=1)
    grads = synthetic.gaussian_grads(4, shapes, 3, 0.02, dtype="bf16")
    errs = run_steps(mir, shapes, 1024, grads, 3, dict(beta2=0.999, eps=1e-12, graft="adam", lr=1e-3),
                     dict(method="cn", iters=34), grad_bf16=True, check_every=True)
    log(f"decoder layer float32 diagnostic, error per step: {errs}")
    assert all(e < 5e-2 for e in errs)


def test_decoder_layer_newton_tolerance(mir):
    """The decoder layer with float64 statistics and a float64 coupled Newton
    chain stopping at ||M - I||_F <= 1e-9 instead of the fixed 34
    iterations: the stated 1e-4."""
    shapes = synthetic.decoder_shapes(layers=1)
    grads = synthetic.gaussian_grads(4, shapes, 3, 0.02, dtype="bf16")
    hp = dict(beta2=0.999, eps=1e-12, graft="adam", lr=1e-3)
    errs = run_steps(mir, shapes, 1024, grads, 3, hp, dict(method="cn", iters=34, tol=1e-9, compute="f64"),
                     grad_bf16=True, check_every=True, stats64=True)
    log(f"decoder layer, Newton tolerance (float64), error per step: {errs}")
    assert all(e < 1e-4 for e in errs)


def test_decoder_layer_newton_tolerance_f32_diagnostic(mir):
    """Float32 diagnostic, not a parity test: float32 statistics and chain
    stopping at ||M - I||_F <= 1e-4; the same float32 limit as the fixed
    count (measured 3.1e-2), fixed ceiling 5e-2."""
    shapes = synthetic.decoder_shapes(layers=1)
    grads = synthetic.gaussian_grads(4, shapes, 3, 0.02, dtype="bf16")
    hp = dict(beta2=0.999, eps=1e-12, graft="adam", lr=1e-3)
    errs = run_steps(mir, shapes, 1024, grads, 3, hp, dict(method="cn", iters=34, tol=1e-4), grad_bf16=True,
                     check_every=True)
    log(f"decoder layer, Newton tolerance (float32 diagnostic), error per step: {errs}")
    assert all(e < 5e-2 for e in errs)


@pytest.mark.parametrize("tol", [0.0, 1e-4])
def test_decoder_layer_f32_chain_residual_checked(mir, tol):
    """The decoder layer with float64 statistics and a float32 coupled Newton
    chain (fixed 34 iterations, or stopping at ||M - I||_F <= 1e-4) whose
    device residual is checked against 1e-4, with the float64 recomputation
    as fallback: step 1's single-Gram factors fail the check and are
    recomputed in float64, later factors (condition number 33, then 14) keep
    their float32 roots.  The stated 1e-4 at every step."""
    shapes = synthetic.decoder_shapes(layers=1)
    grads = synthetic.gaussian_grads(4, shapes, 3, 0.02, dtype="bf16")
    errs = run_steps(mir, shapes, 1024, grads, 3,
                     dict(beta2=0.999, eps=1e-12, graft="adam", lr=1e-3, fallback="f64", residuals=True),
                     dict(method="cn", iters=34, tol=tol, residual_bound=1e-4), grad_bf16=True, check_every=True,
                     stats64=True, allow_flags=True)
    log(f"decoder layer, float32 chain checked by its residual (tol {tol}), error per step: {errs}")
    assert all(e < 1e-4 for e in errs)


def test_decoder_layer_cn_half_products_with_f64_fallback(mir):
    """The decoder layer with coupled Newton on half-precision products (the
    pages' CN-FP16 configuration).  Step 1's factors are single square
    Gram matrices: their scaled smallest eigenvalues (about 1e-8) sit below
    the half-precision rounding of the scaled factor, the half chain diverges
    on all 24 of them, and the float64 fallback recomputes them.  From step
    2 on the factors are sums of several Gram matrices (condition number 33,
    then 14) and the half chain converges on every factor.  The parameters
    stay within the half-precision bar of the oracle at every step."""
    import torch
    shapes = synthetic.decoder_shapes(layers=1)
    grads = synthetic.gaussian_grads(4, shapes, 3, 0.02, dtype="bf16")
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=1024, beta2=0.999, eps=1e-12, root=mir.RootOpts(method="cn", iters=34, compute="f16"),
                      graft="adam", lr=1e-3, grad_dtype=torch.bfloat16, fallback="f64")
    orc = oracle.ShampooOracle(shapes, [1024] * len(shapes), beta2=0.999, eps=1e-12, graft="adam", lr=1e-3)
    Wo = [np.zeros(s) for s in shapes]
    for t in range(3):
        for f in opt.flags():
            f.zero_()
        opt.step([bf16_tensor(g) for g in grads[t]])
        orc.step(Wo, [synthetic.bf16_bits_to_f32(g).astype(np.float64) for g in grads[t]])
        torch.cuda.synchronize()
        fl = torch.cat(opt.flags()).cpu().numpy()
        e = max(rel_fro(w.cpu().numpy(), wo) for w, wo in zip(W, Wo))
        log(f"decoder layer CN f16 step {t + 1}: worst parameter rel err {e:.2e}, flags {np.unique(fl).tolist()}")
        if t == 0:
            assert (fl == (mir.FLAG_NONFINITE | mir.FLAG_RECOMPUTED_F64)).all()
        else:
            assert not fl.any()
        assert e < 2e-2


@pytest.mark.parametrize("cheb_eval,compute", [("clenshaw", "f32"), ("ps", "f32"), ("ps", "f64"),
                                               ("clenshaw", "f16"), ("ps", "f16")])
def test_bottleneck_subset_chebyshev_momentum(mir, cheb_eval, compute):
    """First 12 matrices of the 50-layer bottleneck CNN set (1x1 and 3x3
    kernels as (out, in k k)), block sizes 256 / 1024 by size, ragged edges,
    Chebyshev degree 16 (float32, half-precision or float64 products),
    SGD-momentum 0.9 grafting lr 0.1, gradients variance 1e-2, 3 steps; the
    oracle evaluates the same fitted polynomial exactly."""
    stats64 = compute == "f64"
    shapes = synthetic.bottleneck50_shapes()[:12]
    bs = dict(zip(shapes, synthetic.bottleneck50_block_sizes(shapes)))
    grads = synthetic.gaussian_grads(5, shapes, 3, 0.1)
    errs = run_steps(mir, shapes, bs, grads, 3,
                     dict(beta2=0.999, eps=1e-12, graft="momentum", lr=0.1, momentum=0.9),
                     dict(method="chebyshev", cheb_degree=16, cheb_eval=cheb_eval, compute=compute),
                     oracle_root="chebyshev", stats64=stats64)
    # float64 statistics and chain: the error is the float32 weights' rounding;
    # half-precision products take the half-precision bar
    bar = {"f64": 1e-6, "f32": 1e-4, "f16": 2e-2}[compute]
    assert all(e < bar for e in errs)


def test_step_deterministic_and_infrequent_roots(mir):
    import torch
    shapes = [(256, 256), (128, 384)]
    grads = synthetic.gaussian_grads(7, shapes, 4, 1.0)
    outs = []
    for _ in range(2):
        W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
        opt = mir.Shampoo(W, block_size=128, beta2=0.9, eps=1e-6, root=mir.RootOpts(method="cn", iters=30),
                          graft="sgd", lr=0.1, precondition_frequency=2)
        for t in range(4):
            opt.step([to_dev(g) for g in grads[t]])
        torch.cuda.synchronize()
        outs.append([w.cpu().numpy() for w in W])
    for a, b in zip(*outs):
        assert np.array_equal(a, b)
    # frequency 2: steps 1 and 3 recompute roots; steps 2 and 4 reuse them
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=128, beta2=0.9, eps=1e-6, root=mir.RootOpts(method="cn", iters=30, compute="f64"),
                      graft="none", lr=1.0, precondition_frequency=2, stats_dtype=torch.float64)
    Wo = [np.zeros(s) for s in shapes]
    t_ = oracle.plan_blocks(shapes, [128, 128])
    L = [np.zeros((int(t_[b, 5]),) * 2) for b in range(t_.shape[0])]
    R = [np.zeros((int(t_[b, 6]),) * 2) for b in range(t_.shape[0])]
    roots = [None] * t_.shape[0]
    for t in range(4):
        opt.step([to_dev(g) for g in grads[t]])
        for b in range(t_.shape[0]):
            p = int(t_[b, 0])
            rs, cs = oracle.block_slices(t_, b)
            g = grads[t][p][rs, cs].astype(np.float64)
            L[b], R[b] = oracle.update_stats(L[b], R[b], g, 0.9)
            if t % 2 == 0:
                roots[b] = (oracle.inverse_root_eigh(L[b], 4, 1e-6), oracle.inverse_root_eigh(R[b], 4, 1e-6))
            Wo[p][rs, cs] -= oracle.precondition(roots[b][0], g, roots[b][1])
    torch.cuda.synchronize()
    e = max(rel_fro(w.cpu().numpy(), wo) for w, wo in zip(W, Wo))
    log(f"infrequent roots: rel err {e:.2e}")
    assert e < 1e-4


@pytest.mark.parametrize("graft,blockwise", [("sgd", True), ("momentum", True), ("adam", True), ("none", False)])
def test_blockwise_and_no_graft_vs_oracle(mir, graft, blockwise):
    """Block-wise grafting (norms per block: [DASH] "2. Preliminaries on
    Shampoo" speaks of block-wise Adam grafting) and graft "none" (W <- W -
    lr D) on ragged blocks, float64 statistics and chain, 3 steps, against
    the oracle."""
    import torch
    shapes = [(300, 130), (64, 200)]
    grads = synthetic.gaussian_grads(23, shapes, 3, 0.1)
    lr = 0.05
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=128, beta2=0.9, eps=1e-3, root=mir.RootOpts(method="cn", iters=30, compute="f64"),
                      graft=graft, lr=lr, momentum=0.9, graft_blockwise=blockwise, stats_dtype=torch.float64)
    orc = oracle.ShampooOracle(shapes, [128, 128], beta2=0.9, eps=1e-3, graft=graft, lr=lr, momentum=0.9,
                               graft_blockwise=blockwise)
    Wo = [np.zeros(s) for s in shapes]
    for t in range(3):
        opt.step([to_dev(g) for g in grads[t]])
        orc.step(Wo, [g.astype(np.float64) for g in grads[t]])
        torch.cuda.synchronize()
        e = max(rel_fro(w.cpu().numpy(), wo) for w, wo in zip(W, Wo))
        log(f"graft {graft} blockwise={blockwise} step {t + 1}: worst parameter rel err {e:.2e}")
        assert e < 1e-5
    assert sum(int(f.sum().item()) for f in opt.flags()) == 0


def test_whole_parameter_blocks(mir):
    """block_size 0: each parameter is one block of side max(m, n) (ragged,
    padded to a multiple of 64 in the stack), against the oracle's blocking
    of the same rule; float64 statistics and chain."""
    import torch
    shapes = [(100, 37), (70, 90)]
    grads = synthetic.gaussian_grads(29, shapes, 2, 0.1)
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=0, beta2=0.9, eps=1e-3, root=mir.RootOpts(method="cn", iters=30, compute="f64"),
                      graft="sgd", lr=0.1, stats_dtype=torch.float64)
    orc = oracle.ShampooOracle(shapes, [0, 0], beta2=0.9, eps=1e-3, graft="sgd", lr=0.1)
    assert orc.table.shape[0] == 2
    Wo = [np.zeros(s) for s in shapes]
    for t in range(2):
        opt.step([to_dev(g) for g in grads[t]])
        orc.step(Wo, [g.astype(np.float64) for g in grads[t]])
    torch.cuda.synchronize()
    e = max(rel_fro(w.cpu().numpy(), wo) for w, wo in zip(W, Wo))
    log(f"whole-parameter blocks: worst rel err {e:.2e}")
    assert e < 1e-5


def test_reused_gradient_buffers_rewritten_in_place(mir):
    """Gradient buffers reused across steps (two sets, alternating, refilled in
    place) and then a set of fresh tensors every step: the device descriptor
    tables are kept per set of gradient pointers, so reuse uploads nothing and
    the kernels read the new contents; more than 8 distinct sets evict old
    tables.  Against the oracle with two stacks stepped concurrently."""
    import torch
    shapes = [(256, 384), (64, 200), (512, 128)]
    bs = {(256, 384): 128, (64, 200): 256, (512, 128): 256}
    steps = 12
    grads = synthetic.gaussian_grads(17, shapes, steps, 1.0)
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=lambda m, n: bs[(m, n)], beta2=0.99, eps=1e-2, graft="momentum", lr=0.1,
                      momentum=0.9, root=mir.RootOpts(method="cn", iters=30))
    assert len(opt.stacks) == 2
    orc = oracle.ShampooOracle(shapes, [bs[s] for s in shapes], beta2=0.99, eps=1e-2, root="eigh",
                               graft="momentum", lr=0.1, momentum=0.9)
    Wo = [np.zeros(s) for s in shapes]
    bufs = [[torch.empty(s, dtype=torch.float32, device="cuda") for s in shapes] for _ in range(2)]
    keep = []
    for t in range(steps):
        if t < 6:
            dg = bufs[t % 2]
            for d, g in zip(dg, grads[t]):
                d.copy_(torch.from_numpy(g))
        else:
            dg = [to_dev(g) for g in grads[t]]
            keep.append(dg)  # distinct pointers for every later step
        opt.step(dg)
        orc.step(Wo, [g.astype(np.float64) for g in grads[t]])
        torch.cuda.synchronize()
        e = max(rel_fro(w.cpu().numpy(), wo) for w, wo in zip(W, Wo))
        log(f"step {t + 1}: worst parameter rel err {e:.2e}")
        assert e < 1e-4
    assert sum(int(f.sum().item()) for f in opt.flags()) == 0
    assert all(len(st._desc_cache) <= 8 for st in opt.stacks)


@pytest.mark.parametrize("eps", [1e-2, 0.0])
def test_zero_gradient_parameter(mir, eps):
    """A parameter whose gradient is zero for the first two steps: its
    statistics stay 0, D = 0 and the grafted step is 0 (norm rule for
    ||D|| = 0), so its weights stay exactly 0.  With eps = 0 the zero
    statistics have no scale and their factors are flagged ZERO_SCALE with a
    zero root; with eps > 0 (1e-2, which keeps the square Gaussian blocks of
    the other parameter well conditioned in float32) the whole run matches
    the oracle."""
    import torch
    shapes = [(128, 256), (64, 64)]
    grads = synthetic.gaussian_grads(23, shapes, 4, 1.0)
    for t in (0, 1):
        grads[t][1][:] = 0.0
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=128, beta2=0.99, eps=eps, graft="momentum", lr=0.1, momentum=0.9,
                      root=mir.RootOpts(method="cn", iters=25))
    orc = oracle.ShampooOracle(shapes, [128, 128], beta2=0.99, eps=eps, root="eigh", graft="momentum", lr=0.1,
                               momentum=0.9)
    Wo = [np.zeros(s) for s in shapes]
    stack1 = [k for k, st in enumerate(opt.stacks) if st.B == 64][0]
    for t in range(4):
        opt.step([to_dev(g) for g in grads[t]])
        torch.cuda.synchronize()
        w1 = W[1].cpu().numpy()
        fl = opt.flags()[stack1].cpu().numpy()
        if t < 2:
            assert not w1.any()
            if eps == 0.0:
                assert (fl & mir.FLAG_ZERO_SCALE).all()
            else:
                assert not fl.any()
        if eps > 0.0:
            orc.step(Wo, [g.astype(np.float64) for g in grads[t]])
            e = max(rel_fro(w.cpu().numpy(), wo) if np.abs(wo).sum() else float(np.abs(w.cpu().numpy()).max())
                    for w, wo in zip(W, Wo))
            log(f"eps {eps} step {t + 1}: worst rel err {e:.2e}")
            assert e < 1e-4
    assert np.isfinite(W[0].cpu().numpy()).all() and np.isfinite(W[1].cpu().numpy()).all()


@pytest.mark.parametrize("stats_dtype", ["f32", "f64"])
def test_ragged_step_statistics_bit_exact(mir, stats_dtype):
    """Statistics of ragged blocks inside a full step, where they run as
    products with extents walking device-built tile lists: 128-tile lists on
    the persistent kernel for float32 gradients and statistics at B = 256
    and 1024, 64-tile lists on the tiled kernel at B = 192 and for float64
    statistics.  Small integer gradients make every sum exact, so L and R of
    every block (valid region and zero padding) equal the integer sums of
    G G^T and G^T G over two steps bit for bit."""
    import torch
    shapes = [(300, 700), (130, 1000), (1024, 2100), (64, 100), (250, 390)]
    bsz = {(300, 700): 256, (130, 1000): 256, (1024, 2100): 1024, (64, 100): 1024, (250, 390): 192}
    gen = np.random.default_rng(11)
    grads = [[gen.integers(-3, 4, size=s).astype(np.float32) for s in shapes] for _ in range(2)]
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    sdt = torch.float32 if stats_dtype == "f32" else torch.float64
    opt = mir.Shampoo(W, block_size=lambda m, n: bsz[(m, n)], beta2=1.0, eps=1e-3, stats_dtype=sdt,
                      root=mir.RootOpts(method="cn", iters=4, compute="f32" if stats_dtype == "f32" else "f64"),
                      graft="none", lr=0.0, group_factors=True)
    for g in grads:
        opt.step([to_dev(x) for x in g])
    torch.cuda.synchronize()
    checked = 0
    for st, idx in zip(opt.stacks, opt.members):
        LR = st.LR.cpu().numpy()
        nb = st.nblk
        assert any(int(r[5]) < st.B or int(r[6]) < st.B for r in st.table), "stack without ragged blocks"
        for b, row in enumerate(st.table):
            p, r0, c0, rows, cols = int(row[0]), int(row[3]), int(row[4]), int(row[5]), int(row[6])
            L = np.zeros((rows, rows), dtype=np.int64)
            R = np.zeros((cols, cols), dtype=np.int64)
            for g in grads:
                gb = g[idx[p]][r0:r0 + rows, c0:c0 + cols].astype(np.int64)
                L += gb @ gb.T
                R += gb.T @ gb
            Lg, Rg = LR[b], LR[nb + b]
            assert np.array_equal(Lg[:rows, :rows], L.astype(Lg.dtype))
            assert np.array_equal(Rg[:cols, :cols], R.astype(Rg.dtype))
            assert not Lg[rows:, :].any() and not Lg[:, rows:].any()
            assert not Rg[cols:, :].any() and not Rg[:, cols:].any()
            checked += 1
    assert checked == sum(st.nblk for st in opt.stacks)

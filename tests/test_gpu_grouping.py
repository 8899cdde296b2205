"""Factor-side grouping of the inverse roots in shampoo_step.

With the host table given, each factor is rooted in a stack of its own side
(rounded up to 64) instead of the block size B.  Identity padding makes the
two computations equal up to floating-point rounding order (the Frobenius
scale is summed by a different number of workgroups), so grouped and
ungrouped steps agree to float32 rounding, and both match the oracle.
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


def run(mir, shapes, bs, grads, group, **kw):
    import torch
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=bs, group_factors=group, **kw)
    for g in grads:
        opt.step([to_dev(x) for x in g])
    torch.cuda.synchronize()
    return [w.cpu().numpy() for w in W], opt


@pytest.mark.parametrize("cheb_eval", ["clenshaw", "ps"])
def test_grouped_and_ungrouped_roots_agree(cheb_eval):
    import matrix_inverse_roots_amd as mir
    shapes = synthetic.bottleneck50_shapes()
    sel = [0, 1, 2, 3, 4, 14, 24, 40, 41, 52]        # narrow and full factors in the 256 and 1024 stacks
    sh = [shapes[i] for i in sel]
    bsz = synthetic.bottleneck50_block_sizes(shapes)
    bs = lambda m, n: 1024 if max(m, n) >= 2048 else 256
    grads = synthetic.gaussian_grads(5, sh, 2, 0.1)
    kw = dict(beta2=0.999, eps=1e-12, root=mir.RootOpts(method="chebyshev", cheb_degree=16, cheb_eval=cheb_eval),
              graft="momentum", lr=0.1, momentum=0.9)
    Wg, og = run(mir, sh, bs, grads, True, **kw)
    Wu, ou = run(mir, sh, bs, grads, False, **kw)
    wsg = sum(st.ws.numel() for st in og.stacks)
    wsu = sum(st.ws.numel() for st in ou.stacks)
    worst = max(rel_fro(a, b) for a, b in zip(Wg, Wu))
    log(f"grouped vs ungrouped: worst rel diff {worst:.2e}; workspace {wsg / 2**20:.0f} vs {wsu / 2**20:.0f} MiB")
    assert worst < 1e-5
    for st in og.stacks + ou.stacks:
        assert int(st.flags.sum().item()) == 0
    # and against the oracle
    orc = oracle.ShampooOracle(sh, [bsz[i] for i in sel], beta2=0.999, eps=1e-12, root="chebyshev", cheb_degree=16,
                               graft="momentum", lr=0.1, momentum=0.9)
    Wo = [np.zeros(s) for s in sh]
    for g in grads:
        orc.step(Wo, [x.astype(np.float64) for x in g])
    e = max(rel_fro(a, b) for a, b in zip(Wg, Wo))
    log(f"grouped vs oracle: {e:.2e}")
    assert e < 1e-4


def test_grouping_reduces_root_work():
    """The planned groups cover every factor once, at its own side."""
    import torch
    import matrix_inverse_roots_amd as mir
    W = [torch.zeros(512, 640, device="cuda"), torch.zeros(64, 512, device="cuda")]
    opt = mir.Shampoo(W, block_size=512, group_factors=True)
    st = opt.stacks[0]
    sides = []
    for row in st.table:
        rows, cols = int(row[5]), int(row[6])
        sides += [(rows + 63) // 64 * 64, (cols + 63) // 64 * 64]
    work_grouped = sum(s ** 3 for s in sides)
    work_padded = len(sides) * st.B ** 3
    log(f"factor sides {sorted(sides)}: root work {work_grouped / work_padded:.2f} of the padded stack")
    assert work_grouped < work_padded
    g = [torch.randn(512, 640, device="cuda"), torch.randn(64, 512, device="cuda")]
    opt.step(g)
    torch.cuda.synchronize()
    assert int(st.flags.sum().item()) == 0
    assert all(torch.isfinite(w).all().item() for w in W)


def test_grouped_roots_with_half_products():
    """Half-precision Clenshaw products (the pages' mixed-precision
    Chebyshev) on the same subset: the grouped stacks put factors of side
    128 .. 1024 on the tiled, 128-tile and 256-tile half kernels; grouped and
    ungrouped steps agree within half-precision rounding and both match the
    oracle's exact polynomial within the half-precision bar."""
    import matrix_inverse_roots_amd as mir
    shapes = synthetic.bottleneck50_shapes()
    sel = [0, 1, 2, 3, 4, 14, 24, 40, 41, 52]
    sh = [shapes[i] for i in sel]
    bsz = synthetic.bottleneck50_block_sizes(shapes)
    bs = lambda m, n: 1024 if max(m, n) >= 2048 else 256
    grads = synthetic.gaussian_grads(5, sh, 2, 0.1)
    kw = dict(beta2=0.999, eps=1e-12, root=mir.RootOpts(method="chebyshev", cheb_degree=16, compute="f16"),
              graft="momentum", lr=0.1, momentum=0.9)
    Wg, og = run(mir, sh, bs, grads, True, **kw)
    Wu, ou = run(mir, sh, bs, grads, False, **kw)
    for st in og.stacks + ou.stacks:
        assert int(st.flags.sum().item()) == 0
    orc = oracle.ShampooOracle(sh, [bsz[i] for i in sel], beta2=0.999, eps=1e-12, root="chebyshev", cheb_degree=16,
                               graft="momentum", lr=0.1, momentum=0.9)
    Wo = [np.zeros(s) for s in sh]
    for g in grads:
        orc.step(Wo, [x.astype(np.float64) for x in g])
    eg = max(rel_fro(a, b) for a, b in zip(Wg, Wo))
    eu = max(rel_fro(a, b) for a, b in zip(Wu, Wo))
    d = max(rel_fro(a, b) for a, b in zip(Wg, Wu))
    log(f"half products: grouped vs oracle {eg:.2e}, ungrouped vs oracle {eu:.2e}, grouped vs ungrouped {d:.2e}")
    assert eg < 2e-2 and eu < 2e-2 and d < 2e-2


def test_device_factor_order_many_factors_and_sides():
    """150 parameters of (512 + r, 512 + c), r, c in 1..511, block 512: 600
    blocks and 1200 factors over all 8 sides 64..512 (more than one pass of
    the ordering kernel's 1024 threads).  Grouped roots, ordered on the
    device, give the same bits as roots at the block size."""
    import torch
    import matrix_inverse_roots_amd as mir
    rng = np.random.default_rng(44)
    shapes = [(512 + int(r), 512 + int(c)) for r, c in rng.integers(1, 512, size=(150, 2))]
    grads = synthetic.gaussian_grads(45, shapes, 2, 1.0)
    kw = dict(beta2=0.99, eps=1e-3, root=mir.RootOpts(method="cn", iters=12), graft="sgd", lr=0.1)
    Wg, og = run(mir, shapes, 512, grads, True, **kw)
    Wu, ou = run(mir, shapes, 512, grads, False, **kw)
    sides = set()
    for st in og.stacks:
        t = st.table
        sides |= {int(-(-v // 64) * 64) for v in np.concatenate([t[:, 5], t[:, 6]])}
    nf = sum(2 * st.nblk for st in og.stacks)
    log(f"{nf} factors, sides {sorted(sides)}")
    assert nf > 1024 and sides == set(range(64, 513, 64))
    assert all(np.array_equal(a, b) for a, b in zip(Wg, Wu))

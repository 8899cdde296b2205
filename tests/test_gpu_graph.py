"""Graph capture of the optimizer step (Shampoo.capture): every replay,
with eager work and synchronisations between replays, gives the same bits
as the eager step on the same gradients."""

import numpy as np
import pytest

import synthetic
from helpers import to_dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mir():
    import matrix_inverse_roots_amd as m
    return m


CASES = {
    # one parameter [256, 128] in two 128-blocks: sum of statistics, coupled Newton 30, SGD grafting
    "single_sgd": dict(shapes=[(256, 128)], bs=lambda m, n: 128,
                       kw=dict(beta2=1.0, eps=1e-12, graft="sgd", lr=0.1), root=dict(method="cn", iters=30)),
    # three stacks stepped concurrently, narrow blocks rooted in groups, momentum grafting, Chebyshev (PS split)
    "stacks_grouped_momentum": dict(
        shapes=[(256, 384), (64, 200), (512, 128), (96, 1000)],
        bs=lambda m, n: {(256, 384): 128, (64, 200): 256, (512, 128): 256, (96, 1000): 512}[(m, n)],
        kw=dict(beta2=0.999, eps=1e-6, graft="momentum", lr=0.1, momentum=0.9),
        root=dict(method="chebyshev", cheb_degree=16, cheb_eval="ps")),
    # keep-previous fallback, no grafting, Newton-DB with half products
    "keep_none_ndb_half": dict(shapes=[(512, 512), (128, 640)], bs=lambda m, n: 256,
                               kw=dict(beta2=0.99, eps=1e-3, graft="none", lr=0.05, fallback="keep"),
                               root=dict(method="ndb", iters=12, iters2=8, compute="f16")),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_graph_replays_match_eager_steps(mir, case):
    import torch
    c = CASES[case]
    shapes = c["shapes"]
    steps = 6
    grads = synthetic.gaussian_grads(21, shapes, steps, 1.0)
    Wa = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    Wb = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    kw = dict(block_size=c["bs"], root=mir.RootOpts(**c["root"]), **c["kw"])
    opt_a = mir.Shampoo(Wa, **kw)
    opt_b = mir.Shampoo(Wb, **kw)
    static = [torch.empty(s, dtype=torch.float32, device="cuda") for s in shapes]
    for d, g in zip(static, grads[0]):
        d.copy_(torch.from_numpy(g))
    opt_a.step([to_dev(g) for g in grads[0]])
    opt_b.step(static)
    replay = opt_b.capture(static)
    for t in range(1, steps):
        dg = [to_dev(g) for g in grads[t]]
        for d, g in zip(static, dg):
            d.copy_(g)
        torch.cuda.synchronize()
        replay()
        opt_a.step(dg)
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip(Wa, Wb))
        fa = [f.cpu().numpy() for f in opt_a.flags()]
        fb = [f.cpu().numpy() for f in opt_b.flags()]
        log(f"{case} replay {t}: weights identical {same}, flags {[int(f.sum()) for f in fb]}")
        assert same
        assert all(np.array_equal(x, y) for x, y in zip(fa, fb))
    assert opt_a.t == opt_b.t == steps


def test_capture_rejects_unsupported(mir):
    import torch
    W = [torch.zeros((128, 128), device="cuda")]
    g = [torch.zeros((128, 128), device="cuda")]
    for kw in (dict(graft="adam"), dict(precondition_frequency=2), dict(fallback="f64"),
               dict(root=mir.RootOpts(method="cn", iters=10, tol=1e-6))):
        opt = mir.Shampoo(W, block_size=128, **kw)
        opt.step(g)
        with pytest.raises(ValueError):
            opt.capture(g)
    opt = mir.Shampoo(W, block_size=128)
    with pytest.raises(ValueError):
        opt.capture(g)   # no eager step yet


def test_replay_after_many_eager_gradient_sets(mir):
    """Eager steps on more distinct gradient buffer sets than the descriptor
    cache holds, between replays: the captured graph keeps its own
    descriptor tables, and replays still match eager steps bit for bit."""
    import torch
    shapes = [(256, 128), (64, 96)]
    grads = synthetic.gaussian_grads(31, shapes, 16, 1.0)
    kw = dict(block_size=128, beta2=0.99, eps=1e-3, graft="momentum", lr=0.05, root=mir.RootOpts(method="cn", iters=20))
    Wa = [torch.zeros(s, device="cuda") for s in shapes]
    Wb = [torch.zeros(s, device="cuda") for s in shapes]
    opt_a, opt_b = mir.Shampoo(Wa, **kw), mir.Shampoo(Wb, **kw)
    static = [torch.empty(s, device="cuda") for s in shapes]
    for d, g in zip(static, grads[0]):
        d.copy_(torch.from_numpy(g))
    opt_a.step([to_dev(g) for g in grads[0]])
    opt_b.step(static)
    replay = opt_b.capture(static)
    held = []
    for t in range(1, 16):
        dg = [to_dev(g) for g in grads[t]]
        held.append(dg)
        if t % 5 == 0:
            for d, g in zip(static, dg):
                d.copy_(g)
            replay()
        else:
            opt_b.step(dg)   # a new buffer set every step: the cache evicts
        opt_a.step(dg)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(Wa, Wb)), t
    assert all(len(st._desc_cache) <= 8 for st in opt_b.stacks)


@pytest.mark.parametrize("compute", ["f64", "f32"])
def test_captured_inverse_root_replays_match_eager(mir, compute):
    """One shampoo_inverse_root call on the 64 x 128^2 stack (lambda in
    [1e-6, 1], coupled Newton 20) captured as a graph, as the benchmark
    times it: every replay, with an eager call on other data and a
    synchronisation between replays, gives the eager call's bits."""
    import torch
    A = synthetic.spd_stack(2, 64, 128, 1e-6, 1.0)
    A2 = synthetic.spd_stack(3, 64, 128, 1e-3, 1.0)
    dt = np.float64 if compute == "f64" else np.float32
    inp, other = to_dev(A.astype(dt)), to_dev(A2.astype(dt))
    opts = mir.RootOpts(method="cn", iters=20, compute=compute)
    ws = torch.empty(mir.shampoo_inverse_root_workspace(64, 128, 4, opts), dtype=torch.uint8, device="cuda")
    ref = torch.empty_like(inp)
    mir.shampoo_inverse_root(inp, ref, 4, opts, ws=ws)
    out, scratch = torch.empty_like(inp), torch.empty_like(inp)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mir.shampoo_inverse_root(inp, out, 4, opts, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mir.shampoo_inverse_root(inp, out, 4, opts, ws=ws)
    for r in range(4):
        out.zero_()
        mir.shampoo_inverse_root(other, scratch, 4, opts, ws=ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(out, ref)
        log(f"{compute} solve replay {r}: identical {same}")
        assert same

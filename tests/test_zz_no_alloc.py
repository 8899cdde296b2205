"""The allocation-free inverse-root entry point against the workspace one.

shampoo_inverse_root_noalloc runs the same kernels as shampoo_inverse_root
on a fixed device scratch array inside the library, so its results must be
the same bits.  Two calls in a row, the second with a smaller input (the
scratch keeps the first call's contents), and the size limit.
"""

import numpy as np
import pytest

import synthetic
from helpers import to_dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mir():
    import matrix_inverse_roots_amd as m
    return m


def both(mir, A, p, valid=None, **kw):
    import torch
    inp = to_dev(A)
    n = A.shape[0]
    vd = None if valid is None else to_dev(np.asarray(valid, dtype=np.int32))
    res = []
    for fn in (mir.shampoo_inverse_root, mir.shampoo_inverse_root_noalloc):
        out = torch.full_like(inp, float("nan"))
        flags = torch.zeros(n, dtype=torch.int32, device="cuda")
        scale = torch.zeros(n, dtype=torch.float32, device="cuda")
        resid = torch.zeros(n, dtype=torch.float32, device="cuda")
        opts = mir.RootOpts(residual_out=resid, **kw)
        if opts.scaling == "power":
            opts.pi_start = to_dev(synthetic.pi_start_vectors(7, opts.pi_vectors, A.shape[1]))
        fn(inp, out, p, opts, valid=vd, scale_out=scale, flags=flags)
        torch.cuda.synchronize()
        res.append([t.cpu().numpy() for t in (out, flags, scale, resid)])
    return res


@pytest.mark.parametrize("compute,method,scaling", [("f32", "cn", "frobenius"), ("f64", "ndb", "power"),
                                                    ("f16", "cn", "frobenius")])
def test_noalloc_matches_workspace_entry_point(mir, compute, method, scaling):
    """64 blocks 128 x 128 (the condition-1e6 stack's shape), then 5 blocks
    of 64 x 64 with ragged valid sizes: every output bit equal."""
    dt = np.float64 if compute == "f64" else np.float32
    A1 = synthetic.spd_stack(2, 64, 128, 1e-6, 1.0).astype(dt)
    A2 = synthetic.spd_stack(8, 5, 64, 1e-2, 1.0).astype(dt)
    kw = dict(method=method, scaling=scaling, compute=compute, iters=20, iters2=12)
    for A, valid in ((A1, None), (A2, [64, 50, 64, 3, 17])):
        ws_res, na_res = both(mir, A, 4, valid=valid, **kw)
        for a, b in zip(ws_res, na_res):
            np.testing.assert_array_equal(a, b)
        log(f"{compute} {method} {A.shape}: identical (flags {ws_res[1].tolist()[:5]})")


def test_noalloc_rejects_oversized_calls(mir):
    """A call that needs more than the 64 MiB scratch fails before any
    launch, with a message, and leaves the output untouched."""
    import torch
    inp = torch.zeros((64, 512, 512), dtype=torch.float32, device="cuda")
    out = torch.full_like(inp, 7.0)
    with pytest.raises(mir.ShampooError) as e:
        mir.shampoo_inverse_root_noalloc(inp, out, 4, mir.RootOpts(method="cn", iters=5))
    assert e.value.status == mir.E_WORKSPACE and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all().item())

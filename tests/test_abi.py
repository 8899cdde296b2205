"""Host-only checks of the C ABI (no GPU): the library loads, exports every
function include/shampoo.h declares, the host planner matches the oracle's
table bit for bit, and bad arguments are rejected before any launch."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def mir():
    import matrix_inverse_roots_amd as m
    return m


def declared_functions():
    src = open(os.path.join(ROOT, "include", "shampoo.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(shampoo_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported(mir):
    names = declared_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(mir.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(mir.EXPORTS) == names
    assert "gfx950" in mir.version()


def test_struct_sizes_match_header(mir, tmp_path):
    """Compile a C program against include/shampoo.h and compare every
    struct's size and field offsets with the ctypes mirrors."""
    import subprocess
    structs = {"shampoo_block": mir.Block, "shampoo_matrix": mir.Matrix, "shampoo_param": mir.Param,
               "shampoo_root_opts": mir.RootOptsC, "shampoo_step_args": mir.StepArgsC}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "shampoo.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (cname, cname))
        for f, _ in py._fields_:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (cname, f, cname, f))
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    str(src), "-o", str(exe)], check=True, capture_output=True)
    out = dict(l.rsplit(" ", 1) for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                         check=True).stdout.splitlines())
    for cname, py in structs.items():
        assert int(out[cname]) == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert int(out[cname + "." + f]) == getattr(py, f).offset, (cname, f)
    assert ctypes.sizeof(mir.Block) == 32


@pytest.mark.parametrize("case", ["dash", "decoder", "bottleneck50", "mixed"])
def test_plan_blocks_bit_exact_vs_oracle(mir, case):
    if case == "dash":
        shapes, bs = [(32000, 2048)], [1024]
    elif case == "decoder":
        shapes = synthetic.decoder_shapes()
        bs = [1024] * len(shapes)
    elif case == "bottleneck50":
        shapes = synthetic.bottleneck50_shapes()
        bs = synthetic.bottleneck50_block_sizes(shapes)
    else:
        shapes = [(300, 130), (64, 64), (5, 700), (1, 9), (77, 0), (129, 129)]
        bs = [128, 128, 256, 0, 64, 0]
    t_lib = mir.shampoo_plan_blocks(shapes, bs)
    t_orc = oracle.plan_blocks(shapes, bs)
    assert t_lib.dtype == np.int32
    assert np.array_equal(t_lib.astype(np.int64), t_orc)


def test_plan_blocks_rejects_bad_input(mir):
    with pytest.raises(mir.ShampooError) as e:
        mir.shampoo_plan_blocks([(-1, 4)], [2])
    assert e.value.status == mir.E_INVALID
    # capacity too small
    shapes = np.asarray([[10, 10]], dtype=np.int64)
    bs = np.asarray([4], dtype=np.int32)
    out = np.zeros((2, 8), dtype=np.int32)
    n = ctypes.c_int64(2)
    st = mir.lib.shampoo_plan_blocks(shapes.ctypes.data, bs.ctypes.data, 1, out.ctypes.data, ctypes.byref(n))
    assert st == mir.E_INVALID and n.value == 9


def test_workspace_queries_and_support_matrix(mir):
    o = mir.RootOpts(method="ndb", iters=28, iters2=17, scaling="power", pi_vectors=16)
    b = mir.shampoo_inverse_root_workspace(1024, 512, 4, o)
    assert b >= 1024 * 512 * 512 * 4 * 3
    # same plan: iterate buffers of float64 are twice, of half products 1.5 times
    # the float32 ones (a float32 and a half part); two per-matrix double
    # arrays (scales) come first
    head = 2 * 1024 * 8
    b16 = mir.shampoo_inverse_root_workspace(1024, 512, 4, mir.RootOpts(**{**o.__dict__, "compute": "f16"}))
    b64 = mir.shampoo_inverse_root_workspace(1024, 512, 4, mir.RootOpts(**{**o.__dict__, "compute": "f64"}))
    assert 2 * (b16 - head) == 3 * (b - head) and b64 - head == 2 * (b - head)
    for opts, p, status in [
        (mir.RootOpts(method="ndb", iters=5, iters2=5), 3, mir.E_UNSUPPORTED),
        (mir.RootOpts(method="cn", iters=5), 3, mir.E_UNSUPPORTED),
        (mir.RootOpts(method="cn", iters=0), 4, mir.E_INVALID),
        (mir.RootOpts(method="cn", iters=5, compute="bf16"), 4, mir.E_UNSUPPORTED),
        (mir.RootOpts(method="ndb", iters=5, iters2=5, scaling="power", pi_vectors=32), 4, mir.E_UNSUPPORTED),
        (mir.RootOpts(method="chebyshev", cheb_degree=8, cheb_points=5), 4, mir.E_INVALID),
    ]:
        B = 1024
        with pytest.raises(mir.ShampooError) as e:
            mir.shampoo_inverse_root_workspace(4, B, p, opts)
        assert e.value.status == status, (opts, p)
    with pytest.raises(mir.ShampooError) as e:
        mir.shampoo_inverse_root_workspace(4, 100, 4, mir.RootOpts())
    assert e.value.status == mir.E_UNSUPPORTED


def test_chebyshev_split_workspace_and_validation(mir):
    """The Paterson-Stockmeyer split at degree 16 (m = 4) forms a_0 .. a_3
    in one pass while S, T_2, T_3 and T_4 are live (8 iterate buffers) where
    Clenshaw keeps 4; an unknown cheb_eval is rejected."""
    head = 2 * 94 * 8
    slot = 94 * 1024 * 1024 * 4
    cl = mir.shampoo_inverse_root_workspace(94, 1024, 4, mir.RootOpts(method="chebyshev", cheb_degree=16))
    ps = mir.shampoo_inverse_root_workspace(94, 1024, 4, mir.RootOpts(method="chebyshev", cheb_degree=16,
                                                                       cheb_eval="ps"))
    assert head <= 2 * 1024 and cl - 4 * slot <= 2 * 1024 and ps - 8 * slot == cl - 4 * slot
    # up to degree 3 the split saves no product and Clenshaw's plan is used
    for d in (0, 1, 2, 3):
        a = mir.shampoo_inverse_root_workspace(8, 128, 4, mir.RootOpts(method="chebyshev", cheb_degree=d))
        b = mir.shampoo_inverse_root_workspace(8, 128, 4, mir.RootOpts(method="chebyshev", cheb_degree=d,
                                                                         cheb_eval="ps"))
        assert a == b, d
    o = mir.RootOpts(method="chebyshev", cheb_degree=16).c()
    o.cheb_eval = 7
    sz = ctypes.c_size_t(0)
    assert mir.lib.shampoo_inverse_root_workspace(4, 128, 4, ctypes.byref(o), ctypes.byref(sz)) == mir.E_INVALID
    assert b"cheb_eval" in mir.lib.shampoo_last_error()


def test_newton_tolerance_workspace_and_validation(mir):
    """A Newton tolerance adds the check's scratch to the workspace
    (Frobenius partial sums, 32 per matrix for 64 matrices; the norms; a
    flag slot), for half-precision chains too (their checks read the half
    copies); it is rejected for Chebyshev and when negative."""
    a = mir.shampoo_inverse_root_workspace(64, 256, 4, mir.RootOpts(method="cn", iters=20))
    b = mir.shampoo_inverse_root_workspace(64, 256, 4, mir.RootOpts(method="cn", iters=20, tol=1e-6))
    assert b - a == 32 * 64 * 8 + 64 * 8 + 256
    c = mir.shampoo_inverse_root_workspace(64, 256, 4, mir.RootOpts(method="ndb", iters=9, iters2=7))
    d = mir.shampoo_inverse_root_workspace(64, 256, 4, mir.RootOpts(method="ndb", iters=9, iters2=7, tol=1e-6))
    assert d - c == b - a
    e = mir.shampoo_inverse_root_workspace(64, 256, 4, mir.RootOpts(method="cn", iters=20, compute="f16"))
    f = mir.shampoo_inverse_root_workspace(64, 256, 4, mir.RootOpts(method="cn", iters=20, compute="f16", tol=0.1))
    assert f - e == b - a
    for opts, status in [(mir.RootOpts(method="chebyshev", tol=1e-6), mir.E_INVALID),
                         (mir.RootOpts(method="cn", iters=5, tol=-1.0), mir.E_INVALID)]:
        with pytest.raises(mir.ShampooError) as e:
            mir.shampoo_inverse_root_workspace(4, 128, 4, opts)
        assert e.value.status == status, opts


def test_empty_stack_workspace(mir):
    """Workspace queries for a stack of no matrices succeed for every method
    and precision (the Frobenius partial-sum count once divided by the
    batch size)."""
    for kw in (dict(method="cn", iters=10), dict(method="ndb", iters=5, iters2=4),
               dict(method="cn", iters=10, tol=1e-4), dict(method="chebyshev", cheb_degree=8),
               dict(method="cn", iters=10, compute="f16"), dict(method="ndb", iters=5, iters2=4, compute="f64"),
               dict(method="cn", iters=10, residual_bound=1e-4)):
        assert mir.shampoo_inverse_root_workspace(0, 128, 4, mir.RootOpts(**kw)) >= 0
    a = mir.StepArgsC()
    a.nparams, a.B, a.nblk = 0, 128, 0
    a.g_dt, a.p = mir.F32, 4
    a.root = mir.RootOpts(method="cn", iters=10).c()
    assert mir.shampoo_step_workspace(a) >= 0


def test_invalid_calls_fail_before_launch(mir):
    oc = mir.RootOpts(method="cn", iters=5).c()
    # null input
    st = mir.lib.shampoo_inverse_root(None, None, mir.F32, 4, 128, 4, ctypes.byref(oc), None, None, None, None, 0, None)
    assert st == mir.E_INVALID
    # workspace too small (fake non-null device pointers: rejected before use)
    fake = ctypes.c_void_p(0x1000)
    st = mir.lib.shampoo_inverse_root(fake, fake, mir.F32, 4, 128, 4, ctypes.byref(oc), None, None, None, fake, 16, None)
    assert st == mir.E_WORKSPACE
    assert b"workspace" in mir.lib.shampoo_last_error()
    # bad io dtype
    st = mir.lib.shampoo_inverse_root(fake, fake, mir.BF16, 4, 128, 4, ctypes.byref(oc), None, None, None, fake, 1 << 40, None)
    assert st == mir.E_UNSUPPORTED
    # statistics: beta2 out of range, bad dtype
    st = mir.lib.shampoo_update_stats(fake, fake, mir.F32, 2, 128, fake, mir.F32, 1.5, None)
    assert st == mir.E_INVALID
    st = mir.lib.shampoo_update_stats(fake, fake, mir.F16, 2, 128, fake, mir.F32, 0.9, None)
    assert st == mir.E_UNSUPPORTED
    st = mir.lib.shampoo_update_stats(fake, fake, mir.F32, 2, 128, fake, mir.F16, 0.9, None)
    assert st == mir.E_UNSUPPORTED
    # precondition: short workspace (f32 and f64 roots)
    st = mir.lib.shampoo_precondition(fake, mir.F32, fake, mir.F32, 2, 128, fake, fake, 10, None)
    assert st == mir.E_WORKSPACE
    st = mir.lib.shampoo_precondition(fake, mir.F64, fake, mir.F32, 2, 128, fake, fake, 2 * 128 * 128 * 4, None)
    assert st == mir.E_WORKSPACE
    # n == 0 is a no-op
    st = mir.lib.shampoo_inverse_root(None, None, mir.F32, 0, 128, 4, ctypes.byref(oc), None, None, None, None, 0, None)
    assert st == mir.OK


def test_step_workspace_and_validation(mir):
    a = mir.StepArgsC()
    a.nparams, a.B, a.nblk = 1, 128, 2
    a.g_dt, a.p = mir.F32, 4
    a.root = mir.RootOpts(method="cn", iters=10).c()
    b = mir.shampoo_step_workspace(a)
    assert b >= 2 * 2 * 128 * 128 * 4
    a.B = 96
    with pytest.raises(mir.ShampooError):
        mir.shampoo_step_workspace(a)
    # bfloat16 preconditioning: bfloat16 gradients and float32 statistics only
    a.B = 128
    a.precond_dt = mir.BF16
    with pytest.raises(mir.ShampooError) as e:
        mir.shampoo_step_workspace(a)          # float32 gradients
    assert e.value.status == mir.E_UNSUPPORTED
    a.g_dt = mir.BF16
    c = mir.shampoo_step_workspace(a)
    a.precond_dt = mir.F32
    assert c >= mir.shampoo_step_workspace(a)
    a.precond_dt = mir.BF16
    a.stats_dt = mir.F64
    with pytest.raises(mir.ShampooError) as e:
        mir.shampoo_step_workspace(a)
    assert e.value.status == mir.E_UNSUPPORTED
    a.stats_dt, a.precond_dt = mir.F32, 7
    with pytest.raises(mir.ShampooError):
        mir.shampoo_step_workspace(a)


def test_no_cpu_fallback_in_product():
    """The product package has no path that computes on the host."""
    pkg = os.path.join(ROOT, "matrix_inverse_roots_amd")
    for f in os.listdir(pkg):
        if f.endswith(".py"):
            src = open(os.path.join(pkg, f)).read()
            assert "torch.linalg" not in src and "np.linalg" not in src and "scipy" not in src, f


def test_size_limits_are_rejected(mir):
    """Documented limits fail before any launch: more than 65535 matrices in
    one root call (its workspace query too), statistics or preconditioning of
    more than 65535 blocks, power scaling beyond B = 1024 with 16 vectors,
    more than 32767 blocks in a step, and an unknown fallback."""
    oc = mir.RootOpts(method="cn", iters=5).c()
    fake = ctypes.c_void_p(0x1000)
    st = mir.lib.shampoo_inverse_root(fake, fake, mir.F32, 65536, 64, 4, ctypes.byref(oc), None, None, None, fake,
                                      1 << 40, None)
    assert st == mir.E_UNSUPPORTED
    # the workspace query applies the same batch limit (no size that would overflow)
    with pytest.raises(mir.ShampooError) as e:
        mir.shampoo_inverse_root_workspace(1 << 40, 1024, 4, mir.RootOpts(method="cn", iters=5))
    assert e.value.status == mir.E_UNSUPPORTED
    assert mir.shampoo_inverse_root_workspace(65535, 64, 4, mir.RootOpts(method="cn", iters=5)) > 0
    # statistics and preconditioning: the batch limits hold before any size arithmetic
    sz = ctypes.c_size_t(0)
    assert mir.lib.shampoo_precondition_workspace(1 << 40, 1 << 20, mir.F32, ctypes.byref(sz)) == mir.E_UNSUPPORTED
    assert mir.lib.shampoo_update_stats(fake, fake, mir.F32, 1 << 40, 1 << 20, fake, mir.F32, 0.9,
                                        None) == mir.E_UNSUPPORTED
    assert mir.lib.shampoo_precondition(fake, mir.F32, fake, mir.F32, 1 << 40, 1 << 20, fake, fake, 1 << 62,
                                        None) == mir.E_UNSUPPORTED
    with pytest.raises(mir.ShampooError) as e:
        mir.shampoo_inverse_root_workspace(4, 2048, 4, mir.RootOpts(method="cn", iters=5, scaling="power"))
    assert e.value.status == mir.E_UNSUPPORTED
    a = mir.StepArgsC()
    a.nparams, a.B, a.nblk = 1, 128, 40000
    a.g_dt, a.p = mir.F32, 4
    a.root = mir.RootOpts(method="cn", iters=10).c()
    with pytest.raises(mir.ShampooError) as e:
        mir.shampoo_step_workspace(a)
    assert e.value.status == mir.E_UNSUPPORTED
    a.nblk, a.fallback = 2, 7
    with pytest.raises(mir.ShampooError) as e:
        mir.shampoo_step_workspace(a)
    assert e.value.status == mir.E_INVALID


def test_version_string(mir):
    v = mir.version()
    assert "gfx950" in v and v.startswith("shampoo-mi355x")

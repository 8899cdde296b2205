"""Python binding of ``libshampoo.so``: the batched block preconditioner step of
block-diagonal Shampoo on MI355X (gfx950).

Argument marshalling only.  Every step of the path runs in the library's HIP
kernels; torch supplies device memory (``data_ptr``) and the current stream.
The functions keep the C names (``shampoo_inverse_root`` ...).  Importing the
package loads the library and raises ImportError when it is missing: there is
no fallback.
"""

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libshampoo.so")

# ---------------------------------------------------------------------------
# enums (include/shampoo.h)
# ---------------------------------------------------------------------------
OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP, E_NONFINITE = range(6)
STATUS_NAMES = {0: "OK", 1: "E_INVALID", 2: "E_UNSUPPORTED", 3: "E_WORKSPACE", 4: "E_HIP", 5: "E_NONFINITE"}
F32, F16, BF16, F64 = 0, 1, 2, 3
CN, NDB, CHEBYSHEV = 0, 1, 2
SCALE_FROBENIUS, SCALE_POWER = 0, 1
CHEB_CLENSHAW, CHEB_PS = 0, 1
GRAFT_SGD, GRAFT_MOMENTUM, GRAFT_ADAM, GRAFT_NONE = 0, 1, 2, 3
FLAG_NONFINITE, FLAG_ZERO_SCALE, FLAG_PI_FALLBACK, FLAG_RECOMPUTED_F64, FLAG_KEPT_PREVIOUS = 1, 2, 4, 8, 16
FLAG_RESIDUAL = 32
FALLBACKS = {"none": 0, "keep": 1, "f64": 2}

METHODS = {"cn": CN, "ndb": NDB, "chebyshev": CHEBYSHEV}
SCALINGS = {"frobenius": SCALE_FROBENIUS, "power": SCALE_POWER}
CHEB_EVALS = {"clenshaw": CHEB_CLENSHAW, "ps": CHEB_PS}
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16, "f64": F64}
GRAFTS = {"sgd": GRAFT_SGD, "momentum": GRAFT_MOMENTUM, "adam": GRAFT_ADAM, "none": GRAFT_NONE}


class ShampooError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), msg))
        self.status = status


# ---------------------------------------------------------------------------
# ctypes mirrors of the C structs
# ---------------------------------------------------------------------------
class Block(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("param", "brow", "bcol", "row0", "col0", "rows", "cols", "B")]


class Matrix(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld", ctypes.c_int64)]


class Param(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("g", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("ld", ctypes.c_int64), ("first_block", ctypes.c_int64)]


class RootOptsC(ctypes.Structure):
    _fields_ = [("method", ctypes.c_int32), ("scaling", ctypes.c_int32), ("compute", ctypes.c_int32),
                ("iters", ctypes.c_int32), ("iters2", ctypes.c_int32), ("pi_vectors", ctypes.c_int32),
                ("pi_iters", ctypes.c_int32), ("cheb_degree", ctypes.c_int32),
                ("cheb_points", ctypes.c_int32), ("cheb_eval", ctypes.c_int32),
                ("eps", ctypes.c_double), ("cheb_eps", ctypes.c_double),
                ("pi_start_dev", ctypes.c_void_p), ("tol", ctypes.c_double),
                ("residual_out_dev", ctypes.c_void_p), ("residual_bound", ctypes.c_double)]


class StepArgsC(ctypes.Structure):
    _fields_ = [("nparams", ctypes.c_int32), ("B", ctypes.c_int32), ("nblk", ctypes.c_int64),
                ("params_dev", ctypes.c_void_p), ("table_dev", ctypes.c_void_p),
                ("g_dt", ctypes.c_int32), ("p", ctypes.c_int32),
                ("stats_dt", ctypes.c_int32), ("fallback", ctypes.c_int32),
                ("LR", ctypes.c_void_p), ("roots", ctypes.c_void_p),
                ("beta2", ctypes.c_double), ("recompute_roots", ctypes.c_int32),
                ("root", RootOptsC),
                ("graft", ctypes.c_int32), ("graft_blockwise", ctypes.c_int32),
                ("lr", ctypes.c_float), ("momentum", ctypes.c_float),
                ("beta1", ctypes.c_float), ("graft_beta2", ctypes.c_float), ("graft_eps", ctypes.c_float),
                ("t", ctypes.c_int32), ("flags_dev", ctypes.c_void_p), ("dstack", ctypes.c_void_p),
                ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t), ("table_host", ctypes.c_void_p),
                ("precond_dt", ctypes.c_int32)]


EXPORTS = [
    "shampoo_version", "shampoo_last_error", "shampoo_plan_blocks", "shampoo_pack_blocks",
    "shampoo_unpack_blocks", "shampoo_update_stats", "shampoo_inverse_root_workspace",
    "shampoo_inverse_root", "shampoo_inverse_root_noalloc", "shampoo_precondition_workspace",
    "shampoo_precondition",
    "shampoo_step_workspace", "shampoo_step", "shampoo_check_flags", "shampoo_timing_enable",
    "shampoo_timing_read", "shampoo_mfma_peak",
]


def _load():
    # torch is loaded first so that the library binds to torch's HIP runtime:
    # both runtimes carry the soname libamdhip64.so.7, and whichever is loaded
    # first serves the whole process.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError("libshampoo.so is not built (%s); run `python -m matrix_inverse_roots_amd.build` "
                          "or __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "shampoo_version": ([], ctypes.c_char_p),
        "shampoo_last_error": ([], ctypes.c_char_p),
        "shampoo_plan_blocks": ([vp, vp, i32, vp, P(i64)], ctypes.c_int),
        "shampoo_pack_blocks": ([vp, i32, vp, i64, i32, ctypes.c_int, vp, vp, vp], ctypes.c_int),
        "shampoo_unpack_blocks": ([vp, vp, i64, i32, vp, i32, vp], ctypes.c_int),
        "shampoo_update_stats": ([vp, vp, ctypes.c_int, i64, i32, vp, ctypes.c_int, ctypes.c_double, vp],
                                 ctypes.c_int),
        "shampoo_inverse_root_workspace": ([i64, i32, i32, P(RootOptsC), P(sz)], ctypes.c_int),
        "shampoo_inverse_root": ([vp, vp, ctypes.c_int, i64, i32, i32, P(RootOptsC), vp, vp, vp, vp, sz, vp],
                                 ctypes.c_int),
        "shampoo_inverse_root_noalloc": ([vp, vp, ctypes.c_int, i64, i32, i32, P(RootOptsC), vp, vp, vp, vp],
                                         ctypes.c_int),
        "shampoo_precondition_workspace": ([i64, i32, ctypes.c_int, P(sz)], ctypes.c_int),
        "shampoo_precondition": ([vp, ctypes.c_int, vp, ctypes.c_int, i64, i32, vp, vp, sz, vp], ctypes.c_int),
        "shampoo_step_workspace": ([P(StepArgsC), P(sz)], ctypes.c_int),
        "shampoo_step": ([P(StepArgsC), vp], ctypes.c_int),
        "shampoo_check_flags": ([vp, i64, vp], ctypes.c_int),
        "shampoo_timing_enable": ([i32], ctypes.c_int),
        "shampoo_timing_read": ([vp, i32, P(i32)], ctypes.c_int),
        "shampoo_mfma_peak": ([ctypes.c_int, vp, vp, P(ctypes.c_double)], ctypes.c_int),
    }
    for name in EXPORTS:
        f = getattr(lib, name)
        f.argtypes, f.restype = sig[name]
    return lib


lib = _load()


def _check(status):
    if status != OK:
        raise ShampooError(status, lib.shampoo_last_error().decode())


def version():
    return lib.shampoo_version().decode()


# ---------------------------------------------------------------------------
# torch plumbing
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    m = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16, torch.float64: F64}
    if t.dtype not in m:
        raise TypeError("unsupported dtype %s" % t.dtype)
    return m[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, name):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


@dataclass
class RootOpts:
    """Inverse-root options (mirrors shampoo_root_opts)."""
    method: str = "cn"            # "cn" | "ndb" | "chebyshev"
    scaling: str = "frobenius"    # "frobenius" | "power"
    compute: str = "f32"          # "f32" | "f16" | "f64"
    iters: int = 20
    iters2: int = 0
    pi_vectors: int = 16
    pi_iters: int = 10
    cheb_degree: int = 16
    cheb_points: int = 0
    cheb_eval: str = "clenshaw"   # "clenshaw" | "ps" (Paterson-Stockmeyer split)
    eps: float = 0.0
    cheb_eps: Optional[float] = None   # defaults to eps
    pi_start: object = None       # device float32 [pi_vectors, B]
    tol: float = 0.0              # CN / NDB: stop once ||M - I||_F <= tol (0: run iters; f16 checks the half copy)
    residual_out: object = None   # device float32 [n]: ||X^p A_s - I||_F / sqrt(v) per matrix
    residual_bound: float = 0.0   # > 0: FLAG_RESIDUAL where the residual exceeds it

    def c(self):
        return RootOptsC(METHODS[self.method], SCALINGS[self.scaling], DTYPES[self.compute],
                         int(self.iters), int(self.iters2), int(self.pi_vectors), int(self.pi_iters),
                         int(self.cheb_degree), int(self.cheb_points), CHEB_EVALS[self.cheb_eval], float(self.eps),
                         float(self.eps if self.cheb_eps is None else self.cheb_eps),
                         None if self.pi_start is None else self.pi_start.data_ptr(), float(self.tol),
                         None if self.residual_out is None else self.residual_out.data_ptr(),
                         float(self.residual_bound))


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------
def shampoo_plan_blocks(shapes2d, block_sizes):
    """Block table (host int32 numpy [nblk, 8]) for 2-D shapes and block sizes."""
    shapes = np.ascontiguousarray(np.asarray(shapes2d, dtype=np.int64).reshape(-1, 2))
    bs = np.ascontiguousarray(np.asarray(block_sizes, dtype=np.int32).reshape(-1))
    if shapes.shape[0] != bs.shape[0]:
        raise ValueError("one block size per parameter")
    n = ctypes.c_int64(0)
    _check(lib.shampoo_plan_blocks(shapes.ctypes.data, bs.ctypes.data, shapes.shape[0], None, ctypes.byref(n)))
    out = np.zeros((n.value, 8), dtype=np.int32)
    cap = ctypes.c_int64(n.value)
    if n.value:
        _check(lib.shampoo_plan_blocks(shapes.ctypes.data, bs.ctypes.data, shapes.shape[0], out.ctypes.data,
                                       ctypes.byref(cap)))
    return out


def table_to_device(table, device="cuda"):
    torch = _torch()
    return torch.from_numpy(np.ascontiguousarray(table, dtype=np.int32)).to(device)


def matrices_to_device(mats, device="cuda"):
    """Device array of shampoo_matrix for a list of 2-D row-major tensors."""
    torch = _torch()
    rows = []
    for m in mats:
        if m.dim() != 2 or m.stride(1) != 1:
            raise ValueError("matrices must be 2-D with unit column stride")
        rows.append([m.data_ptr(), m.shape[0], m.shape[1], m.stride(0)])
    return torch.tensor(rows, dtype=torch.int64).reshape(-1, 4).to(device)


def shampoo_pack_blocks(mats, table_dev, B, stack, stack_t=None, stream=None):
    """Pack 2-D matrices (list of device tensors of one dtype) into [nblk, B, B]."""
    _dev(stack, "stack")
    _dev(stack_t, "stack_t")
    desc = matrices_to_device(mats, stack.device)
    nblk = table_dev.shape[0]
    _check(lib.shampoo_pack_blocks(_ptr(desc), len(mats), _ptr(table_dev), nblk, int(B), _dtype_code(stack),
                                   _ptr(stack), _ptr(stack_t), _stream(stream)))
    return desc


def shampoo_unpack_blocks(stack, table_dev, B, outs, stream=None):
    _dev(stack, "stack")
    desc = matrices_to_device(outs, stack.device)
    _check(lib.shampoo_unpack_blocks(_ptr(stack), _ptr(table_dev), table_dev.shape[0], int(B), _ptr(desc),
                                     len(outs), _stream(stream)))
    return desc


def shampoo_update_stats(gstack, gstack_t, LR, beta2, stream=None):
    """L, R (the two halves of LR, float32 or float64) updated from a block
    stack and its transpose."""
    for t, n in ((gstack, "gstack"), (gstack_t, "gstack_t"), (LR, "LR")):
        _dev(t, n)
    nblk, B = gstack.shape[0], gstack.shape[1]
    _check(lib.shampoo_update_stats(_ptr(gstack), _ptr(gstack_t), _dtype_code(gstack), nblk, B, _ptr(LR),
                                    _dtype_code(LR), float(beta2), _stream(stream)))


def shampoo_inverse_root_workspace(n, B, p, opts):
    b = ctypes.c_size_t(0)
    oc = opts.c()
    _check(lib.shampoo_inverse_root_workspace(int(n), int(B), int(p), ctypes.byref(oc), ctypes.byref(b)))
    return b.value


def shampoo_inverse_root(inp, out, p, opts, valid=None, scale_out=None, flags=None, ws=None, stream=None):
    """out = (inp + eps I)^(-1/p) for a stack inp [n, B, B] (float32 or float64)."""
    torch = _torch()
    for t, nm in ((inp, "inp"), (out, "out"), (valid, "valid"), (scale_out, "scale_out"), (flags, "flags")):
        _dev(t, nm)
    n, B = inp.shape[0], inp.shape[1]
    if out.dtype != inp.dtype or out.shape != inp.shape:
        raise ValueError("out must match inp")
    if ws is None:
        nb = shampoo_inverse_root_workspace(n, B, p, opts)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=inp.device)
    oc = opts.c()
    _check(lib.shampoo_inverse_root(_ptr(inp), _ptr(out), _dtype_code(inp), n, B, int(p), ctypes.byref(oc),
                                    _ptr(valid), _ptr(scale_out), _ptr(flags), _ptr(ws), ws.numel(),
                                    _stream(stream)))
    return out


def shampoo_inverse_root_noalloc(inp, out, p, opts, valid=None, scale_out=None, flags=None, stream=None):
    """shampoo_inverse_root with the library's own fixed device scratch
    (no workspace, no allocation); calls on one device must not overlap."""
    for t, nm in ((inp, "inp"), (out, "out"), (valid, "valid"), (scale_out, "scale_out"), (flags, "flags")):
        _dev(t, nm)
    n, B = inp.shape[0], inp.shape[1]
    if out.dtype != inp.dtype or out.shape != inp.shape:
        raise ValueError("out must match inp")
    oc = opts.c()
    _check(lib.shampoo_inverse_root_noalloc(_ptr(inp), _ptr(out), _dtype_code(inp), n, B, int(p), ctypes.byref(oc),
                                            _ptr(valid), _ptr(scale_out), _ptr(flags), _stream(stream)))
    return out


def shampoo_precondition(roots, gstack, dstack, ws=None, stream=None):
    """dstack = Lr G Rr per block; roots float32 or float64 [2 nblk, B, B]."""
    torch = _torch()
    for t, nm in ((roots, "roots"), (gstack, "gstack"), (dstack, "dstack")):
        _dev(t, nm)
    nblk, B = gstack.shape[0], gstack.shape[1]
    if ws is None:
        b = ctypes.c_size_t(0)
        _check(lib.shampoo_precondition_workspace(nblk, B, _dtype_code(roots), ctypes.byref(b)))
        ws = torch.empty(max(b.value, 1), dtype=torch.uint8, device=gstack.device)
    _check(lib.shampoo_precondition(_ptr(roots), _dtype_code(roots), _ptr(gstack), _dtype_code(gstack), nblk, B,
                                    _ptr(dstack), _ptr(ws), ws.numel(), _stream(stream)))


def shampoo_step_workspace(args):
    b = ctypes.c_size_t(0)
    _check(lib.shampoo_step_workspace(ctypes.byref(args), ctypes.byref(b)))
    return b.value


def shampoo_step(args, stream=None):
    """One full step over one stack; ``args`` is a StepArgsC (see optimizer.ShampooStack)."""
    _check(lib.shampoo_step(ctypes.byref(args), _stream(stream)))


def shampoo_check_flags(flags, stream=None):
    """Synchronises the stream; True if no matrix is flagged."""
    st = lib.shampoo_check_flags(_ptr(flags), flags.numel(), _stream(stream))
    if st == E_NONFINITE:
        return False
    _check(st)
    return True


def shampoo_timing_enable(capacity):
    _check(lib.shampoo_timing_enable(int(capacity)))


def shampoo_timing_read(capacity):
    """Durations (ms) of the batched-product launches recorded since enabling."""
    buf = (ctypes.c_float * max(int(capacity), 1))()
    n = ctypes.c_int32(0)
    _check(lib.shampoo_timing_read(buf, int(capacity), ctypes.byref(n)))
    return [buf[i] for i in range(n.value)]


def shampoo_mfma_peak(dtype, stream=None):
    """Measured dense matrix-core TFLOP/s for dtype "f32", "f64", "f16" or "bf16"."""
    import torch
    sink = torch.zeros(16, dtype=torch.float32, device="cuda")
    out = ctypes.c_double(0.0)
    _check(lib.shampoo_mfma_peak(DTYPES[dtype], ctypes.c_void_p(sink.data_ptr()), _stream(stream),
                                 ctypes.byref(out)))
    return out.value


from .optimizer import Shampoo, ShampooStack  # noqa: E402  (needs the binding above)

"""Optimizer facade over ``shampoo_step``: plans the blocks, owns the state
tensors and calls the C ABI once per block-size stack.

[3DS] "How to use" / "Hyperparameters": the optimizer is built from a list of
parameters with ``lr``, ``momentum`` and a hyper-parameter set (block size,
grafting type, preconditioning frequency); [DASH] "4. Blocking Strategy":
blocks of every parameter that share a block size are stacked together (one
stack per size over all parameters, the GPU-wide stacking the summary finds
faster than per-layer stacking).
"""

import ctypes
import math

import numpy as np

from . import (RootOpts, StepArgsC, GRAFTS, FALLBACKS, F32, F64, BF16, shampoo_plan_blocks, shampoo_step,
               shampoo_step_workspace, table_to_device, _ptr)


def reshape_2d(shape):
    """2-D view of a parameter shape: keep dim 0, merge the rest."""
    shape = tuple(int(s) for s in shape)
    if len(shape) == 0:
        return (1, 1)
    if len(shape) == 1:
        return (1, shape[0])
    return (shape[0], int(math.prod(shape[1:])))


def _round64(x):
    return (int(x) + 63) // 64 * 64


class ShampooStack:
    """The parameters whose blocks share one stack side B, with their state."""

    def __init__(self, weights, block_sizes, hp, device):
        import torch
        self.torch = torch
        self.hp = hp
        self.weights = weights                      # 2-D float32 views
        shapes = [tuple(w.shape) for w in weights]
        self.table = shampoo_plan_blocks(shapes, block_sizes)
        self.nblk = self.table.shape[0]
        self.B = _round64(max(int(self.table[:, 7].max()), 1)) if self.nblk else 64
        self.table_dev = table_to_device(self.table, device)
        first = {}
        for b in range(self.nblk):
            first.setdefault(int(self.table[b, 0]), b)
        self.first_block = [first.get(i, 0) for i in range(len(weights))]
        sdt = hp["stats_dtype"]
        self.LR = torch.zeros((2 * self.nblk, self.B, self.B), dtype=sdt, device=device)
        self.roots = torch.zeros_like(self.LR)
        self.flags = torch.zeros(2 * self.nblk, dtype=torch.int32, device=device)
        # solver residual of each factor's latest root (NaN until computed)
        self.residuals = (torch.full((2 * self.nblk,), float("nan"), dtype=torch.float32, device=device)
                          if hp["residuals"] else None)
        g = hp["graft"]
        self.m = [torch.zeros_like(w) for w in weights] if g in ("momentum", "adam") else None
        self.v = [torch.zeros_like(w) for w in weights] if g == "adam" else None
        self.grad_dtype = hp["grad_dtype"]
        self.params_dev = None
        self._grad_ptrs = None
        self._desc_cache = {}   # gradient pointers -> device descriptor table
        self.args = StepArgsC()
        a = self.args
        a.nparams = len(weights)
        a.B = self.B
        a.nblk = self.nblk
        a.table_dev = self.table_dev.data_ptr()
        a.g_dt = BF16 if self.grad_dtype == torch.bfloat16 else F32
        a.p = hp["p"]
        a.stats_dt = F64 if sdt == torch.float64 else F32
        a.fallback = FALLBACKS[hp["fallback"]]
        a.LR = self.LR.data_ptr()
        a.roots = self.roots.data_ptr()
        a.beta2 = hp["beta2"]
        ro = hp["root"]
        self.pi_start = None
        if ro.scaling == "power":
            gen = torch.Generator(device=device)
            gen.manual_seed(hp["pi_seed"] + self.B)
            self.pi_start = torch.randn((ro.pi_vectors, self.B), generator=gen, device=device, dtype=torch.float32)
            ro = RootOpts(**{**ro.__dict__, "pi_start": self.pi_start})
        if self.residuals is not None:
            ro = RootOpts(**{**ro.__dict__, "residual_out": self.residuals})
        a.root = ro.c()
        a.graft = GRAFTS[g]
        a.graft_blockwise = 1 if hp["graft_blockwise"] else 0
        a.lr = hp["lr"]
        a.momentum = hp["momentum"]
        a.beta1 = hp["beta1"]
        a.graft_beta2 = hp["graft_beta2"]
        a.graft_eps = hp["graft_eps"]
        a.flags_dev = self.flags.data_ptr()
        a.precond_dt = BF16 if hp["precond_dtype"] == torch.bfloat16 else F32
        a.dstack = None
        # host copy of the table: roots grouped by each factor's own side
        self.table_host = np.ascontiguousarray(self.table, dtype=np.int32)
        a.table_host = self.table_host.ctypes.data if hp["group_factors"] and self.nblk else None
        nb = shampoo_step_workspace(a)
        self.ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=device)
        a.ws = self.ws.data_ptr()
        a.ws_bytes = self.ws.numel()

    def _descriptors(self, grads, stream):
        """Device table of shampoo_param rows for these gradients.  Tables are
        kept per set of gradient pointers (a training loop reuses a few
        gradient buffers), so a step normally uploads nothing; a new set is
        copied from pinned memory on ``stream``, without blocking the host."""
        torch = self.torch
        ptrs = tuple(g.data_ptr() for g in grads)
        if ptrs == self._grad_ptrs:
            return
        dev = self._desc_cache.get(ptrs)
        if dev is None:
            rows = []
            for i, (w, g) in enumerate(zip(self.weights, grads)):
                rows.append([w.data_ptr(), g.data_ptr(),
                             self.m[i].data_ptr() if self.m is not None else 0,
                             self.v[i].data_ptr() if self.v is not None else 0,
                             w.shape[0], w.shape[1], w.stride(0), self.first_block[i]])
            host = torch.tensor(rows, dtype=torch.int64).reshape(-1, 8).pin_memory()
            dev = torch.empty(host.shape, dtype=torch.int64, device=self.LR.device)
            with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream(self.LR.device)):
                dev.copy_(host, non_blocking=True)
            if len(self._desc_cache) >= 8:
                self._desc_cache.pop(next(iter(self._desc_cache)))
            self._desc_cache[ptrs] = dev
        self.params_dev = dev
        self.args.params_dev = dev.data_ptr()
        self._grad_ptrs = ptrs

    def prepare(self, grads, t, recompute, dstack=None, stream=None):
        """Checks the gradients and sets the step's arguments; a descriptor
        table not seen before is copied to the device on ``stream`` (default:
        the current stream), ahead of the work enqueued there afterwards."""
        for g, w in zip(grads, self.weights):
            if g.dtype != self.grad_dtype or tuple(g.shape) != tuple(w.shape) or not g.is_contiguous():
                raise ValueError("gradient must be a contiguous %s tensor of shape %s" % (self.grad_dtype, tuple(w.shape)))
        self._descriptors(grads, stream)
        self.args.t = int(t)
        self.args.recompute_roots = 1 if recompute else 0
        self.args.dstack = None if dstack is None else dstack.data_ptr()

    def launch(self, stream=None):
        shampoo_step(self.args, stream)

    def step(self, grads, t, recompute, dstack=None, stream=None):
        self.prepare(grads, t, recompute, dstack, stream)
        self.launch(stream)


class Shampoo:
    """Block-diagonal Shampoo over a list of float32 device parameters.

    block_size: int, or a callable (rows, cols) -> block size (0 = whole
    parameter as one block).  graft: "sgd" | "momentum" | "adam" | "none".
    precondition_frequency: roots recomputed every that many steps (the
    statistics are updated every step).  stats_dtype: torch.float32 (the
    pages' float32 statistics) or torch.float64 (statistics, roots and
    preconditioning products in float64).  fallback: "none" | "keep" |
    "f64", what a step does with a factor whose new root is not finite (flag
    it; keep its previous root; recompute it with the float64 chain).
    group_factors: root each factor in a stack of its own side (rounded up
    to 64) rather than the block size, grouped by side.
    concurrent_stacks: with more than one stack (parameters of different
    block sizes), step each stack on its own side stream (default priority),
    forked from and joined back to the calling stream with events, so that
    one stack's launches fill the gaps and partly idle rounds of another's.
    Power-iteration scaling draws its start vectors once per stack from
    ``pi_seed``.  residuals: keep each factor's solver residual
    ||X^p A_s - I||_F / sqrt(v) of its latest root (``residuals()``); with
    ``root.residual_bound`` > 0 a root above the bound is flagged RESIDUAL
    and handled by ``fallback`` like a non-finite one.
    precondition_dtype: None (the products of D = L^{-1/4} G R^{-1/4} in the
    roots' precision) or torch.bfloat16 (bfloat16 operands, float32
    accumulation and D; bfloat16 gradients and float32 statistics only).
    """

    def __init__(self, params, block_size=1024, beta2=1.0, eps=1e-12, p=4, root=None, graft="sgd",
                 lr=0.1, momentum=0.9, beta1=0.9, graft_beta2=0.999, graft_eps=1e-8,
                 graft_blockwise=False, precondition_frequency=1, grad_dtype=None, stats_dtype=None,
                 pi_seed=0, fallback="none", group_factors=True, concurrent_stacks=True, residuals=False,
                 precondition_dtype=None):
        import torch
        params = list(params)
        if not params:
            raise ValueError("no parameters")
        for w in params:
            if w.dtype != torch.float32 or not w.is_cuda or not w.is_contiguous():
                raise ValueError("parameters must be contiguous float32 device tensors")
        self.params = params
        self.views = [w.view(reshape_2d(w.shape)) for w in params]
        root = root if root is not None else RootOpts(method="cn", iters=20, eps=eps)
        if root.eps != eps:
            root = RootOpts(**{**root.__dict__, "eps": eps})
        self.hp = dict(beta2=float(beta2), p=int(p), root=root, graft=graft, lr=float(lr),
                       momentum=float(momentum), beta1=float(beta1), graft_beta2=float(graft_beta2),
                       graft_eps=float(graft_eps), graft_blockwise=bool(graft_blockwise),
                       grad_dtype=grad_dtype if grad_dtype is not None else torch.float32,
                       stats_dtype=stats_dtype if stats_dtype is not None else torch.float32,
                       pi_seed=int(pi_seed), fallback=str(fallback), group_factors=bool(group_factors),
                       residuals=bool(residuals), precond_dtype=precondition_dtype)
        if precondition_dtype not in (None, torch.float32, torch.bfloat16):
            raise ValueError("precondition_dtype must be None, torch.float32 or torch.bfloat16")
        if fallback not in FALLBACKS:
            raise ValueError("fallback must be one of %s" % sorted(FALLBACKS))
        bs_of = block_size if callable(block_size) else (lambda m, n, b=int(block_size): b)
        groups = {}
        for i, v in enumerate(self.views):
            m, n = v.shape
            b = int(bs_of(m, n))
            plan_b = max(m, n) if (b == 0 or b >= max(m, n)) else b
            groups.setdefault(_round64(plan_b), []).append((i, plan_b))
        self.stacks = []
        self.members = []
        for side in sorted(groups):
            idx = [i for i, _ in groups[side]]
            st = ShampooStack([self.views[i] for i in idx], [b for _, b in groups[side]], self.hp,
                              params[0].device)
            self.stacks.append(st)
            self.members.append(idx)
        self.frequency = int(precondition_frequency)
        self.t = 0
        self.device = params[0].device
        nside = min(len(self.stacks), 4) if concurrent_stacks and len(self.stacks) > 1 else 0
        self._side = [torch.cuda.Stream(device=self.device) for _ in range(nside)]
        # concurrent stacks are enqueued heaviest first (block work ~ nblk B^3),
        # so that the longest chain starts while the host enqueues the rest
        self._order = sorted(range(len(self.stacks)), key=lambda k: -self.stacks[k].nblk * self.stacks[k].B ** 3)

    def step(self, grads, stream=None):
        """One step with gradients given per parameter (same order as params)."""
        self.t += 1
        recompute = (self.t - 1) % self.frequency == 0
        views = [g.reshape(v.shape) for g, v in zip(grads, self.views)]
        if not self._side:
            for st, idx in zip(self.stacks, self.members):
                st.step([views[i] for i in idx], self.t, recompute, stream=stream)
            return
        torch = self.stacks[0].torch
        cur = stream if stream is not None else torch.cuda.current_stream(self.device)
        for st, idx in zip(self.stacks, self.members):
            st.prepare([views[i] for i in idx], self.t, recompute, stream=cur)
        fork = torch.cuda.Event()
        fork.record(cur)
        joins = []
        for j, k in enumerate(self._order):
            st = self.stacks[k]
            side = self._side[j % len(self._side)]
            side.wait_event(fork)
            st.launch(side)
            done = torch.cuda.Event()
            done.record(side)
            joins.append(done)
        for done in joins:
            cur.wait_event(done)

    def capture(self, grads):
        """Record one step on the gradient buffers ``grads`` into a graph and
        return a function that replays it (and advances the step count).
        Refill the buffers in place before each replay.  The graph replays
        the launches of an eager step with the same arguments, so it needs a
        step whose kernels do not change with the step count: SGD, momentum
        or no grafting (Adam's bias correction depends on it), roots every
        step, fallback "none" or "keep" (the float64 fallback counts the
        failed factors on the host) and no Newton tolerance (its checks read
        a flag on the host).  Take at least one eager step first, so
        that one-time set-up (kernel attributes, descriptor tables of these
        buffers) happens outside the capture."""
        torch = self.stacks[0].torch
        if self.hp["graft"] == "adam":
            raise ValueError("capture: Adam grafting depends on the step count")
        if self.frequency != 1:
            raise ValueError("capture: roots must be recomputed every step")
        if self.hp["fallback"] == "f64":
            raise ValueError("capture: the float64 fallback synchronises with the host")
        if self.hp["root"].tol > 0:
            raise ValueError("capture: a coupled-Newton tolerance synchronises with the host")
        if self.t < 1:
            raise ValueError("capture: take one eager step first")
        views = [g.reshape(v.shape) for g, v in zip(grads, self.views)]
        # descriptor tables of these buffers, uploaded before the capture
        cur = torch.cuda.current_stream(self.device)
        for st, idx in zip(self.stacks, self.members):
            st.prepare([views[i] for i in idx], self.t + 1, True, stream=cur)
        torch.cuda.synchronize(self.device)
        # the graph reads these descriptor tables: the replay function owns
        # them, so that later eager steps cannot evict and free them
        tables = [st.params_dev for st in self.stacks]
        graph = torch.cuda.CUDAGraph()
        t_saved = self.t
        with torch.cuda.graph(graph):
            self.step(grads)
        self.t = t_saved

        def replay():
            self.t += 1
            graph.replay()

        replay.graph = graph
        replay.tables = tables
        return replay

    def flags(self):
        return [st.flags for st in self.stacks]

    def residuals(self):
        """Per stack: the solver residual of each factor's latest root (L
        factors, then R factors), or None without ``residuals=True``."""
        return [st.residuals for st in self.stacks]

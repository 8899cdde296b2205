#!/usr/bin/env python
"""Benchmark of the batched block preconditioner step on one MI355X.

Headline: inverse 4th roots of a stack of 1024 SPD blocks 512 x 512 with
eigenvalues log-uniform in [1e-8, 1] (Q diag(lambda) Q^T, Haar Q), by
Newton-DB (28 + 17 iterations) after half-precision multi-start power
iteration scaling (16 vectors, 10 products), with the float64 chain: at
condition number 1e8 it is the arithmetic that meets the stated 1e-4 (float32
cannot resolve the spectrum and its roots diverge).  A step is one
shampoo_inverse_root call over the whole stack (1024 blocks), input resident
in HBM.  value = blocks/s.

Also reported, each with the bar it is held to:
* the float32 and half-product solves of the same stack (diagnostics: their
  non-finite counts);
* 64 SPD blocks 128 x 128 (lambda in [1e-6, 1]), coupled Newton 20 with
  Frobenius scaling, float64 (and float32 as a diagnostic);
* the full optimizer step (pack, statistics, roots, preconditioning,
  grafting, update) on the single 256 x 128 parameter, the 12-layer decoder
  set and the 50-layer bottleneck set, on the paths that meet 1e-4 (float64,
  or a float32 chain whose solver residual is checked on the device with
  the float64 recomputation as fallback) and on the pages' float32 and
  half-product configurations;
* the roofline of the dominant kernel (the float64 batched product) from
  HIP events around its launches, and the CPU oracle timed on a bounded
  sample, which also gives the parity of every block it computes.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_MFMA = 157.3  # TFLOP/s, MI355X dense
PEAK_FP16_MFMA = 2516.6
PEAK_FP64_MFMA = 78.6
PEAK_HBM = 8000.0       # GB/s

N_BLOCKS, B = 1024, 512
ITERS1, ITERS2 = 28, 17
PI_VECTORS, PI_ITERS = 16, 10
METRIC = "inverse-root blocks/sec at B=512 (+% MFMA peak); full optimizer step ms"
RESIDUAL_BOUND = 1e-4   # solver residual above which a float32 root is recomputed in float64
# coupled-Newton tolerance for half-product chains on 1024^2 factors: the
# half copy of M settles near ||M - I||_F = 2.6e-2 there, so 0.1 is reached
# once the iteration has converged to half precision
HALF_TOL = 0.1
DECODER = "decoder_12x(1024x3072,1024x1024,1024x4096,4096x1024)_bf16_adam_b1024"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_count_ndb(k1, k2):
    """Batched products the Newton-DB chain launches for p = 4 (k1, k2 >= 2)."""
    return (3 * k1 - 3) + (3 * k2 - 3)


def make_stack(n=None):
    import synthetic
    t = time.time()
    A = synthetic.spd_stack(3, N_BLOCKS if n is None else n, B, 1e-8, 1.0)
    log(f"generated the SPD stack in {time.time() - t:.1f} s")
    return A


def time_roots(mir, inp, opts, steps, warmup, timing_cap=0, p=4):
    """Median-free plain timing of `steps` calls after `warmup`; with
    timing_cap > 0 also the HIP-event durations of the batched products."""
    import torch
    out = torch.empty_like(inp)
    n, b = inp.shape[0], inp.shape[1]
    flags = torch.zeros(n, dtype=torch.int32, device=inp.device)
    nb = mir.shampoo_inverse_root_workspace(n, b, p, opts)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=inp.device)
    for _ in range(warmup):
        mir.shampoo_inverse_root(inp, out, p, opts, flags=flags, ws=ws)
    torch.cuda.synchronize()
    if timing_cap:
        mir.shampoo_timing_enable(timing_cap)
    flags.zero_()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        mir.shampoo_inverse_root(inp, out, p, opts, flags=flags, ws=ws)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    gemm_ms = []
    if timing_cap:
        gemm_ms = mir.shampoo_timing_read(timing_cap)
        mir.shampoo_timing_enable(0)
    nflag = int((flags != 0).sum().item())
    nonfinite = int(((flags & mir.FLAG_NONFINITE) != 0).sum().item())
    del ws
    return dt, gemm_ms, nflag, nonfinite, out


def device_residuals(mir, inp, opts, p=4):
    """One more call with the device residual ||X^p A_s - I||_F / sqrt(B) of
    every matrix (not timed): numpy float64 [n]."""
    import numpy as np
    import torch
    res = torch.full((inp.shape[0],), float("nan"), dtype=torch.float32, device=inp.device)
    o = mir.RootOpts(**{**opts.__dict__, "residual_out": res})
    out = torch.empty_like(inp)
    mir.shampoo_inverse_root(inp, out, p, o)
    torch.cuda.synchronize()
    del out
    return res.cpu().numpy().astype(np.float64)


def residual_summary(r):
    import numpy as np
    fin = np.isfinite(r)
    return {"finite": int(fin.sum()), "max": float(r[fin].max()) if fin.any() else None,
            "median": float(np.median(r[fin])) if fin.any() else None}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(A64, X64, budget_s=15.0):
    """The oracle (float64 eigh inverse 4th root) timed on the host on the
    first blocks of the same stack for about budget_s, with a one-thread
    rate.  The roots it computed then give the parity of the GPU's float64
    roots of those blocks (relative Frobenius error), beside the oracle's own
    residual on a few of them."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        cores = max(i.get("num_threads", 1) for i in info) if info else 1
    except Exception:
        threadpoolctl = None
        cores = os.cpu_count()
    roots = []
    t0 = time.perf_counter()
    for i in range(A64.shape[0]):
        roots.append(oracle.inverse_root_eigh(A64[i], 4))
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    done = len(roots)
    one = None
    if threadpoolctl is not None:
        with threadpoolctl.threadpool_limits(1):
            t1 = time.perf_counter()
            k = 0
            while k < A64.shape[0] and (k == 0 or time.perf_counter() - t1 < budget_s / 3):
                oracle.inverse_root_eigh(A64[k], 4)
                k += 1
            one = k / (time.perf_counter() - t1)
    base = {"value": done / dt, "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
            "sample": f"the first {done} of the {N_BLOCKS} blocks (512 x 512, float64), float64 eigh inverse 4th "
                      f"root each",
            "value_1thread": one, "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}
    errs = np.array([np.linalg.norm(X64[i] - roots[i]) / np.linalg.norm(roots[i]) for i in range(done)])
    par = {"blocks_checked": done, "f64_rel_err_max": float(errs.max()), "f64_rel_err_median": float(np.median(errs)),
           "bar": 1e-4, "oracle_residual_blocks_0_1_2": [oracle.residual(roots[i], A64[i], 4) for i in range(min(3, done))]}
    return base, par


def oracle_full_steps():
    """The oracle's full step (statistics, float64 eigh or exact-polynomial
    roots, direction, grafting) on the host, for the two step workloads:
    one whole bottleneck-50 step, and one of the 12 identical decoder layers
    scaled by 12 (the layers are independent and equal in shape)."""
    import numpy as np
    import oracle
    import synthetic
    res = {}
    shapes = synthetic.bottleneck50_shapes()
    bsz = synthetic.bottleneck50_block_sizes(shapes)
    g = synthetic.gaussian_grads(5, shapes, 1, 0.1)[0]
    orc = oracle.ShampooOracle(shapes, bsz, beta2=0.999, eps=1e-12, root="chebyshev", cheb_degree=16,
                               graft="momentum", lr=0.1, momentum=0.9)
    W = [np.zeros(sh) for sh in shapes]
    t0 = time.perf_counter()
    orc.step(W, [x.astype(np.float64) for x in g])
    res["bottleneck50_step_ms"] = round((time.perf_counter() - t0) * 1e3, 1)
    res["bottleneck50_sample"] = "one whole step, 53 matrices, Chebyshev degree 16 as the exact polynomial"
    layer = synthetic.decoder_shapes(layers=1)
    g = synthetic.gaussian_grads(4, layer, 1, 0.02)[0]
    orc = oracle.ShampooOracle(layer, [1024] * len(layer), beta2=0.999, eps=1e-12, root="eigh", graft="adam",
                               lr=1e-3)
    W = [np.zeros(sh) for sh in layer]
    t0 = time.perf_counter()
    orc.step(W, [x.astype(np.float64) for x in g])
    res["decoder12_step_ms"] = round((time.perf_counter() - t0) * 1e3 * 12, 1)
    res["decoder12_sample"] = "one decoder layer (24 factors of 1024^2, eigh roots) timed, times 12"
    return res


def oracle_decoder_parity(mir):
    """Parity of the decoder set's two fastest timed step forms against the
    oracle: 3 steps on the whole set (bfloat16 gradients N(0, 0.02^2), seed
    4), the oracle run on the first 4 parameters (one layer); the largest
    relative Frobenius error of those parameters over the 3 steps."""
    import numpy as np
    import torch
    import oracle
    import synthetic
    shapes = synthetic.decoder_shapes()
    grads = synthetic.gaussian_grads(4, shapes, 3, 0.02, dtype="bf16")
    sample = [0, 1, 2, 3]
    forms = {
        "cn_f16_products_tol0.1_power_scaling_bf16_precondition":
            (dict(compute="f16", tol=HALF_TOL, scaling="power"), dict(fallback="f64", precondition_dtype=torch.bfloat16),
             2e-2),
        "f32_chain_tol1e-4_power_scaling_residual_checked":
            (dict(compute="f32", tol=1e-4, scaling="power", residual_bound=RESIDUAL_BOUND),
             dict(fallback="f64", stats_dtype=torch.float64), 1e-4),
    }
    res = {}
    for name, (root_kw, kw, bar) in forms.items():
        W = [torch.zeros(sh, dtype=torch.float32, device="cuda") for sh in shapes]
        opt = mir.Shampoo(W, block_size=1024, beta2=0.999, eps=1e-12, root=mir.RootOpts(method="cn", iters=34, **root_kw),
                          graft="adam", lr=1e-3, grad_dtype=torch.bfloat16, **kw)
        orc = oracle.ShampooOracle([shapes[i] for i in sample], [1024] * len(sample), beta2=0.999, eps=1e-12,
                                   graft="adam", lr=1e-3)
        Wo = [np.zeros(shapes[i]) for i in sample]
        worst = 0.0
        for t in range(3):
            bits = [torch.from_numpy(np.ascontiguousarray(g).view(np.int16)).view(torch.bfloat16).cuda()
                    for g in grads[t]]
            opt.step(bits)
            orc.step(Wo, [synthetic.bf16_bits_to_f32(grads[t][i]).astype(np.float64) for i in sample])
            torch.cuda.synchronize()
            for k, i in enumerate(sample):
                w = W[i].cpu().numpy().astype(np.float64)
                worst = max(worst, float(np.linalg.norm(w - Wo[k]) / np.linalg.norm(Wo[k])))
        res[name] = {"rel_err_max": worst, "bar": bar, "parameters_checked": len(sample), "steps": 3}
        del opt, W
    return res


def oracle_spd128(X64_dev):
    """Parity of the float64 coupled-Newton roots of the 64 x 128^2 stack
    against the oracle (all 64 blocks)."""
    import numpy as np
    import oracle
    import synthetic
    A = synthetic.spd_stack(2, 64, 128, 1e-6, 1.0)
    X = X64_dev.cpu().numpy()
    errs = [np.linalg.norm(X[i] - oracle.inverse_root_eigh(A[i], 4)) / np.linalg.norm(oracle.inverse_root_eigh(A[i], 4))
            for i in range(64)]
    return {"blocks_checked": 64, "f64_rel_err_max": float(max(errs)), "bar": 1e-4}


def traffic_from_profiles(kernel_tag):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current source of the kernel (else None)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for name in rec.get("kernel_sources", []):
        with open(os.path.join(ROOT, "matrix_inverse_roots_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if not rec.get("kernel_sources") or rec.get("kernel_sources_sha256") != h.hexdigest():
        return None
    return rec.get("bytes_per_launch")


def spd128_solve(mir, compute, calls=50):
    """64 SPD blocks 128 x 128, lambda log-uniform in [1e-6, 1] (seed 2),
    coupled Newton 20 with Frobenius scaling: ms per call (median of `calls`
    event-timed calls), blocks/s, and the mean product duration and rate."""
    import numpy as np
    import torch
    import synthetic
    A = synthetic.spd_stack(2, 64, 128, 1e-6, 1.0)
    inp = torch.from_numpy(A if compute == "f64" else A.astype(np.float32)).cuda()
    opts = mir.RootOpts(method="cn", iters=20, compute=compute)
    out = torch.empty_like(inp)
    ws = torch.empty(mir.shampoo_inverse_root_workspace(64, 128, 4, opts), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        mir.shampoo_inverse_root(inp, out, 4, opts, ws=ws)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(calls)]
    for a, b in ev:
        a.record()
        mir.shampoo_inverse_root(inp, out, 4, opts, ws=ws)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    # the same call captured once as a graph and replayed: the chain's 80
    # launches without the host's per-launch cost
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mir.shampoo_inverse_root(inp, out, 4, opts, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mir.shampoo_inverse_root(inp, out, 4, opts, ws=ws)
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        graph.replay()
        b.record()
    torch.cuda.synchronize()
    ms_graph = float(np.median([a.elapsed_time(b) for a, b in ev]))
    mir.shampoo_timing_enable(1024)
    mir.shampoo_inverse_root(inp, out, 4, opts, ws=ws)
    torch.cuda.synchronize()
    g = mir.shampoo_timing_read(1024)
    mir.shampoo_timing_enable(0)
    flop = 64 * 2.0 * 128 ** 3
    mg = float(np.mean(g)) * 1e-3
    peak = PEAK_FP64_MFMA if compute == "f64" else PEAK_FP32_MFMA
    rec = {"ms_per_call": round(ms, 4), "blocks_per_s": round(64 / ms * 1e3, 1),
           "ms_per_graph_replay": round(ms_graph, 4), "blocks_per_s_graph_replay": round(64 / ms_graph * 1e3, 1),
           "products": len(g),
           "product_mean_us": round(mg * 1e6, 2), "product_tflops": round(flop / mg / 1e12, 2),
           "product_frac": round(flop / mg / 1e12 / peak, 4),
           "call_tflops": round(len(g) * flop / (ms * 1e-3) / 1e12, 2)}
    return rec, out


def step_timer(steps, warmup):
    import numpy as np
    import torch

    def timed(fn, before_timed=None):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        if before_timed is not None:
            before_timed()
            torch.cuda.synchronize()
        times = []
        for i in range(warmup, warmup + steps):
            t0 = time.perf_counter()
            fn(i)
            torch.cuda.synchronize()
            times.append((time.perf_counter() - t0) * 1e3)
        return float(np.median(times))

    return timed


def flagged(opt):
    return sum(int((f != 0).sum().item()) for f in opt.flags())


def decoder_step_ms(mir, steps, warmup, compute="f32", stats64=False, fallback="none", tol=0.0, bound=0.0,
                    scaling="frobenius", precond_bf16=False):
    """Full step on the 12-layer decoder set (151 M parameters, block 1024,
    bfloat16 gradients N(0, 0.02^2), beta2 0.999, eps 1e-12, Adam grafting,
    coupled Newton 34 iterations (or stopping at ||M - I||_F <= tol) after
    Frobenius (or power-iteration) scaling, roots every step).  Returns the median step time and the number of factors
    flagged during the timed steps."""
    import torch
    import synthetic
    shapes = synthetic.decoder_shapes()
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=1024, beta2=0.999, eps=1e-12,
                      root=mir.RootOpts(method="cn", iters=34, compute=compute, tol=tol, residual_bound=bound,
                                        scaling=scaling),
                      graft="adam", lr=1e-3, grad_dtype=torch.bfloat16, fallback=fallback,
                      stats_dtype=torch.float64 if stats64 else torch.float32,
                      precondition_dtype=torch.bfloat16 if precond_bf16 else None)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    grads = [[(torch.randn(s, generator=gen, device="cuda") * 0.02).to(torch.bfloat16) for s in shapes]
             for _ in range(2)]
    def zero_flags():
        for f in opt.flags():
            f.zero_()

    ms = step_timer(steps, warmup)(lambda i: opt.step(grads[i % 2]), zero_flags)
    return ms, flagged(opt)


def single_step_ms(mir, steps, warmup, compute="f32", stats64=False, fallback="none", bound=0.0, graph=False):
    """Step on one [256, 128] float32 parameter in two 128-blocks (gradients
    N(0, 1), statistics summed (beta2 1), eps 1e-12, coupled Newton 30, SGD
    grafting lr 0.1): a launch-bound step, timed eagerly and (graph=True) as
    a graph replay.  Returns (eager ms, replay ms or None, flagged)."""
    import torch
    W = [torch.zeros((256, 128), dtype=torch.float32, device="cuda")]
    opt = mir.Shampoo(W, block_size=128, beta2=1.0, eps=1e-12,
                      root=mir.RootOpts(method="cn", iters=30, compute=compute, residual_bound=bound),
                      graft="sgd", lr=0.1, stats_dtype=torch.float64 if stats64 else torch.float32,
                      fallback=fallback)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    grads = [[torch.randn((256, 128), generator=gen, device="cuda")] for _ in range(2)]
    static = [torch.empty((256, 128), device="cuda")]
    timed = step_timer(steps, warmup)

    def zero_flags():
        for f in opt.flags():
            f.zero_()

    eager = timed(lambda i: opt.step(grads[i % 2]), zero_flags)
    nf = flagged(opt)
    rep = None
    if graph:
        static[0].copy_(grads[0][0])
        opt.step(static)
        replay = opt.capture(static)
        rep = timed(lambda i: replay())
    return eager, rep, nf


def chebyshev_sweep(mir, degrees=(16, 40, 60, 100)):
    """Chebyshev inverse 4th roots of 288 SPD matrices 1024 x 1024 (the
    decoder set's factor stack; A = X X^T / 1024 + 1e-3 I with X N(0, 1) drawn
    on the device), Frobenius scaling, for the degree sweep: float32 and
    half-precision products, Clenshaw's recurrence and the Paterson-Stockmeyer
    split.  Returns {(degree, compute, eval): (ms per call, products)}."""
    import torch
    n, b = 288, 1024
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    A = torch.empty((n, b, b), device="cuda")
    for i in range(0, n, 32):
        X = torch.randn((32, b, b), generator=gen, device="cuda")
        A[i:i + 32] = torch.bmm(X, X.transpose(1, 2).contiguous()) / b
    A += 1e-3 * torch.eye(b, device="cuda")
    out = torch.empty_like(A)
    res = {}
    for d in degrees:
        for compute in ("f32", "f16"):
            for ev in ("clenshaw", "ps"):
                opts = mir.RootOpts(method="chebyshev", cheb_degree=d, cheb_eval=ev, compute=compute, eps=1e-3)
                ws = torch.empty(mir.shampoo_inverse_root_workspace(n, b, 4, opts), dtype=torch.uint8, device="cuda")
                mir.shampoo_inverse_root(A, out, 4, opts, ws=ws)
                torch.cuda.synchronize()
                mir.shampoo_timing_enable(512)
                t0 = time.perf_counter()
                for _ in range(2):
                    mir.shampoo_inverse_root(A, out, 4, opts, ws=ws)
                torch.cuda.synchronize()
                ms = (time.perf_counter() - t0) / 2 * 1e3
                prods = len(mir.shampoo_timing_read(512)) // 2
                mir.shampoo_timing_enable(0)
                res[(d, compute, ev)] = (ms, prods)
                log(f"chebyshev d={d} {compute} {ev}: {ms:.1f} ms per call, {prods} products")
                del ws
    return res


def bottleneck_root_gflop(mir, products):
    """Root work per step of the bottleneck-50 set, counted as full products
    (2 v^3 flop each): on the factors' valid sides, on their grouped sides
    (valid side rounded up to 64) and padded to the block size."""
    import numpy as np
    import synthetic
    shapes = [(s[0], int(np.prod(s[1:]))) for s in synthetic.bottleneck50_shapes()]
    bs = [1024 if max(m, n) >= 2048 else 256 for m, n in shapes]
    table = mir.shampoo_plan_blocks(shapes, bs)
    v = np.concatenate([table[:, 5], table[:, 6]]).astype(np.float64)
    blk = np.concatenate([table[:, 7], table[:, 7]]).astype(np.float64)
    side = np.ceil(v / 64) * 64
    f = lambda x: round(float(2.0 * products * np.sum(x ** 3)) / 1e9, 1)
    return {"valid_region": f(v), "grouped_sides": f(side), "padded_to_block": f(blk)}


def bottleneck_step_ms(mir, steps, warmup, group, cheb_eval="clenshaw", compute="f32"):
    """Full step on the bottleneck-50 set (53 matrices, 25.5 M parameters,
    block 1024 if max(m, n) >= 2048 else 256, float32 gradients N(0, 1e-2),
    beta2 0.999, eps 1e-12, Chebyshev degree 16 summed by Clenshaw's
    recurrence or by the Paterson-Stockmeyer split, float32 or half-precision
    products, momentum grafting), with the roots grouped by factor side or
    computed at the block size."""
    import torch
    import synthetic
    shapes = synthetic.bottleneck50_shapes()
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=lambda m, n: 1024 if max(m, n) >= 2048 else 256, beta2=0.999, eps=1e-12,
                      root=mir.RootOpts(method="chebyshev", cheb_degree=16, cheb_eval=cheb_eval, compute=compute),
                      graft="momentum",
                      lr=0.1, momentum=0.9, group_factors=group)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    grads = [[torch.randn(s, generator=gen, device="cuda") * 0.1 for s in shapes] for _ in range(2)]
    ms = step_timer(steps, warmup)(lambda i: opt.step(grads[i % 2]))
    return ms, flagged(opt)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-full-step", action="store_true")
    ap.add_argument("--blocks", type=int, default=None,
                    help="with --only roots*: solve only the first this-many blocks (counter runs whose "
                         "per-dispatch counts would otherwise overflow 32 bits)")
    ap.add_argument("--only", choices=["roots", "roots_f32", "roots_f16", "copy", "spd128", "step", "step_f16",
                                       "step_f16_tol", "step_f16_tol_pi", "step_f16_tol_pi_pbf16", "step_tol_res_pi", "step_tol", "step_res", "step_tol_res", "step_f64", "step5", "step5_ps",
                                       "step1", "step1_f64", "cheb_sweep"],
                    default=None,
                    help="profiling runs: only the float64 solve (roots) or its float32 / half-product "
                         "variants, only a 1 GiB copy, only the 64 x 128^2 solve, only one decoder-set step "
                         "form, only a bottleneck-50 step form, only a single-parameter step form")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the batched solve is single-GPU; "
                                   "multi-GPU sharding is a design note, not an implemented path"}))
        sys.exit(2)

    import numpy as np
    import torch
    import matrix_inverse_roots_amd as mir
    import synthetic

    dev = torch.device("cuda:0")
    K, W_ = args.steps, args.warmup
    if args.only == "copy":
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        log("copied 1 GiB three times")
        return
    step_forms = {
        "step": dict(compute="f32"),
        "step_f16": dict(compute="f16", fallback="f64"),
        "step_f16_tol": dict(compute="f16", fallback="f64", tol=HALF_TOL),
        "step_f16_tol_pi": dict(compute="f16", fallback="f64", tol=HALF_TOL, scaling="power"),
        "step_f16_tol_pi_pbf16": dict(compute="f16", fallback="f64", tol=HALF_TOL, scaling="power", precond_bf16=True),
        "step_tol_res_pi": dict(compute="f32", stats64=True, fallback="f64", tol=1e-4, bound=RESIDUAL_BOUND,
                                scaling="power"),
        "step_tol": dict(compute="f32", tol=1e-4),
        "step_res": dict(compute="f32", stats64=True, fallback="f64", bound=RESIDUAL_BOUND),
        "step_tol_res": dict(compute="f32", stats64=True, fallback="f64", tol=1e-4, bound=RESIDUAL_BOUND),
        "step_f64": dict(compute="f64", stats64=True),
    }
    if args.only in step_forms:
        ms, nf = decoder_step_ms(mir, K, max(1, W_), **step_forms[args.only])
        log(f"decoder step ({args.only}): {ms:.2f} ms, flagged {nf}")
        return
    if args.only == "cheb_sweep":
        chebyshev_sweep(mir)
        return
    if args.only in ("step1", "step1_f64"):
        f64 = args.only == "step1_f64"
        e, gr, _ = single_step_ms(mir, max(K, 20), max(W_, 3), compute="f64" if f64 else "f32", stats64=f64,
                                  graph=True)
        log(f"single-parameter step: {e:.3f} ms eager, {gr:.3f} ms as a graph replay")
        return
    if args.only in ("step5", "step5_ps"):
        ms, nf = bottleneck_step_ms(mir, K, W_, True, "ps" if args.only == "step5_ps" else "clenshaw")
        log(f"bottleneck-50 step {ms:.2f} ms, flags {nf}")
        return
    if args.only == "spd128":
        for c in ("f64", "f32"):
            rec, _ = spd128_solve(mir, c)
            log(f"64 x 128^2 CN 20 {c}: {rec}")
        return

    if args.blocks is not None and not (args.only or "").startswith("roots"):
        print(json.dumps({"error": "--blocks is for --only roots* profiling runs"}))
        sys.exit(2)
    A64 = make_stack(args.blocks)
    n = A64.shape[0]
    V0 = torch.from_numpy(synthetic.pi_start_vectors(3, PI_VECTORS, B)).to(dev)
    opts = mir.RootOpts(method="ndb", scaling="power", compute="f64", iters=ITERS1, iters2=ITERS2,
                        pi_vectors=PI_VECTORS, pi_iters=PI_ITERS, pi_start=V0)
    ngemm = gemm_count_ndb(ITERS1, ITERS2)
    if args.only in ("roots_f32", "roots_f16"):
        comp = args.only[-3:]
        inp = torch.from_numpy(A64.astype(np.float32)).to(dev)
        dt, _, nflag, nnf, _ = time_roots(mir, inp, mir.RootOpts(**{**opts.__dict__, "compute": comp}), K, W_)
        log(f"{comp} NDB+PI: {dt * 1e3:.1f} ms per call, {n / dt:.1f} blocks/s, non-finite blocks {nnf}")
        return
    inp64 = torch.from_numpy(A64).to(dev)
    dt, gemm_ms, nflag, nnf, out64 = time_roots(mir, inp64, opts, K, W_, timing_cap=K * ngemm)
    value = n / dt
    log(f"f64 NDB+PI: {dt * 1e3:.1f} ms per call, {value:.1f} blocks/s, flagged blocks {nflag}")
    if args.only == "roots":
        return

    # roofline of the dominant kernel: the float64 batched product (Newton-DB
    # multiplies full matrices, so the executed work equals the algorithmic
    # work: 2 B^3 flop per block, 1024 blocks per launch)
    flops_alg = N_BLOCKS * 2.0 * B ** 3
    mean_gemm = float(np.mean(gemm_ms)) * 1e-3 if gemm_ms else float("nan")
    achieved = flops_alg / mean_gemm / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP64_MFMA, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP64_MFMA, 4), "traffic": traffic_from_profiles("gemm_f64_b512"),
            "kernel": "gemm_p128_kernel<double, true, false>", "launches_timed": len(gemm_ms),
            "mean_launch_ms": round(mean_gemm * 1e3, 4), "flop_per_launch": flops_alg,
            "algorithmic_bytes_per_launch": 3 * N_BLOCKS * B * B * 8}
    gemm_share = float(np.sum(gemm_ms)) * 1e-3 / (dt * K) if gemm_ms else None
    # matrix-core ceilings re-measured on this part (register-only MFMA chains);
    # the datasheet peak stays the denominator of frac
    peaks = {d: round(mir.shampoo_mfma_peak(d), 1) for d in ("f32", "f64", "f16", "bf16")}
    log(f"measured matrix-core peaks (TFLOP/s): {peaks}")
    roof["peak_measured"] = peaks["f64"]
    roof["frac_of_measured"] = round(achieved / peaks["f64"], 4)

    result = {"metric": METRIC, "value": round(value, 2), "unit": "blocks/s", "n_gpus": 1,
              "steps": K, "warmup": W_, "ms_per_step": round(dt * 1e3, 3),
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f64",
              "data": "synthetic",
              "config": {"workload": "spd_stack_1024x512_lambda_1e-8_1_newton_db_28_17_power_16x10",
                         "n_blocks": N_BLOCKS, "B": B, "p": 4, "method": "ndb", "iters": [ITERS1, ITERS2],
                         "scaling": "power", "pi_vectors": PI_VECTORS, "pi_iters": PI_ITERS,
                         "compute": "f64", "batched_products": ngemm, "parity_bar": 1e-4},
              "roofline": roof, "measured_mfma_peaks_tflops": peaks, "flagged_blocks": nflag,
              "gemm_time_share": None if gemm_share is None else round(gemm_share, 4)}
    res64 = device_residuals(mir, inp64, opts)
    out64_host = out64.cpu().numpy()
    del out64
    del inp64
    dres = {"f64": residual_summary(res64)}

    if not args.no_variants:
        var = {}
        inp32 = torch.from_numpy(A64.astype(np.float32)).to(dev)
        for comp in ("f32", "f16"):
            o2 = mir.RootOpts(**{**opts.__dict__, "compute": comp})
            steps = max(1, K // 2)
            d2, gm, nf2, nnf2, o_var = time_roots(mir, inp32, o2, steps, 1, timing_cap=steps * ngemm)
            del o_var
            peak = PEAK_FP16_MFMA if comp == "f16" else PEAK_FP32_MFMA
            mg = float(np.mean(gm)) * 1e-3
            var[comp] = {"blocks_per_s": round(N_BLOCKS / d2, 2), "ms_per_call": round(d2 * 1e3, 2),
                         "nonfinite_blocks": nnf2, "flagged_blocks": nf2, "gemm_mean_ms": round(mg * 1e3, 4),
                         "gemm_tflops": round(flops_alg / mg / 1e12, 2),
                         "gemm_frac": round(flops_alg / mg / 1e12 / peak, 4),
                         "parity": "diagnostic: %s cannot resolve condition number 1e8 (non-finite blocks "
                                   "flagged)" % ("float32" if comp == "f32" else "half precision")}
            dres[comp] = residual_summary(device_residuals(mir, inp32, o2))
            log(f"{comp}: {var[comp]}")
        del inp32
        result["variants"] = var
    result["device_residual"] = dres
    log(f"device residuals ||X^4 A - I||_F / sqrt(B): {dres}")

    cfg = {}
    if not args.no_full_step:
        # 64 x 128^2, coupled Newton 20 (float64 meets 1e-4; float32 is a diagnostic)
        r64, x128 = spd128_solve(mir, "f64")
        r32, _ = spd128_solve(mir, "f32")
        r32["parity"] = "diagnostic: float32 rounding at condition number 1e6 moves the root by >1e-4"
        cfg["spd_stack_64x128_lambda_1e-6_1_cn20_frobenius"] = {"f64": r64, "f32": r32, "parity_bar": 1e-4}
        log(f"64 x 128^2 CN 20: f64 {r64}, f32 {r32}")
        # single parameter 256 x 128
        e64, g64, _ = single_step_ms(mir, 50, 5, compute="f64", stats64=True, graph=True)
        eres, _, nres = single_step_ms(mir, 50, 5, compute="f32", stats64=True, fallback="f64", bound=RESIDUAL_BOUND)
        e32, g32, _ = single_step_ms(mir, 50, 5, compute="f32", graph=True)
        cfg["single_256x128_b128_sum_stats_cn30_sgd"] = {
            "f64_ms": round(e64, 3), "f64_graph_replay_ms": round(g64, 3),
            "f32_chain_residual_checked_ms": round(eres, 3), "f32_chain_residual_flagged": nres,
            "f32_diagnostic_ms": round(e32, 3), "f32_diagnostic_graph_replay_ms": round(g32, 3),
            "parity_bar": 1e-4, "parity_paths": ["f64", "f32_chain_residual_checked"]}
        log(f"single parameter: {cfg['single_256x128_b128_sum_stats_cn30_sgd']}")
        # decoder set
        ks = max(3, K)
        dec = {"parity_bar": 1e-4, "parity_paths": ["f64", "f32_chain_residual_checked",
                                                    "f32_chain_tol1e-4_residual_checked",
                                                    "f32_chain_tol1e-4_power_scaling_residual_checked"]}
        ms, nf = decoder_step_ms(mir, ks, 1, compute="f32", stats64=True, fallback="f64", tol=1e-4,
                                 bound=RESIDUAL_BOUND)
        dec["f32_chain_tol1e-4_residual_checked_ms"], dec["f32_chain_tol1e-4_residual_checked_flagged"] = round(ms, 2), nf
        ms, nf = decoder_step_ms(mir, ks, 1, compute="f32", stats64=True, fallback="f64", tol=1e-4,
                                 bound=RESIDUAL_BOUND, scaling="power")
        dec["f32_chain_tol1e-4_power_scaling_residual_checked_ms"] = round(ms, 2)
        dec["f32_chain_tol1e-4_power_scaling_residual_checked_flagged"] = nf
        ms, nf = decoder_step_ms(mir, ks, 1, compute="f32", stats64=True, fallback="f64", bound=RESIDUAL_BOUND)
        dec["f32_chain_residual_checked_ms"], dec["f32_chain_residual_checked_flagged"] = round(ms, 2), nf
        ms, nf = decoder_step_ms(mir, 2, 1, compute="f64", stats64=True)
        dec["f64_ms"] = round(ms, 2)
        ms, nf = decoder_step_ms(mir, ks, 1, compute="f16", fallback="f64")
        dec["cn_f16_products_ms"], dec["cn_f16_products_flagged"] = round(ms, 2), nf
        dec["cn_f16_products_parity_bar"] = 2e-2
        ms, nf = decoder_step_ms(mir, ks, 1, compute="f16", fallback="f64", tol=HALF_TOL)
        dec["cn_f16_products_tol0.1_ms"], dec["cn_f16_products_tol0.1_flagged"] = round(ms, 2), nf
        ms, nf = decoder_step_ms(mir, ks, 1, compute="f16", fallback="f64", tol=HALF_TOL, scaling="power")
        dec["cn_f16_products_tol0.1_power_scaling_ms"] = round(ms, 2)
        dec["cn_f16_products_tol0.1_power_scaling_flagged"] = nf
        ms, nf = decoder_step_ms(mir, ks, 1, compute="f16", fallback="f64", tol=HALF_TOL, scaling="power",
                                 precond_bf16=True)
        dec["cn_f16_products_tol0.1_power_scaling_bf16_precondition_ms"] = round(ms, 2)
        dec["cn_f16_products_tol0.1_power_scaling_bf16_precondition_flagged"] = nf
        ms, nf = decoder_step_ms(mir, ks, 1, compute="f32")
        dec["f32_diagnostic_ms"] = round(ms, 2)
        cfg[DECODER + "_cn34"] = dec
        log(f"decoder set: {dec}")
        # bottleneck-50 set
        msg, nfg = bottleneck_step_ms(mir, max(5, K), 2, True)
        msu, nfu = bottleneck_step_ms(mir, max(5, K), 2, False)
        msp, nfp = bottleneck_step_ms(mir, max(5, K), 2, True, "ps")
        msh, nfh = bottleneck_step_ms(mir, max(5, K), 2, True, "ps", "f16")
        cfg["bottleneck50_53_matrices_b256_1024_chebyshev16_momentum"] = {
            "ms_grouped_by_factor_side": round(msg, 2), "ms_padded_to_block": round(msu, 2),
            "ms_grouped_paterson_stockmeyer": round(msp, 2),
            "ms_grouped_paterson_stockmeyer_f16_products": round(msh, 2), "flagged_factors": nfg + nfu + nfp + nfh,
            "parity_bar": 1e-4, "f16_products_parity_bar": 2e-2,
            "root_gflop_per_step_clenshaw_15_products": bottleneck_root_gflop(mir, 15),
            "root_gflop_per_step_paterson_stockmeyer_6_products": bottleneck_root_gflop(mir, 6)}
        log(f"bottleneck-50: {cfg['bottleneck50_53_matrices_b256_1024_chebyshev16_momentum']}")
        result["configs"] = cfg
    if not args.no_cpu_baseline:
        base, par = cpu_baseline(A64, out64_host)
        result["cpu_baseline"] = base
        if not args.no_full_step:
            result["cpu_baseline"]["full_steps"] = oracle_full_steps()
            par["spd_stack_64x128_cn20_f64"] = oracle_spd128(x128)
            par["decoder12_fastest_step_forms"] = oracle_decoder_parity(mir)
        log(f"cpu baseline: {result['cpu_baseline']}")
        result["parity_sample"] = par
        log(f"parity sample: {par}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python
"""Benchmark of the batched block preconditioner step on one MI355X.

Headline: inverse 4th roots of a stack of 1024 SPD blocks 512 x 512 with
eigenvalues log-uniform in [1e-8, 1] (Q diag(lambda) Q^T, Haar Q), by
Newton-DB (28 + 17 iterations) after half-precision multi-start power
iteration scaling (16 vectors, 10 products), float32 arithmetic.  A step is
one shampoo_inverse_root call over the whole stack (1024 blocks), input
resident in HBM.  value = blocks/s.

Also reported: the half-precision-product and float64 variants of the same
solve, the full optimizer step (pack, statistics, roots, preconditioning,
grafting, update) on the 12-layer decoder parameter set in ms, the roofline
of the dominant kernel (the float32 batched product) from HIP events around
its launches, and the CPU oracle timed on a bounded sample.

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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_count_ndb(k1, k2):
    """Batched products the Newton-DB chain launches for p = 4 (k1, k2 >= 2)."""
    return (3 * k1 - 3) + (3 * k2 - 3)


def make_stack(dtype, n=None):
    import numpy as np
    import synthetic
    t = time.time()
    A = synthetic.spd_stack(3, N_BLOCKS if n is None else n, B, 1e-8, 1.0)
    log(f"generated the SPD stack in {time.time() - t:.1f} s")
    return A


def time_roots(mir, inp, opts, steps, warmup, timing_cap=0):
    import torch
    out = torch.empty_like(inp)
    flags = torch.zeros(inp.shape[0], dtype=torch.int32, device=inp.device)
    nb = mir.shampoo_inverse_root_workspace(inp.shape[0], B, 4, opts)
    ws = torch.empty(nb, dtype=torch.uint8, device=inp.device)
    for _ in range(warmup):
        mir.shampoo_inverse_root(inp, out, 4, opts, flags=flags, ws=ws)
    torch.cuda.synchronize()
    if timing_cap:
        mir.shampoo_timing_enable(timing_cap)
    flags.zero_()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        mir.shampoo_inverse_root(inp, out, 4, opts, flags=flags, ws=ws)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    gemm_ms = []
    if timing_cap:
        gemm_ms = mir.shampoo_timing_read(timing_cap)
        mir.shampoo_timing_enable(0)
    nflag = int((flags != 0).sum().item())
    del ws
    return dt, gemm_ms, nflag, out


PARITY_SAMPLE = (0, 511, 1023)


def parity_sample(A64, out32, out64):
    """The oracle's roots of sampled blocks beside the GPU's: relative
    Frobenius error and the solver residual ||X^4 A - I||_F / sqrt(B) of the
    float64 and float32 chains and of the oracle's eigendecomposition root."""
    import numpy as np
    import oracle
    rep = {"blocks": list(PARITY_SAMPLE), "oracle_residual": [], "f64_rel_err": [], "f64_residual": [],
           "f32_finite": [], "f32_residual": []}
    for k, i in enumerate(PARITY_SAMPLE):
        A = A64[i]
        ref = oracle.inverse_root_eigh(A, 4)
        rep["oracle_residual"].append(oracle.residual(ref, A, 4))
        if out64 is not None:
            rep["f64_rel_err"].append(float(np.linalg.norm(out64[k] - ref) / np.linalg.norm(ref)))
            rep["f64_residual"].append(oracle.residual(out64[k], A, 4))
        x32 = out32[k].astype(np.float64)
        fin = bool(np.isfinite(x32).all())
        rep["f32_finite"].append(fin)
        rep["f32_residual"].append(oracle.residual(x32, A, 4) if fin else None)
    return rep


def cpu_baseline(sample_f32, budget_s=15.0):
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        cores = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) if threadpoolctl.threadpool_info() else 1
    except Exception:
        cores = os.cpu_count()
    t0 = time.perf_counter()
    done = 0
    for i in range(sample_f32.shape[0]):
        oracle.inverse_root_eigh(sample_f32[i].astype(np.float64), 4)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    # the same roots on one thread (a few seconds)
    one = None
    try:
        import threadpoolctl
        with threadpoolctl.threadpool_limits(1):
            t1 = time.perf_counter()
            k = 0
            while k < sample_f32.shape[0] and (k == 0 or time.perf_counter() - t1 < budget_s / 3):
                oracle.inverse_root_eigh(sample_f32[k].astype(np.float64), 4)
                k += 1
            one = k / (time.perf_counter() - t1)
    except Exception:
        pass
    return {"value": done / dt, "unit": "blocks/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of the {N_BLOCKS} blocks (512 x 512, float32 input), float64 eigh inverse 4th root each",
            "value_1thread": one, "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model()}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


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


def full_step_ms(mir, steps, warmup, compute="f32", fallback="none", tol=0.0):
    """Full step on the 12-layer decoder set (151 M parameters, block 1024,
    bfloat16 gradients N(0, 0.02^2), beta2 0.999, eps 1e-12, Adam grafting,
    coupled Newton 34 iterations with float32 or half-precision products,
    or stopping at a tolerance, roots every step).  Returns the median step time and the number of
    factors flagged during the timed steps."""
    import numpy as np
    import torch
    import synthetic
    shapes = synthetic.decoder_shapes()
    W = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in shapes]
    opt = mir.Shampoo(W, block_size=1024, beta2=0.999, eps=1e-12,
                      root=mir.RootOpts(method="cn", iters=34, compute=compute, tol=tol),
                      graft="adam", lr=1e-3, grad_dtype=torch.bfloat16, fallback=fallback)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4)
    grads = [[(torch.randn(s, generator=gen, device="cuda") * 0.02).to(torch.bfloat16) for s in shapes]
             for _ in range(2)]
    for i in range(warmup):
        opt.step(grads[i % 2])
    torch.cuda.synchronize()
    for f in opt.flags():
        f.zero_()
    times = []
    for i in range(warmup, warmup + steps):
        t0 = time.perf_counter()
        opt.step(grads[i % 2])
        torch.cuda.synchronize()
        times.append((time.perf_counter() - t0) * 1e3)
    nflag = sum(int((f != 0).sum().item()) for f in opt.flags())
    return float(np.median(times)), nflag


def chebyshev_sweep(mir, degrees=(16, 40, 60, 100)):
    """Chebyshev inverse 4th roots of 288 SPD matrices 1024 x 1024 (the
    decoder set's factor stack; A = X X^T / 1024 + 1e-3 I with X N(0, 1) drawn
    on the device), Frobenius scaling, for the degree sweep: float32 and
    half-precision products, Clenshaw's recurrence and the Paterson-Stockmeyer
    split.  Returns {(degree, compute, eval): (ms per call, products)}."""
    import torch
    n, B = 288, 1024
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    A = torch.empty((n, B, B), device="cuda")
    for i in range(0, n, 32):
        X = torch.randn((32, B, B), generator=gen, device="cuda")
        A[i:i + 32] = torch.bmm(X, X.transpose(1, 2).contiguous()) / B
    A += 1e-3 * torch.eye(B, device="cuda")
    out = torch.empty_like(A)
    res = {}
    for d in degrees:
        for compute in ("f32", "f16"):
            for ev in ("clenshaw", "ps"):
                opts = mir.RootOpts(method="chebyshev", cheb_degree=d, cheb_eval=ev, compute=compute, eps=1e-3)
                ws = torch.empty(mir.shampoo_inverse_root_workspace(n, B, 4, opts), dtype=torch.uint8, device="cuda")
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


def single_step_ms(mir, steps, warmup):
    """Step on one [256, 128] float32 parameter in two 128-blocks (gradients
    N(0, 1), statistics summed (beta2 1), eps 1e-12, coupled Newton 30 in
    float32, SGD grafting lr 0.1): a launch-bound step, timed eagerly and as
    a graph replay.  Returns (eager ms, replay ms)."""
    import numpy as np
    import torch
    W = [torch.zeros((256, 128), dtype=torch.float32, device="cuda")]
    opt = mir.Shampoo(W, block_size=128, beta2=1.0, eps=1e-12, root=mir.RootOpts(method="cn", iters=30),
                      graft="sgd", lr=0.1)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0)
    grads = [[torch.randn((256, 128), generator=gen, device="cuda")] for _ in range(2)]
    static = [torch.empty((256, 128), device="cuda")]

    def timed(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        times = []
        for i in range(warmup, warmup + steps):
            t0 = time.perf_counter()
            fn(i)
            torch.cuda.synchronize()
            times.append((time.perf_counter() - t0) * 1e3)
        return float(np.median(times))

    eager = timed(lambda i: opt.step(grads[i % 2]))
    static[0].copy_(grads[0][0])
    opt.step(static)
    replay = opt.capture(static)

    def rep(i):
        replay()

    graph = timed(rep)
    return eager, graph


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
    import numpy as np
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
    for i in range(warmup):
        opt.step(grads[i % 2])
    torch.cuda.synchronize()
    times = []
    for i in range(warmup, warmup + steps):
        t0 = time.perf_counter()
        opt.step(grads[i % 2])
        torch.cuda.synchronize()
        times.append((time.perf_counter() - t0) * 1e3)
    nflag = sum(int((f != 0).sum().item()) for f in opt.flags())
    return float(np.median(times)), nflag


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true")
    ap.add_argument("--no-full-step", action="store_true")
    ap.add_argument("--blocks", type=int, default=None,
                    help="with --only roots: solve only the first this-many blocks (counter runs whose "
                         "per-dispatch cycle counts would otherwise overflow 32 bits)")
    ap.add_argument("--only", choices=["roots", "copy", "step", "step_f16", "step_tol", "step5", "step5_ps", "step1",
                                       "cheb_sweep"],
                    default=None,
                    help="profiling runs: only the float32 solve, only a 1 GiB copy, only the decoder-set step "
                         "(float32 or half-precision products) or only the bottleneck-50 step (Clenshaw or "
                         "Paterson-Stockmeyer Chebyshev sums)")
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
    if args.only == "copy":
        x = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        log("copied 1 GiB three times")
        return
    if args.only in ("step", "step_f16"):
        half = args.only == "step_f16"
        ms, nf = full_step_ms(mir, args.steps, max(1, args.warmup), "f16" if half else "f32", "f64" if half else "none")
        log(f"full step {ms:.2f} ms, flags {nf}")
        return
    if args.only == "cheb_sweep":
        chebyshev_sweep(mir)
        return
    if args.only == "step_tol":
        ms, nf = full_step_ms(mir, args.steps, max(1, args.warmup), "f32", "none", 1e-4)
        log(f"full step, Newton tolerance 1e-4: {ms:.2f} ms, flags {nf}")
        return
    if args.only == "step1":
        e, gr = single_step_ms(mir, max(args.steps, 20), max(args.warmup, 3))
        log(f"single-parameter step: {e:.3f} ms eager, {gr:.3f} ms as a graph replay")
        return
    if args.only in ("step5", "step5_ps"):
        ms, nf = bottleneck_step_ms(mir, args.steps, args.warmup, True,
                                    "ps" if args.only == "step5_ps" else "clenshaw")
        log(f"bottleneck-50 step {ms:.2f} ms, flags {nf}")
        return

    if args.blocks is not None and args.only != "roots":
        print(json.dumps({"error": "--blocks is for --only roots profiling runs"}))
        sys.exit(2)
    A64 = make_stack(np.float64, args.blocks)
    inp = torch.from_numpy(A64.astype(np.float32)).to(dev)
    V0 = torch.from_numpy(synthetic.pi_start_vectors(3, PI_VECTORS, B)).to(dev)
    opts = mir.RootOpts(method="ndb", scaling="power", compute="f32", iters=ITERS1, iters2=ITERS2,
                        pi_vectors=PI_VECTORS, pi_iters=PI_ITERS, pi_start=V0)
    ngemm = gemm_count_ndb(ITERS1, ITERS2)
    dt, gemm_ms, nflag, out = time_roots(mir, inp, opts, args.steps, args.warmup, timing_cap=args.steps * ngemm)
    value = inp.shape[0] / dt
    log(f"f32 NDB+PI: {dt * 1e3:.1f} ms per call, {value:.1f} blocks/s, flagged blocks {nflag}")
    if args.only == "roots":
        return

    # roofline of the dominant kernel: the float32 batched product (Newton-DB
    # multiplies full matrices, so the executed work equals the algorithmic
    # work: 2 B^3 flop per block, 1024 blocks per launch)
    flops_alg = N_BLOCKS * 2.0 * B ** 3
    mean_gemm = float(np.mean(gemm_ms)) * 1e-3 if gemm_ms else float("nan")
    achieved = flops_alg / mean_gemm / 1e12
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_FP32_MFMA, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_FP32_MFMA, 4), "traffic": traffic_from_profiles("gemm_f32_b512"),
            "kernel": "gemm_f32_nn256_kernel", "launches_timed": len(gemm_ms),
            "mean_launch_ms": round(mean_gemm * 1e3, 4), "flop_per_launch": flops_alg,
            "algorithmic_bytes_per_launch": 3 * N_BLOCKS * B * B * 4}
    gemm_share = float(np.sum(gemm_ms)) * 1e-3 / (dt * args.steps) if gemm_ms else None
    # matrix-core ceilings re-measured on this part (register-only MFMA chains);
    # the datasheet peak stays the denominator of frac
    peaks = {d: round(mir.shampoo_mfma_peak(d), 1) for d in ("f32", "f64", "f16", "bf16")}
    log(f"measured matrix-core peaks (TFLOP/s): {peaks}")
    roof["peak_measured"] = peaks["f32"]
    roof["frac_of_measured"] = round(achieved / peaks["f32"], 4)

    result = {"metric": METRIC, "value": round(value, 2), "unit": "blocks/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 3),
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
              "data": "synthetic",
              "config": {"workload": "spd_stack_1024x512_lambda_1e-8_1_newton_db_28_17_power_16x10",
                         "n_blocks": N_BLOCKS, "B": B, "p": 4, "method": "ndb", "iters": [ITERS1, ITERS2],
                         "scaling": "power", "pi_vectors": PI_VECTORS, "pi_iters": PI_ITERS,
                         "compute": "f32", "batched_products": ngemm},
              "roofline": roof, "measured_mfma_peaks_tflops": peaks, "flagged_blocks": nflag,
              "gemm_time_share": None if gemm_share is None else round(gemm_share, 4)}

    if not args.no_variants:
        var = {}
        for comp in ("f16", "f64"):
            o2 = mir.RootOpts(**{**opts.__dict__, "compute": comp})
            x = inp if comp != "f64" else torch.from_numpy(A64).to(dev)
            steps = max(1, args.steps // 2)
            d2, gm, nf2, o_var = time_roots(mir, x, o2, steps, 1, timing_cap=steps * ngemm)
            if comp == "f64":
                out64_sample = o_var[list(PARITY_SAMPLE)].cpu().numpy()
            peak = PEAK_FP16_MFMA if comp == "f16" else PEAK_FP64_MFMA
            mg = float(np.mean(gm)) * 1e-3
            var[comp] = {"blocks_per_s": round(N_BLOCKS / d2, 2), "ms_per_call": round(d2 * 1e3, 2),
                         "flagged_blocks": nf2, "gemm_mean_ms": round(mg * 1e3, 4),
                         "gemm_tflops": round(flops_alg / mg / 1e12, 2),
                         "gemm_frac": round(flops_alg / mg / 1e12 / peak, 4)}
            log(f"{comp}: {var[comp]}")
            del x
        result["variants"] = var
    if not args.no_full_step:
        ms, nf = full_step_ms(mir, max(3, args.steps), 1)
        result["full_step"] = {"workload": "decoder_12x(1024x3072,1024x1024,1024x4096,4096x1024)_bf16_adam_cn34_f32",
                               "ms": round(ms, 2), "flagged_factors": nf}
        log(f"full step: {ms:.1f} ms")
        # the pages' CN-FP16 configuration: half-precision products; the
        # single-Gram step-1 factors (warm-up) diverge in half precision and
        # are recomputed by the float64 fallback, later ones converge
        ms16, nf16 = full_step_ms(mir, max(3, args.steps), 1, "f16", "f64")
        result["full_step_cn_f16"] = {
            "workload": "decoder_12x(1024x3072,1024x1024,1024x4096,4096x1024)_bf16_adam_cn34_f16_products_f64_fallback",
            "ms": round(ms16, 2), "flagged_factors": nf16}
        log(f"full step, half-precision products: {ms16:.1f} ms (flagged {nf16})")
        mst, nft = full_step_ms(mir, max(3, args.steps), 2, "f32", "none", 1e-4)
        result["full_step_cn_tol"] = {
            "workload": "decoder_12x(1024x3072,1024x1024,1024x4096,4096x1024)_bf16_adam_cn_tol1e-4_max34_f32",
            "ms": round(mst, 2), "flagged_factors": nft}
        log(f"full step, Newton tolerance 1e-4 (at most 34 iterations): {mst:.1f} ms (flagged {nft})")
        msg, nfg = bottleneck_step_ms(mir, max(5, args.steps), 2, True)
        msu, nfu = bottleneck_step_ms(mir, max(5, args.steps), 2, False)
        msp, nfp = bottleneck_step_ms(mir, max(5, args.steps), 2, True, "ps")
        msh, nfh = bottleneck_step_ms(mir, max(5, args.steps), 2, True, "ps", "f16")
        result["full_step_bottleneck50"] = {
            "workload": "bottleneck50_53_matrices_b256_1024_chebyshev16_f32_momentum",
            "ms_grouped_by_factor_side": round(msg, 2), "ms_padded_to_block": round(msu, 2),
            "ms_grouped_paterson_stockmeyer": round(msp, 2),
            "ms_grouped_paterson_stockmeyer_f16_products": round(msh, 2), "flagged_factors": nfg + nfu + nfp + nfh,
            "root_gflop_per_step_clenshaw_15_products": bottleneck_root_gflop(mir, 15),
            "root_gflop_per_step_paterson_stockmeyer_6_products": bottleneck_root_gflop(mir, 6)}
        log(f"bottleneck-50 step: {msg:.1f} ms grouped, {msu:.1f} ms padded, {msp:.1f} ms grouped with the "
            f"Paterson-Stockmeyer sum, {msh:.1f} ms with half-precision products")
        e1, g1 = single_step_ms(mir, 50, 5)
        result["full_step_single"] = {
            "workload": "one_256x128_f32_param_b128_sum_stats_cn30_f32_sgd",
            "ms_eager": round(e1, 3), "ms_graph_replay": round(g1, 3)}
        log(f"single-parameter step: {e1:.3f} ms eager, {g1:.3f} ms graph replay")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp[:256].cpu().numpy())
        if not args.no_full_step:
            result["cpu_baseline"]["full_steps"] = oracle_full_steps()
        log(f"cpu baseline: {result['cpu_baseline']}")
        result["parity_sample"] = parity_sample(A64, out[list(PARITY_SAMPLE)].cpu().numpy(),
                                                None if args.no_variants else out64_sample)
        log(f"parity sample: {result['parity_sample']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

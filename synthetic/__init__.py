"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke run.

This module only draws random numbers and builds the shapes of the workloads.
It holds none of the method's arithmetic, and neither the oracle nor the HIP
path is imported here.  All draws use numpy's PCG64 generator in float64 and
are cast with round-to-nearest-even (float64 -> float32 by numpy; float32 ->
bfloat16 by the bit rule below), so both sides consume identical bits.

Workloads (shapes and distributions; no dataset is used):

* ``single``: one 256 x 128 float32 parameter, gradients N(0, 1), seed 0.
* ``spd_stack``: Q diag(lambda) Q^T with Haar-random Q (QR of a Gaussian,
  column signs fixed by diag(R)) and lambda log-uniform in [lo, hi].
* ``decoder``: 12 decoder layers, d_model 1024, MLP 4096: per layer QKV
  1024 x 3072, attention out 1024 x 1024, MLP up 1024 x 4096 and MLP down
  4096 x 1024; bfloat16 gradients N(0, 0.02^2), seed 4.
* ``bottleneck50``: a 50-layer bottleneck CNN (stages of width 64/128/256/512
  with 3/4/6/3 blocks, 1x1 -> 3x3 -> 1x1 convolutions with expansion 4, a 1x1
  projection in each stage's first block, the 7x7 stem left out) with kernels
  viewed as (out, in * k * k), plus a 2048 x 1000 fully connected layer;
  float32 gradients with variance 1e-2, seed 5; block size 1024 for matrices
  with a side of at least 2048, else 256.
"""

import numpy as np


def rng(seed):
    return np.random.Generator(np.random.PCG64(int(seed)))


# ----------------------------------------------------------------------------
# casts
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits):
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32)


# ----------------------------------------------------------------------------
# SPD stacks
# ----------------------------------------------------------------------------

def haar_orthogonal(gen, n, b):
    """n Haar-random b x b orthogonal matrices."""
    Z = gen.standard_normal((n, b, b))
    Q, R = np.linalg.qr(Z)
    d = np.sign(np.diagonal(R, axis1=1, axis2=2))
    d = np.where(d == 0, 1.0, d)
    return Q * d[:, None, :]


def spd_stack(seed, n, b, lam_lo, lam_hi, return_factors=False, chunk=64):
    """n SPD matrices Q diag(lambda) Q^T (float64, exactly symmetric).

    Draw order: all Gaussian matrices for Q (chunk by chunk), then all
    eigenvalue uniforms.  Returns A [n, b, b] (and lambda [n, b], Q [n, b, b]
    if ``return_factors``).
    """
    gen = rng(seed)
    Q = np.empty((n, b, b))
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        Q[i:i + m] = haar_orthogonal(gen, m, b)
    u = gen.uniform(size=(n, b))
    lam = 10.0 ** (np.log10(lam_lo) + u * (np.log10(lam_hi) - np.log10(lam_lo)))
    A = np.empty((n, b, b))
    for i in range(0, n, chunk):
        m = min(chunk, n - i)
        Ai = (Q[i:i + m] * lam[i:i + m, None, :]) @ np.swapaxes(Q[i:i + m], 1, 2)
        A[i:i + m] = 0.5 * (Ai + np.swapaxes(Ai, 1, 2))
    if return_factors:
        return A, lam, Q
    return A


def pi_start_vectors(seed, k, b):
    """k Gaussian power-iteration start vectors of length b ([k, b] float32)."""
    return rng(seed).standard_normal((k, b)).astype(np.float32)


# ----------------------------------------------------------------------------
# parameter sets
# ----------------------------------------------------------------------------

def single_shapes():
    return [(256, 128)]


def decoder_shapes(layers=12, d_model=1024, d_mlp=4096):
    out = []
    for _ in range(layers):
        out += [(d_model, 3 * d_model), (d_model, d_model), (d_model, d_mlp), (d_mlp, d_model)]
    return out


def bottleneck50_shapes():
    """2-D views (out, in * k * k) of the 52 convolutions plus the fc layer."""
    out = []
    cin = 64
    for width, nblocks in ((64, 3), (128, 4), (256, 6), (512, 3)):
        for i in range(nblocks):
            out.append((width, cin * 1))          # 1x1 reduce
            out.append((width, width * 9))        # 3x3
            out.append((4 * width, width * 1))    # 1x1 expand
            if i == 0:
                out.append((4 * width, cin * 1))  # 1x1 projection
            cin = 4 * width
    out.append((2048, 1000))                      # fully connected
    return out


def bottleneck50_block_sizes(shapes):
    return [1024 if max(m, n) >= 2048 else 256 for (m, n) in shapes]


def gaussian_grads(seed, shapes, steps, std, dtype=np.float32):
    """Gradients per step: a list (one per step) of lists of arrays.

    Draw order: step by step, parameter by parameter.  ``dtype`` float32
    returns float32 arrays; "bf16" returns uint16 bfloat16 bit patterns.
    """
    gen = rng(seed)
    out = []
    for _ in range(steps):
        gs = []
        for s in shapes:
            g = (gen.standard_normal(s) * std).astype(np.float32)
            gs.append(f32_to_bf16_bits(g) if dtype == "bf16" else g)
        out.append(gs)
    return out


def gram_spectrum_grads(seed, n, b, lam_lo, lam_hi):
    """n gradients G = Q diag(sqrt(lambda)) P^T (float32, b x b) with Q, P
    Haar and lambda log-uniform in [lam_lo, lam_hi]: G G^T and G^T G then
    have the eigenvalues lambda (up to float32 rounding of G).

    Draw order: all Gaussian matrices for Q, then for P, then the eigenvalue
    uniforms.
    """
    gen = rng(seed)
    Q = haar_orthogonal(gen, n, b)
    P = haar_orthogonal(gen, n, b)
    u = gen.uniform(size=(n, b))
    lam = 10.0 ** (np.log10(lam_lo) + u * (np.log10(lam_hi) - np.log10(lam_lo)))
    G = (Q * np.sqrt(lam)[:, None, :]) @ np.swapaxes(P, 1, 2)
    return G.astype(np.float32)

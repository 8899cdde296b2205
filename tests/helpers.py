"""Shared helpers of the GPU parity tests."""

import numpy as np


def rel_fro(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / d) if d > 0 else float(np.linalg.norm(x))


def device():
    import torch
    return torch.device("cuda:0")


def to_dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device())


def bf16_tensor(bits):
    """uint16 bfloat16 bit patterns -> device bfloat16 tensor (same bits)."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device())


def log(msg):
    print(msg, flush=True)


U32 = 2.0 ** -24


def _rounding_perturbation(A):
    """Typical size of a float32 rounding perturbation of one entry of A in
    its eigenbasis: u32 ||A||_F / sqrt(n)."""
    n = A.shape[0]
    return U32 * np.linalg.norm(A) / np.sqrt(n)


def f32_root_floor(A, p=4, eps=0.0):
    """First-order estimate of the relative Frobenius error of a float32 chain
    computing (A + eps I)^(-1/p): each eigenvalue moves by about
    e = u32 ||A||_F / sqrt(n), so lambda^(-1/p) moves by (e/p) lambda^(-1/p-1):
    error ~ (e/p) sqrt(sum lambda^(-2/p-2)) / sqrt(sum lambda^(-2/p))."""
    A = np.asarray(A, dtype=np.float64) + eps * np.eye(A.shape[0])
    lam = np.linalg.eigvalsh(A)
    lam = lam[lam > 0]
    e = _rounding_perturbation(A)
    return float(e / p * np.sqrt(np.sum(lam ** (-2.0 / p - 2))) / np.sqrt(np.sum(lam ** (-2.0 / p))))


def f32_direction_floor(L, R, p=4, eps=0.0):
    """The same estimate for D = L^(-1/p) G R^(-1/p) with L, R built from G:
    along a singular pair (sigma_j, u_j, v_j) of G, D carries
    l_j sigma_j r_j ~ 1, and a rounding move of lambda_j = sigma_j^2 changes
    it by about (e/p)/lambda_j per factor; over the rank r of G:
    error ~ sqrt(sum_F (e_F/p)^2 sum_j lambda_j^-2) / sqrt(r)."""
    tot = 0.0
    r = 1
    for F in (L, R):
        F = np.asarray(F, dtype=np.float64) + eps * np.eye(F.shape[0])
        lam = np.linalg.eigvalsh(F)
        lam = lam[lam > 1e-12 * lam.max()]
        r = max(r, lam.size)
        tot += (_rounding_perturbation(F) / p) ** 2 * np.sum(lam ** -2.0)
    return float(np.sqrt(tot) / np.sqrt(r))

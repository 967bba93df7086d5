"""Shared helpers of the GPU parity tests (host side only)."""
import math
import sys

import numpy as np

BF16_TOL = 2e-2   # relative Frobenius error, bf16 MFMA path
FP32_TOL = 1e-4   # relative Frobenius error, fp32 path
BUF_TOL = 1e-6    # momentum buffer, fp32 arithmetic vs fp64


def tol(compute):
    return BF16_TOL if compute == "bf16" else FP32_TOL


def announce(*parts):
    """Name the case before any GPU work, so a failing run says which one."""
    print("CASE", *parts, flush=True)
    sys.stdout.flush()


def to64(t):
    return t.detach().to("cpu").double().numpy()


def scalar_map(x, coeffs):
    for a, b, c in coeffs:
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def gram_eig(x0):
    """Eigendecomposition (l, v) of the Gram matrix x0 x0^T, fp64."""
    return np.linalg.eigh(x0 @ x0.T)


def gram_closed_form(x0, coeffs, eig=None):
    """U phi(Sigma) V^T of a normalised wide-or-square x0 (fp64), computed from
    the eigendecomposition of the Gram matrix x0 x0^T: O = V f(L) V^T x0 with
    f(l) = phi(sqrt l) / sqrt l.  Polynomial functional calculus, valid at any
    size; used where the step-by-step oracle would take minutes."""
    lam, v = eig if eig is not None else gram_eig(x0)
    s = np.sqrt(np.maximum(lam, 0.0))
    prod_a = float(np.prod([a for a, _, _ in coeffs]))
    f = np.empty_like(s)
    nz = s > 0
    f[nz] = scalar_map(s[nz], coeffs) / s[nz]
    f[~nz] = prod_a
    return (v * f) @ (v.T @ x0)


def normalise(g, eps=1e-7):
    g = np.asarray(g, np.float64)
    return g / (math.sqrt(float(np.sum(g * g))) + eps)

"""Shared helpers of the GPU parity tests (host side only)."""
import math
import sys

import numpy as np

BF16_TOL = 2e-2   # relative Frobenius error, bf16 MFMA path
FP32_TOL = 1e-4   # relative Frobenius error, fp32 path
BUF_TOL = 1e-6    # momentum buffer, fp32 arithmetic vs fp64
# bf16 path on matrices with min(rows, cols) < 64: the rounding of a few
# bf16 operands does not average out.  Emulating the bf16 design (bf16 X, A,
# B operands, fp32 accumulation and fp32 X) on 200 Gaussian draws per shape
# gives median ~2e-2 and maxima 3e-2 (16x8), 4.5e-2 (5x5), 8.6e-2 (8x2);
# from min dim 128 on the spread collapses to 1.5e-2 +- 5e-4.
BF16_SMALL_TOL = 1.5e-1
SMALL_DIM = 64


def tol(compute, shape=None):
    if compute != "bf16":
        return FP32_TOL
    if shape is not None and min(shape) < SMALL_DIM:
        return BF16_SMALL_TOL
    return BF16_TOL


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

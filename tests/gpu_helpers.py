"""Shared helpers of the GPU parity tests (host side only)."""
import math
import sys

import numpy as np

BF16_TOL = 2e-2   # relative Frobenius error, bf16 MFMA path
FP32_TOL = 1e-4   # relative Frobenius error, fp32 path
BUF_TOL = 1e-6    # momentum buffer, fp32 arithmetic vs fp64
# bf16 path on matrices with min(rows, cols) < 64: the rounding of a few bf16
# operands does not average out, and the error spreads well past 2e-2.  One
# bound per oriented shape (m, n) the GPU tests use, each between the maximum
# over 1000 Gaussian draws of the emulated bf16 path and 1.25 times it
# (tests/test_bf16_emulation.py recomputes the maxima and checks every entry:
# 1x1 0.118, 1x5 0.099, 2x8 0.117, 5x5 0.062, 8x16 0.037).  From min dim 64 on
# the emulated maximum stays below 2e-2 (64x64: 1.8e-2, 128x128: 1.5e-2).
BF16_SMALL_TOL = {(1, 1): 0.14, (1, 5): 0.11, (2, 8): 0.14, (5, 5): 0.075, (8, 16): 0.045}
SMALL_DIM = 64
# bf16 path on degenerate inputs (workloads.degenerate_matrix) whose
# singular vectors are flat: the bf16 rounding of B is then the same in many
# entries and adds up instead of averaging out.  A kind keeps BF16_TOL when
# the emulated bf16 path stays within 0.8 BF16_TOL on the shapes the GPU test
# uses (DEGENERATE_SHAPES); otherwise its bound lies between 1.1 and 1.25
# times the emulated maximum (tests/test_bf16_emulation.py checks both:
# constant 2.04e-2, duplicated rows 1.73e-2).
DEGENERATE_SHAPES = ((256, 384), (384, 256), (1024, 3072))
DEGENERATE_BF16_TOL = {"constant": 2.5e-2, "dup_rows": 2.1e-2}


def degenerate_tol(kind, compute):
    if compute != "bf16":
        return FP32_TOL
    return DEGENERATE_BF16_TOL.get(kind, BF16_TOL)


def tol(compute, shape=None):
    if compute != "bf16":
        return FP32_TOL
    if shape is not None and min(shape) < SMALL_DIM:
        key = (min(shape), max(shape))
        if key not in BF16_SMALL_TOL:
            raise KeyError(f"no derived bf16 bound for the small shape {key}")
        return BF16_SMALL_TOL[key]
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


def tile_errors(y, ref, tile=256):
    """Relative Frobenius error of every tile x tile block (ragged edge blocks
    included; blocks whose reference is zero are skipped)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    out = []
    for i in range(0, ref.shape[0], tile):
        for j in range(0, ref.shape[1], tile):
            r = ref[i:i + tile, j:j + tile]
            den = float(np.linalg.norm(r))
            if den > 0.0:
                out.append(float(np.linalg.norm(y[i:i + tile, j:j + tile] - r)) / den)
    return np.array(out)


# A fault confined to a few rows or one tile barely moves a large matrix's
# whole-matrix error; each 256 x 256 tile is held to the bar as well, and to
# 1.25x the matrix's own error (in the emulated bf16 path the tiles of one
# matrix stay within 1.1x of it: tests/test_bf16_emulation.py).
TILE_SPREAD = 1.25


def check_tiles(y, ref, bound, what=""):
    e = tile_errors(y, ref)
    whole = float(np.linalg.norm(np.asarray(y, np.float64) - ref)) / float(np.linalg.norm(ref))
    assert e.max() <= bound, (what, "tile", float(e.max()), int(e.argmax()))
    assert e.max() <= TILE_SPREAD * whole + 1e-12, (what, "spread", float(e.max()), whole)
    return float(e.max())

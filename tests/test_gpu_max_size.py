"""The largest matrix the library accepts, 2**31 elements after padding
(16384 x 131072, wide and tall), where element and byte offsets no longer fit
32 bits.  The input is a rectangular diagonal with its support scattered
over the columns (G[i][c_i] = d_i, c_i distinct): the Newton-Schulz
iteration then acts on each d_i alone, so the result has the same support
and O[i][c_i] = sign(d_i) phi(|d_i| / ||d||), phi the scalar quintic map
x -> a x + b x^3 + c x^5 composed five times (the identity the oracle pins
test on small rectangular diagonals).  Everything off the support must stay
exactly zero.  fp64 host arithmetic on the m support values only."""
import numpy as np
import pytest
import torch

import muon_newton_schulz_step_amd as mn
import oracle
import workloads as wl
from gpu_helpers import BF16_TOL, TILE_SPREAD, announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
M, N = 16384, 131072  # M * N = 2**31
EPS = 1e-7


def support(seed):
    rng = np.random.default_rng(seed)
    cols = rng.permutation(N)[:M]
    d = rng.uniform(0.5, 1.5, M) * rng.choice([-1.0, 1.0], M)
    d_bf16 = torch.tensor(d, dtype=torch.float32).to(torch.bfloat16)
    return cols, d_bf16


def expected(d_bf16, steps=5):
    d = d_bf16.double().numpy()
    x = d / (np.sqrt(np.sum(d * d)) + EPS)
    a, b, c = wl.QUINTIC
    for _ in range(steps):
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def scatter(tall, cols, vals, dtype):
    rows_idx = torch.arange(M, device=DEV)
    c = torch.tensor(cols, device=DEV)
    g = torch.zeros((N, M) if tall else (M, N), dtype=dtype, device=DEV)
    if tall:
        g[c, rows_idx] = vals.to(DEV, dtype)
    else:
        g[rows_idx, c] = vals.to(DEV, dtype)
    return g


def check(o, tall, cols, ref, scale=1.0):
    rows_idx = torch.arange(M, device=DEV)
    c = torch.tensor(cols, device=DEV)
    got = (o[c, rows_idx] if tall else o[rows_idx, c]).double().cpu().numpy()
    assert int(torch.count_nonzero(o)) == M  # nothing off the support
    assert np.all(got != 0.0)
    err = oracle.relative_frobenius_error(got, scale * ref)
    # each block of 256 rows (256 support values) on its own too: a fault in
    # a few rows barely moves the whole error (emulated blocks stay within
    # 1.13x of it)
    blocks = np.array([oracle.relative_frobenius_error(got[i:i + 256], scale * ref[i:i + 256])
                       for i in range(0, M, 256)])
    print("  support rel err", err, "worst 256-row block", blocks.max(), flush=True)
    assert err <= BF16_TOL
    assert blocks.max() <= BF16_TOL and blocks.max() <= TILE_SPREAD * err


@pytest.mark.parametrize("tall", [False, True], ids=["wide", "tall"])
def test_orthogonalize_at_maximum_size(tall):
    announce("orthogonalize maximum size", "tall" if tall else "wide", M, N)
    cols, d = support(21 + tall)
    g = scatter(tall, cols, d, torch.bfloat16)
    o = mn.orthogonalize(g, [wl.QUINTIC] * 5, compute="bf16", out_dtype=torch.float32)
    torch.cuda.synchronize()
    del g
    check(o, tall, cols, expected(d))
    del o
    torch.cuda.empty_cache()


def test_step_at_maximum_size_tall():
    # momentum (zero buffer: u = (1 + mu) g, the same direction), the Newton-
    # Schulz steps and the transposed write-back of a tall weight matrix
    announce("step maximum size tall", N, M)
    cols, d = support(23)
    g = scatter(True, cols, d, torch.bfloat16)
    buf = torch.zeros((N, M), dtype=torch.float32, device=DEV)
    w = torch.zeros((N, M), dtype=torch.float32, device=DEV)
    lr, mu = 0.02, 0.95
    mn.step([w], [g], [buf], mu=mu, lr=lr, scales=[1.0], coeffs=[wl.QUINTIC] * 5,
            compute="bf16")
    torch.cuda.synchronize()
    check(w, True, cols, expected(d), scale=-lr)
    # the momentum buffer is the gradient itself (zero start), exactly
    assert torch.equal(buf, g.float())
    del g, buf, w
    torch.cuda.empty_cache()

"""The identity behind the bf16 path's Q A Q Gram steps, in fp64 on the host.

A Newton-Schulz step maps X to Q X with Q = a I + B, B = b A + c A^2, so the
next Gram matrix is Q X X^T Q^T = Q A Q (Q is symmetric).  Iterating with
A formed that way at steps 1 and 3 must reproduce the oracle's iteration up
to rounding, for a per-step table too; taking Q from the wrong step's a
must not (the GPU parity test with an alternating table relies on that)."""
import numpy as np
import pytest

import oracle
import workloads as wl

TABLE = [wl.QUINTIC, wl.CUBIC, wl.QUINTIC, wl.CUBIC, wl.QUINTIC]


def iterate_with_qaq(g, table, a_of_step):
    x = g / (np.linalg.norm(g) + oracle.DEFAULT_EPS)
    a_prev = b_prev = None
    for k, (a, b, c) in enumerate(table):
        if k in (1, 3) and k <= len(table) - 2:
            q = table[a_of_step(k)][0] * np.eye(a_prev.shape[0]) + b_prev
            A = q @ a_prev @ q
        else:
            A = x @ x.T
        B = b * A + c * (A @ A)
        a_prev, b_prev = A, B
        x = a * x + B @ x
    return x


@pytest.mark.parametrize("shape", [(64, 256), (48, 200)])
@pytest.mark.parametrize("table", [[wl.QUINTIC] * 5, TABLE], ids=["quintic", "alternating"])
def test_qaq_gram_steps_reproduce_the_iteration(shape, table):
    g = np.random.default_rng(7).standard_normal(shape)
    ref = oracle.orthogonalize(g, table)
    got = iterate_with_qaq(g, table, lambda k: k - 1)
    assert oracle.relative_frobenius_error(got, ref) <= 1e-12


def test_qaq_with_the_wrong_step_coefficient_is_far_off():
    g = np.random.default_rng(8).standard_normal((64, 256))
    ref = oracle.orthogonalize(g, TABLE)
    wrong = iterate_with_qaq(g, TABLE, lambda k: k)
    assert oracle.relative_frobenius_error(wrong, ref) > 0.5

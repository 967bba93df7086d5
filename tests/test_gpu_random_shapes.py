"""A seeded sweep of ragged shapes through one muon_step each: 16 matrices
with sides drawn from 64 to 1500 (min side >= 64, so the plain bars apply),
pairs of one oriented shape in both orientations among them (one chunk, one
weight-update launch for both), bf16 and fp32 gradients, both compute
precisions; every matrix against the fp64 oracle, dW and momentum."""
import dataclasses

import numpy as np
import pytest
import torch

import muon_newton_schulz_step_amd as mn
import oracle
import workloads as wl
from gpu_helpers import BUF_TOL, announce, to64, tol

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def random_shapes(seed, count=16):
    rng = np.random.default_rng(seed)
    shapes = []
    while len(shapes) < count:
        a, b = (int(v) for v in rng.integers(64, 1501, size=2))
        shapes.append((a, b))
        if len(shapes) < count and rng.random() < 0.4:
            shapes.append((b, a))  # the same oriented shape, transposed
    return tuple(shapes)


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
@pytest.mark.parametrize("grad_dtype", [torch.bfloat16, torch.float32])
def test_random_shapes_step(compute, grad_dtype):
    seed = 100 + (compute == "fp32") * 2 + (grad_dtype == torch.float32)
    shapes = random_shapes(seed)
    announce("random shapes", compute, grad_dtype, seed, shapes)
    w = dataclasses.replace(wl.GPT_D768, shapes=shapes, grad_dtype=grad_dtype, seed=seed)
    inp = wl.make_inputs(w, device=DEV)
    before = [to64(p) for p in inp["params"]]
    bufs0 = [to64(b) for b in inp["bufs"]]
    mn.step(inp["params"], inp["grads"], inp["bufs"], mu=w.mu, lr=w.lr, scales=inp["scales"],
            coeffs=w.coeff_table, compute=compute)
    torch.cuda.synchronize()
    worst = 0.0
    for k, shape in enumerate(shapes):
        new_w, new_buf, _ = oracle.muon_step(before[k], to64(inp["grads"][k]), bufs0[k], w.mu,
                                             w.lr, inp["scales"][k], w.coeff_table)
        err = oracle.relative_frobenius_error(to64(inp["params"][k]) - before[k],
                                              new_w - before[k])
        assert oracle.relative_frobenius_error(to64(inp["bufs"][k]), new_buf) <= BUF_TOL, shape
        assert err <= tol(compute, shape), (shape, err)
        worst = max(worst, err)
    print("worst dW rel err %.3e" % worst)

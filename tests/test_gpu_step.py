"""muon_step on the GPU vs the fp64 oracle: momentum buffer, weight update
(compared as dW = W' - W) and the workloads at their real shapes."""
import dataclasses

import numpy as np
import pytest
import torch

import muon_newton_schulz_step_amd as mn
import oracle
import workloads as wl
from gpu_helpers import BUF_TOL, announce, gram_closed_form, gram_eig, normalise, to64, tol

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_step(w, inputs, compute, coeffs=None):
    params = inputs["params"]
    before = [to64(p) for p in params]
    bufs_before = [to64(b) for b in inputs["bufs"]]
    mn.step(params, inputs["grads"], inputs["bufs"], mu=w.mu, lr=w.lr,
            scales=inputs["scales"], coeffs=coeffs or w.coeff_table, compute=compute)
    torch.cuda.synchronize()
    return before, bufs_before


def check_matrix(w, inputs, k, before, bufs_before, compute, coeffs=None):
    g = to64(inputs["grads"][k])
    new_w, new_buf, _ = oracle.muon_step(before[k], g, bufs_before[k], w.mu, w.lr,
                                         inputs["scales"][k], coeffs or w.coeff_table)
    buf_err = oracle.relative_frobenius_error(to64(inputs["bufs"][k]), new_buf)
    dw_err = oracle.relative_frobenius_error(to64(inputs["params"][k]) - before[k],
                                             new_w - before[k])
    assert buf_err <= BUF_TOL, (k, buf_err)
    assert dw_err <= tol(compute, w.shapes[k]), (k, dw_err)
    return dw_err


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
@pytest.mark.parametrize("grad_dtype", [torch.bfloat16, torch.float32])
def test_step_mixed_shapes(compute, grad_dtype):
    announce("step mixed", compute, grad_dtype)
    shapes = ((64, 128), (128, 64), (100, 300), (300, 100), (64, 64), (1, 5), (5, 1),
              (257, 129), (64, 128))
    w = dataclasses.replace(wl.GPT_D768, shapes=shapes, grad_dtype=grad_dtype)
    inputs = wl.make_inputs(w, device=DEV)
    before, bufs_before = run_step(w, inputs, compute)
    for k in range(len(shapes)):
        check_matrix(w, inputs, k, before, bufs_before, compute)


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_single_256x128_workload(compute):
    announce("single 256x128", compute)
    w = wl.SINGLE_256x128
    inputs = wl.make_inputs(w, device=DEV)
    before, bufs_before = run_step(w, inputs, compute)
    check_matrix(w, inputs, 0, before, bufs_before, compute)


def test_step_deterministic_and_tall_wide_consistent():
    announce("step determinism")
    w = dataclasses.replace(wl.GPT_D768, shapes=((96, 320), (320, 96)))
    a = wl.make_inputs(w, device=DEV)
    # make the tall matrix the transpose of the wide one
    a["grads"][1] = a["grads"][0].t().contiguous()
    a["bufs"][1] = a["bufs"][0].t().contiguous()
    a["params"][1] = a["params"][0].t().contiguous()
    a["scales"] = [1.0, 1.0]
    b = {k: [t.clone() for t in v] if k != "scales" and k != "indices" else v
         for k, v in a.items()}
    for inp in (a, b):
        mn.step(inp["params"], inp["grads"], inp["bufs"], mu=w.mu, lr=w.lr,
                scales=inp["scales"], coeffs=w.coeff_table)
    torch.cuda.synchronize()
    for k in range(2):
        assert torch.equal(a["params"][k], b["params"][k])
        assert torch.equal(a["bufs"][k], b["bufs"][k])
    assert torch.equal(a["params"][0], a["params"][1].t())


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_gpt_d768_workload_full(compute):
    announce("gpt d768 full", compute)
    w = wl.GPT_D768
    inputs = wl.make_inputs(w, device=DEV)
    before, bufs_before = run_step(w, inputs, compute)
    for k in range(len(w.shapes)):
        check_matrix(w, inputs, k, before, bufs_before, compute)


def test_gpt_d1280_workload_sampled():
    announce("gpt d1280 all 120, oracle on samples")
    w = wl.GPT_D1280
    inputs = wl.make_inputs(w, device=DEV)
    before, bufs_before = run_step(w, inputs, "bf16")
    for k in wl.sample_indices(w, 1) + [len(w.shapes) - 1]:
        check_matrix(w, inputs, k, before, bufs_before, "bf16")


def test_gpt_3p8b_workload_sampled():
    # the full 168-matrix 3.8B set in the launch configuration the benchmark
    # times; the oracle checks one matrix of every raw shape
    announce("gpt 3.8b all 168, oracle on samples")
    w = wl.GPT_3P8B
    inputs = wl.make_inputs(w, device=DEV)
    samples = wl.sample_indices(w, 1) + [len(w.shapes) - 1]
    before = {k: to64(inputs["params"][k]) for k in samples}
    bufs_before = {k: to64(inputs["bufs"][k]) for k in samples}
    mn.step(inputs["params"], inputs["grads"], inputs["bufs"], mu=w.mu, lr=w.lr,
            scales=inputs["scales"], coeffs=w.coeff_table, compute="bf16")
    torch.cuda.synchronize()
    for k in samples:
        print("  oracle matrix", k, w.shapes[k], flush=True)
        check_matrix(w, inputs, k, before, bufs_before, "bf16")


def test_stress_full_shape_reduced_batch():
    # conditioning stress at its real matrix shape: one wide and one tall
    # 4096 x 16384 matrix.  Oracle = spectral closed form from the Gram
    # eigendecomposition (exact for the polynomial iteration, any size).
    announce("stress 4096x16384, 1 wide + 1 tall")
    w = dataclasses.replace(wl.STRESS_4096x16384,
                            shapes=((4096, 16384), (16384, 4096)))
    for i in range(2):
        gt = wl.make_grad(w, i, device=DEV)
        g = to64(gt)
        x0 = normalise(g if g.shape[0] <= g.shape[1] else g.T)
        eig = gram_eig(x0)
        for coeffs, compute in (([wl.QUINTIC] * 5, "bf16"), ([wl.CUBIC] * 30, "fp32")):
            o = mn.orthogonalize(gt, coeffs, compute=compute, out_dtype=torch.float32)
            torch.cuda.synchronize()
            o = to64(o)
            o = o if g.shape[0] <= g.shape[1] else o.T
            ref = gram_closed_form(x0, coeffs, eig)
            err = oracle.relative_frobenius_error(o, ref)
            print("  ", i, compute, len(coeffs), "steps rel err", err, flush=True)
            assert err <= tol(compute)
        del gt
        torch.cuda.empty_cache()


def test_refuses_tensors_off_the_device():
    # every tensor must be on the weights' GPU; a host gradient, momentum
    # buffer or workspace is refused before anything is enqueued
    announce("device checks")
    p = torch.zeros(8, 16, device=DEV)
    g = torch.zeros(8, 16, dtype=torch.bfloat16, device=DEV)
    b = torch.zeros(8, 16, device=DEV)
    for kw in (dict(grads=[g.cpu()]), dict(bufs=[b.cpu()]),
               dict(workspace=torch.empty(1 << 20, dtype=torch.uint8))):
        args = dict(params=[p], grads=[g], bufs=[b])
        args.update({k: v for k, v in kw.items() if k != "workspace"})
        with pytest.raises(ValueError):
            mn.step(args["params"], args["grads"], args["bufs"], mu=0.95, lr=0.02,
                    workspace=kw.get("workspace"))
    with pytest.raises(ValueError):
        mn.orthogonalize(g, out=torch.empty(8, 16))
    assert torch.count_nonzero(p) == 0 and torch.count_nonzero(b) == 0

"""muon_step on the GPU vs the fp64 oracle: momentum buffer, weight update
(compared as dW = W' - W) and the workloads at their real shapes."""
import dataclasses

import numpy as np
import pytest
import torch

import muon_newton_schulz_step_amd as mn
import oracle
import workloads as wl
from gpu_helpers import (BUF_TOL, announce, check_tiles, gram_closed_form, gram_eig, normalise,
                         scalar_map, to64, tol)

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


def check_matrix(w, inputs, k, before, bufs_before, compute, coeffs=None, tiles=False):
    g = to64(inputs["grads"][k])
    new_w, new_buf, _ = oracle.muon_step(before[k], g, bufs_before[k], w.mu, w.lr,
                                         inputs["scales"][k], coeffs or w.coeff_table)
    buf_err = oracle.relative_frobenius_error(to64(inputs["bufs"][k]), new_buf)
    dw_err = oracle.relative_frobenius_error(to64(inputs["params"][k]) - before[k],
                                             new_w - before[k])
    assert buf_err <= BUF_TOL, (k, buf_err)
    assert dw_err <= tol(compute, w.shapes[k]), (k, dw_err)
    if tiles:
        check_tiles(to64(inputs["params"][k]) - before[k], new_w - before[k],
                    tol(compute, w.shapes[k]), k)
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


@pytest.mark.parametrize("n_steps", [1, 2, 3])
@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_step_few_newton_schulz_steps(compute, n_steps):
    """The first step is also the last (the normalisation folded into the
    Gram and the weight update of one launch pair), two steps, and three,
    whose step 1 forms the 2048x8192 group's Gram matrix as Q A Q on the
    bf16 path."""
    announce("few NS steps", compute, n_steps)
    shapes = ((96, 256), (256, 96), (300, 700), (2048, 8192))
    w = dataclasses.replace(wl.GPT_D768, shapes=shapes)
    coeffs = w.coeff_table[:n_steps]
    inputs = wl.make_inputs(w, device=DEV)
    before, bufs_before = run_step(w, inputs, compute, coeffs=coeffs)
    for k in range(len(shapes)):
        check_matrix(w, inputs, k, before, bufs_before, compute, coeffs=coeffs)


def test_step_final_parts_with_their_own_tiles():
    """One oriented chunk of 32 wide 512x2048 matrices and one tall 2048x512:
    the wide part's weight update runs on 256x256 tiles (512 of them), the
    tall part's alone on 128x128 tiles."""
    announce("step final parts, different tiles")
    shapes = ((512, 2048),) * 32 + ((2048, 512),)
    w = dataclasses.replace(wl.GPT_D768, shapes=shapes)
    inputs = wl.make_inputs(w, device=DEV)
    before, bufs_before = run_step(w, inputs, "bf16")
    for k in (0, 17, 31, 32):
        check_matrix(w, inputs, k, before, bufs_before, "bf16", tiles=True)


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
        check_matrix(w, inputs, k, before, bufs_before, "bf16", tiles=True)


def test_stress_full_chunk_step():
    """The conditioning-stress workload as the benchmark times it: one
    muon_step over all 64 wide and 64 tall 4096 x 16384 matrices (two chunks
    of 64, Q A Q Gram steps, streamed X state).  Two matrices per orientation
    are checked against the spectral closed form (from the Gram matrix's
    eigendecomposition; exact for the polynomial iteration at any size), as
    a whole and tile by tile, with the momentum against the oracle's."""
    w = wl.STRESS_4096x16384
    announce("stress 4096x16384, all 128 in one step (~120 GB)")
    inputs = wl.make_inputs(w, device=DEV)
    samples = [0, 63, 64, 127]
    before = {k: to64(inputs["params"][k]) for k in samples}
    bufs_before = {k: to64(inputs["bufs"][k]) for k in samples}
    mn.step(inputs["params"], inputs["grads"], inputs["bufs"], mu=w.mu, lr=w.lr,
            scales=inputs["scales"], coeffs=w.coeff_table, compute="bf16")
    torch.cuda.synchronize()
    for k in samples:
        g = to64(inputs["grads"][k])
        new_buf, u = oracle.nesterov_momentum(g, bufs_before[k], w.mu)
        assert oracle.relative_frobenius_error(to64(inputs["bufs"][k]), new_buf) <= BUF_TOL
        tall = u.shape[0] > u.shape[1]
        x0 = normalise(u.T if tall else u)
        o = gram_closed_form(x0, w.coeff_table)
        o = o.T if tall else o
        dw_ref = -w.lr * inputs["scales"][k] * o
        dw = to64(inputs["params"][k]) - before[k]
        err = oracle.relative_frobenius_error(dw, dw_ref)
        worst = check_tiles(dw, dw_ref, tol("bf16"), k)
        print("  matrix", k, "tall" if tall else "wide", "dW rel err %.3e, worst tile %.3e"
              % (err, worst), flush=True)
        assert err <= tol("bf16"), (k, err)
        del g, u, x0, o, dw, dw_ref


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
            if compute == "bf16":
                check_tiles(o, ref, tol(compute), i)
            else:
                polar_distance_report(o, ref, x0, eig, coeffs, i)
        del gt
        torch.cuda.empty_cache()


def polar_distance_report(o, o_cf, x0, eig, coeffs, i):
    """The web3.cnoyu.systems review of karpathy/autoresearch's train.py (Muon
    paragraph) names the orthogonal factor U of G = U S as the target.  For the
    bf16-rounded G fed here, that factor is P = G (G^T G)^(-1/2) (from the
    Gram eigendecomposition); 30 cubic steps leave directions with tiny
    normalised singular values s unconverged, so O is not P: ||O - P||_F is
    predicted in closed form as ||phi_30(s) - 1||_2 (O = U phi(S) V^T,
    P = U V^T).  The measured distance must match the prediction within what
    separates O from the closed form (the fp32 bound)."""
    lam, v = eig
    s = np.sqrt(np.maximum(lam, 0.0))
    assert s.min() > 0.0
    p = (v / s) @ (v.T @ x0)
    m = x0.shape[0]
    pred = float(np.linalg.norm(scalar_map(s, coeffs) - 1.0)) / np.sqrt(m)
    meas = float(np.linalg.norm(o - p)) / float(np.linalg.norm(p))
    slack = float(np.linalg.norm(o - o_cf)) / float(np.linalg.norm(p))
    print("   matrix %d: ||O - UV^T|| / ||UV^T|| measured %.6e, predicted %.6e "
          "(smallest normalised singular value %.3e)" % (i, meas, pred, s.min()), flush=True)
    assert abs(meas - pred) <= slack + 1e-9
    assert slack <= 1e-4


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


def test_non_finite_values_propagate_like_the_oracle():
    """One NaN gradient element and one infinite weight, in two different
    matrices of one call: NaN exactly where the oracle has NaN (the momentum
    at that element, all of that matrix's new weights), the infinite weight
    stays infinite and leaves the rest of its matrix bitwise as in a clean
    run (its direction does not depend on W), and the third matrix is
    bitwise unchanged by the others' non-finite values."""
    announce("non-finite propagation")
    w = dataclasses.replace(wl.GPT_D768, shapes=((96, 256), (256, 96), (128, 128)))
    clean = wl.make_inputs(w, device=DEV)
    dirty = {k: ([t.clone() for t in v] if k in ("params", "grads", "bufs") else v)
             for k, v in clean.items()}
    dirty["grads"][0][5, 7] = float("nan")
    dirty["params"][1][3, 2] = float("inf")
    ref_in = {k: [to64(t) for t in dirty[k]] for k in ("params", "grads", "bufs")}
    for inp in (clean, dirty):
        mn.step(inp["params"], inp["grads"], inp["bufs"], mu=w.mu, lr=w.lr,
                scales=inp["scales"], coeffs=w.coeff_table, compute="bf16")
    torch.cuda.synchronize()
    for k in range(3):
        new_w, new_buf, _ = oracle.muon_step(ref_in["params"][k], ref_in["grads"][k],
                                             ref_in["bufs"][k], w.mu, w.lr, dirty["scales"][k],
                                             w.coeff_table)
        got_w, got_buf = to64(dirty["params"][k]), to64(dirty["bufs"][k])
        assert np.array_equal(np.isnan(got_w), np.isnan(new_w)), k
        assert np.array_equal(np.isnan(got_buf), np.isnan(new_buf)), k
        assert np.array_equal(np.isinf(got_w), np.isinf(new_w)), k
    assert torch.isnan(dirty["params"][0]).all()
    assert torch.isnan(dirty["bufs"][0]).sum() == 1
    keep = torch.ones_like(dirty["bufs"][0], dtype=torch.bool)
    keep[5, 7] = False
    assert torch.equal(dirty["bufs"][0][keep], clean["bufs"][0][keep])
    assert dirty["params"][1][3, 2] == float("inf")
    keep = torch.ones_like(dirty["params"][1], dtype=torch.bool)
    keep[3, 2] = False
    assert torch.equal(dirty["params"][1][keep], clean["params"][1][keep])
    assert torch.equal(dirty["params"][2], clean["params"][2])
    assert torch.equal(dirty["bufs"][2], clean["bufs"][2])


def test_shared_gradient_and_aliasing_refused():
    """Gradients are only read, so two matrices may take the same gradient
    tensor: the result is bitwise that of two separate copies.  A weight
    tensor passed for two matrices is refused before anything runs."""
    announce("shared gradient")
    w = dataclasses.replace(wl.GPT_D768, shapes=((300, 700), (300, 700), (700, 300)))
    a = wl.make_inputs(w, device=DEV)
    b = {k: ([t.clone() for t in v] if k in ("params", "bufs") else v) for k, v in a.items()}
    shared = [a["grads"][0], a["grads"][0], a["grads"][2]]
    copies = [a["grads"][0].clone(), a["grads"][0].clone(), a["grads"][2]]
    for inp, grads in ((a, shared), (b, copies)):
        mn.step(inp["params"], grads, inp["bufs"], mu=w.mu, lr=w.lr, scales=inp["scales"],
                coeffs=w.coeff_table, compute="bf16")
    torch.cuda.synchronize()
    for x, y in zip(a["params"] + a["bufs"], b["params"] + b["bufs"]):
        assert torch.equal(x, y)
    kept = [p.clone() for p in a["params"]]
    with pytest.raises(mn.MuonError) as err:
        mn.step([a["params"][0], a["params"][0]], shared[:2], a["bufs"][:2], mu=w.mu,
                lr=w.lr, compute="bf16")
    assert err.value.status == mn.MUON_ERR_INVALID_ARG
    torch.cuda.synchronize()
    for x, y in zip(a["params"], kept):
        assert torch.equal(x, y)


@pytest.mark.skipif(torch.cuda.device_count() < 2, reason="needs a second GPU for a stream "
                    "that belongs to another device")
def test_stream_of_another_device_refused():
    """The step works on the calling thread's current device (its stream
    lanes and static scratch live there): with device 0 current, a stream of
    device 1 returns MUON_ERR_INVALID_ARG and nothing is written."""
    announce("stream of another device")
    from muon_newton_schulz_step_amd import _lib
    torch.cuda.set_device(0)
    rows, cols = 64, 128
    p = torch.zeros(rows, cols, device=DEV)
    g = torch.ones(rows, cols, device=DEV, dtype=torch.bfloat16)
    b = torch.zeros(rows, cols, device=DEV)
    lib = mn.lib()
    need = lib.muon_step_workspace_bytes(1, _lib.int_array([rows]), _lib.int_array([cols]), 0)
    ws = torch.empty(need + 256, dtype=torch.uint8, device=DEV)
    wp = (ws.data_ptr() + 255) // 256 * 256
    other = torch.cuda.Stream(device=1)
    for call in (lambda s: lib.muon_step(
            1, _lib.int_array([rows]), _lib.int_array([cols]), _lib.ptr_array([p.data_ptr()]),
            _lib.MUON_FP32, _lib.ptr_array([g.data_ptr()]), _lib.MUON_BF16,
            _lib.ptr_array([b.data_ptr()]), 0.95, 0.02, _lib.float_array([1.0]),
            _lib.coeff_array([wl.QUINTIC] * 5), 5, 1e-7, 0, wp, need, s),
                 lambda s: lib.muon_step_static(
            1, _lib.int_array([rows]), _lib.int_array([cols]), _lib.ptr_array([p.data_ptr()]),
            _lib.MUON_FP32, _lib.ptr_array([g.data_ptr()]), _lib.MUON_BF16,
            _lib.ptr_array([b.data_ptr()]), 0.95, 0.02, _lib.float_array([1.0]),
            _lib.coeff_array([wl.QUINTIC] * 5), 5, 1e-7, 0, s)):
        assert call(other.cuda_stream) == _lib.MUON_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(p == 0) and torch.all(b == 0)

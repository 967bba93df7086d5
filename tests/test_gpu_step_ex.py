"""muon_step_ex on the GPU vs the fp64 oracle: the cautious weight decay and
NorMuon scaling of the web3.cnoyu.systems review of karpathy/autoresearch's
train.py (paragraph after the Muon one) on top of the plain step, mixed shapes (tall,
wide, square, ragged), both compute precisions, and the second-moment
moving average carried over two steps.

The cautious mask is a sign decision on O'*W.  The GPU's own direction O'
is read from a twin call without decay on copies of the same state (the
same kernels, so the same O'); where it and the oracle's O' differ in sign
(|O'_ref| within the GPU's measured error of that element) both decisions
are correct, and the comparison takes the oracle's value for whichever
decision the GPU made; the magnitude part (-lr*scale*O') is still compared.
Everywhere else the mask must agree with the oracle's."""
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
SHAPES = ((64, 128), (128, 64), (100, 300), (300, 100), (64, 64), (1, 5), (5, 1),
          (257, 129), (64, 128), (256, 768), (768, 256))


def expected_dw(ref, w_before, dw_gpu, lr, scale, wd, cautious, o_gpu):
    """Oracle dW, with the cautious mask taken from the GPU where the GPU's
    direction o_gpu and the oracle's differ in sign (both decisions are
    correct there); the fp32 rounding of the recovered o_gpu is allowed for."""
    o, w = ref["o"], w_before
    dw_keep = -lr * scale * o
    dw_decay = dw_keep - lr * wd * w
    if not cautious or wd == 0:
        return dw_decay
    mask = o * w >= 0
    dw = np.where(mask, dw_decay, dw_keep)
    slack = 4.0 * np.spacing(np.abs(w).astype(np.float32)) / (lr * scale)
    amb = np.abs(o) <= np.abs(o_gpu - o) + slack
    closer = np.where(np.abs(dw_gpu - dw_decay) <= np.abs(dw_gpu - dw_keep), dw_decay, dw_keep)
    return np.where(amb, closer, dw)


def gpu_direction(w, inp, vs, indices, **call):
    """The update direction O' the GPU applies, for matrices ``indices``: the
    same step_ex call without weight decay on copies of the weights,
    momentum and second moments, read back from its weight change."""
    params = [p.clone() for p in inp["params"]]
    bufs = [b.clone() for b in inp["bufs"]]
    vv = [v.clone() for v in vs] if vs is not None else None
    before = {k: to64(params[k]) for k in indices}
    mn.step_ex(params, inp["grads"], bufs, mu=w.mu, lr=w.lr, scales=inp["scales"],
               coeffs=w.coeff_table, second_moments=vv, **{**call, "weight_decay": 0.0})
    torch.cuda.synchronize()
    out = {k: (to64(params[k]) - before[k]) / (-w.lr * inp["scales"][k]) for k in indices}
    del params, bufs, vv
    return out


def run_case(compute, wd, cautious, normuon, steps=1, shapes=SHAPES, beta2=0.9,
             normuon_eps=1e-8, ns_steps=5):
    announce("step_ex", compute, wd, cautious, normuon, steps, ns_steps)
    w = dataclasses.replace(wl.GPT_D768, shapes=shapes, n_steps=ns_steps)
    inp = wl.make_inputs(w, device=DEV)
    vs = [wl.make_second_moment(w, i, device=DEV) for i in range(len(shapes))] if normuon else None
    state = [dict(w=to64(inp["params"][k]), buf=to64(inp["bufs"][k]),
                  v=to64(vs[k]) if normuon else None) for k in range(len(shapes))]
    for step in range(steps):
        before = [to64(p) for p in inp["params"]]
        call = dict(compute=compute, cautious=cautious, beta2=beta2 if normuon else None,
                    normuon_eps=normuon_eps if normuon else None)
        o_gpu = (gpu_direction(w, inp, vs, range(len(shapes)), **call)
                 if cautious and wd > 0 else {})
        mn.step_ex(inp["params"], inp["grads"], inp["bufs"], mu=w.mu, lr=w.lr,
                   scales=inp["scales"], coeffs=w.coeff_table, second_moments=vs,
                   weight_decay=wd, **call)
        torch.cuda.synchronize()
        for k, shape in enumerate(shapes):
            g = to64(inp["grads"][k])
            st = state[k]
            ref = oracle.muon_step_ex(before[k], g, st["buf"], w.mu, w.lr, inp["scales"][k],
                                      w.coeff_table, weight_decay=wd, cautious=cautious,
                                      second_moment=st["v"] if normuon else None,
                                      beta2=beta2, normuon_eps=normuon_eps)
            t = tol(compute, shape)
            dw_gpu = to64(inp["params"][k]) - before[k]
            dw_ref = expected_dw(ref, before[k], dw_gpu, w.lr, inp["scales"][k], wd, cautious,
                                 o_gpu.get(k))
            err = oracle.relative_frobenius_error(dw_gpu, dw_ref)
            assert err <= t, (step, shape, err)
            assert oracle.relative_frobenius_error(to64(inp["bufs"][k]), ref["buf"]) <= BUF_TOL
            if normuon:
                v_err = oracle.relative_frobenius_error(to64(vs[k]), ref["v"])
                assert v_err <= 2 * t, (step, shape, v_err)
                st["v"] = to64(vs[k])  # carry the GPU's state, as the caller would
            st["buf"] = to64(inp["bufs"][k])


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
@pytest.mark.parametrize("cautious", [True, False])
def test_weight_decay(compute, cautious):
    run_case(compute, wd=0.5, cautious=cautious, normuon=False)


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_normuon(compute):
    run_case(compute, wd=0.0, cautious=True, normuon=True)


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_normuon_with_cautious_decay_two_steps(compute):
    run_case(compute, wd=0.5, cautious=True, normuon=True, steps=2, beta2=0.75)


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_normuon_cautious_decay_one_newton_schulz_step(compute):
    # the row statistics and the decay taken from the first step's update,
    # which is also the last
    run_case(compute, wd=0.5, cautious=True, normuon=True, ns_steps=1)


def test_normuon_beta2_one_keeps_state_and_zero_eps():
    # beta2 = 1: v stays as given; the update is O / sqrt(v) row by row
    run_case("fp32", wd=0.0, cautious=True, normuon=True, beta2=1.0, normuon_eps=0.0,
             shapes=((64, 192), (192, 64)))


def test_step_ex_without_options_is_the_plain_step():
    announce("step_ex equals step")
    w = dataclasses.replace(wl.GPT_D768, shapes=((100, 300), (300, 100)))
    a = wl.make_inputs(w, device=DEV)
    b = wl.make_inputs(w, device=DEV)
    mn.step(a["params"], a["grads"], a["bufs"], mu=w.mu, lr=w.lr, scales=a["scales"],
            coeffs=w.coeff_table)
    mn.step_ex(b["params"], b["grads"], b["bufs"], mu=w.mu, lr=w.lr, scales=b["scales"],
               coeffs=w.coeff_table, weight_decay=0.0)
    torch.cuda.synchronize()
    for x, y in zip(a["params"] + a["bufs"], b["params"] + b["bufs"]):
        assert torch.equal(x, y)


def test_gpt_3p8b_step_ex_sampled():
    # the full 168-matrix 3.8B set through muon_step_ex with NorMuon and
    # cautious decay (the bench's normuon_cwd variant); the oracle checks one
    # matrix of every raw shape, weights and second moments
    announce("gpt 3.8b all 168, step_ex normuon + cautious decay, oracle on samples")
    w = wl.GPT_3P8B
    inp = wl.make_inputs(w, device=DEV)
    vs = [wl.make_second_moment(w, i, device=DEV) for i in range(len(w.shapes))]
    samples = wl.sample_indices(w, 1) + [len(w.shapes) - 1]
    before = {k: to64(inp["params"][k]) for k in samples}
    bufs = {k: to64(inp["bufs"][k]) for k in samples}
    v0 = {k: to64(vs[k]) for k in samples}
    opt = dict(weight_decay=0.1, cautious=True, beta2=0.95, normuon_eps=1e-8)
    o_gpu = gpu_direction(w, inp, vs, samples, compute="bf16", cautious=True, beta2=0.95,
                          normuon_eps=1e-8)
    mn.step_ex(inp["params"], inp["grads"], inp["bufs"], mu=w.mu, lr=w.lr,
               scales=inp["scales"], coeffs=w.coeff_table, compute="bf16",
               second_moments=vs, **opt)
    torch.cuda.synchronize()
    amb_frac = []
    for k in samples:
        print("  oracle matrix", k, w.shapes[k], flush=True)
        ref = oracle.muon_step_ex(before[k], to64(inp["grads"][k]), bufs[k], w.mu, w.lr,
                                  inp["scales"][k], w.coeff_table, second_moment=v0[k], **opt)
        t = tol("bf16", w.shapes[k])
        dw_gpu = to64(inp["params"][k]) - before[k]
        dw_ref = expected_dw(ref, before[k], dw_gpu, w.lr, inp["scales"][k], 0.1, True,
                             o_gpu[k])
        amb_frac.append(float(np.mean(np.abs(ref["o"]) <= np.abs(o_gpu[k] - ref["o"]))))
        assert oracle.relative_frobenius_error(dw_gpu, dw_ref) <= t, k
        assert oracle.relative_frobenius_error(to64(inp["bufs"][k]), ref["buf"]) <= BUF_TOL
        assert oracle.relative_frobenius_error(to64(vs[k]), ref["v"]) <= 2 * t
    # the sign of O' is in doubt (either mask decision valid) for few elements
    print("  elements with either mask decision valid:", amb_frac, flush=True)
    assert max(amb_frac) <= 0.02


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_normuon_row_statistics_match_the_applied_update(compute):
    """Each oriented row's second moment is the moving average of the mean
    square of exactly the direction the same call applied to that row.

    Without weight decay the call moves W by -lr*scale*O[i]/(sqrt(v'[i]) + eps),
    so O is recovered from the weights and v' (to ~1e-7), and the mean of its
    squares along the row must give v'.  This pins the row statistics at the
    arithmetic's precision (the bf16 path sums the update's fp32 values, the
    weights get its 16-bit hi + lo form: 2^-16 apart at most), where the
    comparison with the oracle only bounds them by the Newton-Schulz error.
    Eight 1024x4096 matrices run on 256-wide tiles (64 column blocks per
    row), the ragged 300x1000 pair (one wide, one tall) on 128-wide ones."""
    shapes = ((1024, 4096),) * 8 + ((300, 1000), (1000, 300))
    beta2, eps = 0.5, 1e-8
    announce("normuon row statistics", compute, shapes)
    w = dataclasses.replace(wl.GPT_D768, shapes=shapes)
    inp = wl.make_inputs(w, device=DEV)
    vs = [wl.make_second_moment(w, i, device=DEV) for i in range(len(shapes))]
    v0 = [to64(v) for v in vs]
    before = [to64(p) for p in inp["params"]]
    mn.step_ex(inp["params"], inp["grads"], inp["bufs"], mu=w.mu, lr=w.lr,
               scales=inp["scales"], coeffs=w.coeff_table, compute=compute,
               weight_decay=0.0, cautious=False, second_moments=vs, beta2=beta2,
               normuon_eps=eps)
    torch.cuda.synchronize()
    for k, (r, c) in enumerate(shapes):
        dw = to64(inp["params"][k]) - before[k]
        if r > c:
            dw = dw.T  # oriented: rows along the shorter side
        v1 = to64(vs[k])
        o = dw * (np.sqrt(v1) + eps)[:, None] / (-w.lr * inp["scales"][k])
        mean_sq = np.mean(o ** 2, axis=1)
        mean_gpu = (v1 - beta2 * v0[k]) / (1.0 - beta2)
        rel = np.abs(mean_gpu - mean_sq) / mean_sq
        assert rel.max() <= 1e-4, (k, (r, c), float(rel.max()), int(rel.argmax()))


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_normuon_zero_eps_zero_row_is_non_finite_like_the_oracle(compute):
    """normuon_eps = 0 with a zero second moment and a gradient whose row 5
    (wide) or column 5 (tall) is zero: that line of O stays exactly zero
    through the iteration, v' is 0 and the scaling divides 0 by 0.  The new
    weights are non-finite on exactly that line, as in the oracle; the other
    lines agree with the oracle to the usual bar."""
    announce("normuon eps 0, zero row", compute)
    shapes = ((64, 192), (192, 64))
    w = dataclasses.replace(wl.GPT_D768, shapes=shapes)
    inp = wl.make_inputs(w, device=DEV)
    inp["grads"][0][5, :] = 0
    inp["grads"][1][:, 5] = 0
    inp["bufs"] = [torch.zeros_like(b) for b in inp["bufs"]]
    vs = [torch.zeros(min(s), device=DEV) for s in shapes]
    before = [to64(p) for p in inp["params"]]
    mn.step_ex(inp["params"], inp["grads"], inp["bufs"], mu=w.mu, lr=w.lr,
               scales=inp["scales"], coeffs=w.coeff_table, compute=compute,
               weight_decay=0.0, cautious=False, second_moments=vs, beta2=0.9,
               normuon_eps=0.0)
    torch.cuda.synchronize()
    for k, shape in enumerate(shapes):
        with np.errstate(invalid="ignore", divide="ignore"):
            ref = oracle.muon_step_ex(before[k], to64(inp["grads"][k]), np.zeros(shape), w.mu,
                                      w.lr, inp["scales"][k], w.coeff_table, weight_decay=0.0,
                                      cautious=False, second_moment=np.zeros(min(shape)),
                                      beta2=0.9, normuon_eps=0.0)
        got = to64(inp["params"][k])
        bad_ref, bad_got = ~np.isfinite(ref["w"]), ~np.isfinite(got)
        assert bad_ref.any() and np.array_equal(bad_ref, bad_got), (shape, bad_got.sum())
        line = (slice(5, 6), slice(None)) if k == 0 else (slice(None), slice(5, 6))
        assert bad_got[line].all() and bad_got.sum() == bad_got[line].size
        ok = np.isfinite(ref["w"])
        err = oracle.relative_frobenius_error(got[ok] - before[k][ok], ref["w"][ok] - before[k][ok])
        assert err <= tol(compute, shape), (shape, err)


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_random_shapes_normuon_cautious(compute):
    """The seeded sweep of ragged shapes (test_gpu_random_shapes) through
    muon_step_ex with NorMuon and cautious decay."""
    from test_gpu_random_shapes import random_shapes
    run_case(compute, wd=0.1, cautious=True, normuon=True,
             shapes=random_shapes(200 + (compute == "fp32"), count=10))

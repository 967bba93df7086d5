"""muon_orthogonalize on the GPU vs the fp64 oracle, element by element.

Shapes span one tile, several tiles and ragged tails in both dimensions,
tall, wide and square, batches, both compute precisions and both I/O dtypes.
"""
import numpy as np
import pytest
import torch

import muon_newton_schulz_step_amd as mn
import oracle
import workloads as wl
from gpu_helpers import announce, check_tiles, gram_closed_form, normalise, to64, tol

pytestmark = pytest.mark.gpu
Q5 = [wl.QUINTIC] * 5
DEV = "cuda:0"

SHAPES = [(1, 1), (2, 8), (8, 2), (5, 5), (16, 8), (128, 128), (128, 256), (256, 128),
          (257, 129), (129, 257), (300, 700), (700, 300), (384, 384), (130, 1000)]


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}x{s[1]}")
def test_orthogonalize_matches_oracle(shape, compute):
    announce("orthogonalize", shape, compute)
    x = wl.gaussian_matrix(*shape, seed=shape[0] * 7919 + shape[1], device=DEV)
    o = mn.orthogonalize(x, Q5, compute=compute, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.orthogonalize(to64(x), Q5)
    err = oracle.relative_frobenius_error(to64(o), ref)
    assert err <= tol(compute, shape), err


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
@pytest.mark.parametrize("in_dtype,out_dtype", [(torch.bfloat16, torch.bfloat16),
                                                (torch.bfloat16, torch.float32),
                                                (torch.float32, torch.bfloat16)])
def test_batch_and_dtypes(compute, in_dtype, out_dtype):
    announce("batch", compute, in_dtype, out_dtype)
    x = wl.gaussian_batch(5, 96, 200, seed=3, device=DEV, dtype=in_dtype)
    o = mn.orthogonalize(x, Q5, compute=compute, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert o.dtype == out_dtype
    # bf16 output adds one rounding of |O| ~ 0.1 (relative 2^-9)
    extra = 4e-3 if out_dtype == torch.bfloat16 else 0.0
    for b in range(5):
        ref = oracle.orthogonalize(to64(x[b]), Q5)
        err = oracle.relative_frobenius_error(to64(o[b]), ref)
        assert err <= tol(compute) + extra, (b, err)


def test_batch_larger_than_one_chunk():
    announce("batch 70 (two chunks)")
    x = wl.gaussian_batch(70, 40, 24, seed=4, device=DEV)
    o = mn.orthogonalize(x, Q5, compute="fp32", out_dtype=torch.float32)
    torch.cuda.synchronize()
    for b in (0, 63, 64, 69):
        ref = oracle.orthogonalize(to64(x[b]), Q5)
        assert oracle.relative_frobenius_error(to64(o[b]), ref) <= 1e-4


def test_in_place():
    announce("in place")
    x = wl.gaussian_batch(2, 64, 160, seed=5, device=DEV)
    ref = [oracle.orthogonalize(to64(x[b]), Q5) for b in range(2)]
    mn.orthogonalize(x, Q5, compute="fp32", out=x)
    torch.cuda.synchronize()
    for b in range(2):
        assert oracle.relative_frobenius_error(to64(x[b]), ref[b]) <= 1e-4


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_in_place_across_chunks(compute, dtype):
    # 70 tall matrices run as two chunks (64 + 6); writing each chunk's
    # output over its own input gives bitwise the out-of-place result
    announce("in place across chunks", compute, dtype)
    x = wl.gaussian_batch(70, 96, 40, seed=8, device=DEV).to(dtype)
    o = mn.orthogonalize(x, Q5, compute=compute, out_dtype=dtype)
    mn.orthogonalize(x, Q5, compute=compute, out=x)
    torch.cuda.synchronize()
    assert torch.equal(x, o)


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_transpose_equivalence_is_bitwise(compute):
    # a tall matrix runs the same oriented kernels on the same data as its
    # transpose, so the outputs agree bit for bit
    announce("transpose equivalence", compute)
    x = wl.gaussian_matrix(320, 96, seed=6, device=DEV)
    o_tall = mn.orthogonalize(x, Q5, compute=compute)
    o_wide = mn.orthogonalize(x.t().contiguous(), Q5, compute=compute)
    torch.cuda.synchronize()
    assert torch.equal(o_tall, o_wide.t())


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_deterministic(compute):
    announce("determinism", compute)
    x = wl.gaussian_batch(3, 200, 520, seed=7, device=DEV)
    a = mn.orthogonalize(x, Q5, compute=compute)
    b = mn.orthogonalize(x, Q5, compute=compute)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_zero_input_gives_zero(compute):
    announce("zero input", compute)
    x = torch.zeros((3, 40, 70), device=DEV)
    o = mn.orthogonalize(x, Q5, compute=compute)
    torch.cuda.synchronize()
    assert torch.count_nonzero(o) == 0


def test_per_step_table_and_step_counts():
    announce("per-step table")
    table = [(3.4445, -4.7750, 2.0315), (1.5, -0.5, 0.0), (2.0, -1.5, 0.5),
             (1.875, -1.25, 0.375)]
    x = wl.gaussian_matrix(100, 260, seed=8, device=DEV)
    for coeffs in (table, table[:1], [wl.CUBIC] * 64):
        o = mn.orthogonalize(x, coeffs, compute="fp32")
        torch.cuda.synchronize()
        ref = oracle.orthogonalize(to64(x), coeffs)
        assert oracle.relative_frobenius_error(to64(o), ref) <= 1e-4


@pytest.mark.parametrize("shape", [(1, 1), (2, 8), (8, 2), (3, 4), (4, 3), (5, 5), (16, 8)])
def test_cubic_reaches_polar_factor(shape):
    announce("cubic polar factor", shape)
    rng = np.random.default_rng(shape[0] * 31 + shape[1])
    k = min(shape)
    u, _ = np.linalg.qr(rng.standard_normal((shape[0], k)))
    v, _ = np.linalg.qr(rng.standard_normal((shape[1], k)))
    g = (u * np.exp(rng.uniform(np.log(1e-2), 0.0, k))) @ v.T
    x = torch.tensor(g, dtype=torch.float32, device=DEV)
    o = mn.orthogonalize(x, [wl.CUBIC] * 40, compute="fp32")
    torch.cuda.synchronize()
    uu, _, vt = np.linalg.svd(to64(x), full_matrices=False)
    # fp32 arithmetic: 1e-6 is the fp64 oracle's bound; the GPU gets fp32's
    assert np.max(np.abs(to64(o) - uu @ vt)) <= 2e-5


def test_quintic_band_single_256x128():
    announce("quintic band 256x128")
    x = wl.make_grad(wl.SINGLE_256x128, 0, device=DEV)
    for compute in ("bf16", "fp32"):
        o = mn.orthogonalize(x, Q5, compute=compute)
        torch.cuda.synchronize()
        sv = np.linalg.svd(to64(o), compute_uv=False)
        assert sv.min() >= 0.5 and sv.max() <= 1.5


def test_scale_invariance():
    announce("scale invariance")
    x = wl.gaussian_matrix(64, 192, seed=9, device=DEV)
    base = to64(mn.orthogonalize(x, Q5, compute="fp32"))
    for alpha in (1e-3, 1e3, -1.0):
        o = to64(mn.orthogonalize(x * alpha, Q5, compute="fp32"))
        assert oracle.relative_frobenius_error(o, np.sign(alpha) * base) <= 1e-4


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_magnitude_range(compute):
    """The normalisation is folded into the first Gram and update epilogues,
    so X_0 is stored unnormalised and the first Gram accumulates products of
    raw entries in fp32.  Entries from 2^-60 (8.7e-19) to 2^55 (3.6e16), K =
    192: each against the oracle on the same scaled input.  At 2^-60 the norm
    is far below eps = 1e-7, so X_0 = u / (||u|| + eps) is tiny and the
    iteration runs in its linear range, in the oracle as on the GPU."""
    announce("magnitude range", compute)
    x = wl.gaussian_matrix(64, 192, seed=19, device=DEV)
    for k in (-60, -30, 30, 55):
        xs = x * (2.0 ** k)  # exact: a power of two
        o = to64(mn.orthogonalize(xs, Q5, compute=compute))
        ref = oracle.orthogonalize(to64(xs), Q5)
        err = oracle.relative_frobenius_error(o, ref)
        print(compute, k, "%.3e" % err)
        assert err <= tol(compute, (64, 192)), (k, err)


@pytest.mark.parametrize("shape", [(200, 520), (520, 200)], ids=["wide", "tall"])
@pytest.mark.parametrize("n_steps", [1, 3])
def test_x_state_holds_sixteen_bits(shape, n_steps):
    """With the coefficients (1, 0, 0) every Newton-Schulz step gives X back
    (a X + (0 A + 0 A^2) X), so the bf16 path's output is the normalised
    fp32 input as carried by its X state: prep encodes it once, every further
    update re-encodes it, the last one decodes it.  Each encoding keeps 16
    significant bits (hi = bf16(x) and a signed byte of 1/256 of hi's
    spacing: relative error at most 2^-16, 2^-15 where the byte saturates),
    so every element is within n_steps * 2^-15 of the oracle's u / (||u|| +
    eps), plus fp32 rounding.  A state that kept hi alone would be off by up
    to 2^-9."""
    announce("X state precision", shape, n_steps)
    x = wl.gaussian_matrix(*shape, seed=23, device=DEV)
    ident = [(1.0, 0.0, 0.0)] * n_steps
    o = to64(mn.orthogonalize(x, ident, compute="bf16", out_dtype=torch.float32))
    ref = oracle.orthogonalize(to64(x), ident)
    assert np.allclose(ref, normalise(to64(x)), rtol=1e-15, atol=0)
    rel = np.abs(o - ref) / np.abs(ref)
    print("max relative error per element %.3e" % rel.max())
    assert rel.max() <= n_steps * 2.0 ** -15 + 8 * 2.0 ** -24
    # the low part carries information: hi alone is much further off
    hi_only = to64(torch.from_numpy(ref).float().to(torch.bfloat16))
    assert (np.abs(hi_only - ref) / np.abs(ref)).max() > 16 * rel.max()


def test_permutation_invariance():
    announce("permutation invariance")
    x = wl.gaussian_matrix(200, 330, seed=10, device=DEV)
    g = torch.Generator(device="cpu").manual_seed(1)
    pr, pc = torch.randperm(200, generator=g), torch.randperm(330, generator=g)
    o = mn.orthogonalize(x, Q5, compute="bf16")
    op = mn.orthogonalize(x[pr][:, pc].contiguous(), Q5, compute="bf16")
    torch.cuda.synchronize()
    assert oracle.relative_frobenius_error(to64(op), to64(o[pr][:, pc])) <= 2e-2


def test_stress_logspec_reduced_size():
    # conditioning-stress spectrum (log-uniform in [1e-4, 1]) at 512 x 2048
    announce("logspec 512x2048")
    import dataclasses
    w = dataclasses.replace(wl.STRESS_4096x16384, shapes=((512, 2048), (2048, 512)))
    for i in range(2):
        gt = wl.make_grad(w, i, device=DEV)
        g = to64(gt)
        o = mn.orthogonalize(gt, Q5, compute="bf16", out_dtype=torch.float32)
        ref = oracle.orthogonalize(g, Q5)
        assert oracle.relative_frobenius_error(to64(o), ref) <= 2e-2
        o = mn.orthogonalize(gt, [wl.CUBIC] * 30, compute="fp32", out_dtype=torch.float32)
        torch.cuda.synchronize()
        ref = oracle.orthogonalize(g, [wl.CUBIC] * 30)
        assert oracle.relative_frobenius_error(to64(o), ref) <= 1e-4
        x0 = normalise(g if g.shape[0] <= g.shape[1] else g.T)
        cf = gram_closed_form(x0, [wl.CUBIC] * 30)
        cf = cf if g.shape[0] <= g.shape[1] else cf.T
        assert oracle.relative_frobenius_error(ref, cf) <= 1e-8


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("pad", [0, 1, 4])
def test_tall_batch_stride_through_c_abi(compute, out_dtype, pad):
    # Tall matrices store the result transposed to the oriented X; with
    # m % 4 == 0 the result rows are written in aligned runs of 4 unless the
    # batch stride breaks the alignment (pad 1), which must give the same values.
    announce("tall batch stride", compute, out_dtype, pad)
    from muon_newton_schulz_step_amd import _lib
    batch, rows, cols = 3, 300, 44
    stride = rows * cols + pad
    x = wl.gaussian_batch(batch, rows, cols, seed=11, device=DEV)
    xin = torch.zeros(batch * stride, dtype=torch.float32, device=DEV)
    out = torch.full((batch * stride,), 7.0, dtype=out_dtype, device=DEV)
    for b in range(batch):
        xin[b * stride:b * stride + rows * cols] = x[b].reshape(-1)
    lib = mn.lib()
    c = 0 if compute == "bf16" else 1
    need = lib.muon_orthogonalize_workspace_bytes(batch, rows, cols, c)
    ws = torch.empty(need + 256, dtype=torch.uint8, device=DEV)
    wp = (ws.data_ptr() + 255) // 256 * 256
    st = lib.muon_orthogonalize(
        xin.data_ptr(), _lib.MUON_FP32, out.data_ptr(),
        _lib.MUON_BF16 if out_dtype == torch.bfloat16 else _lib.MUON_FP32,
        batch, rows, cols, stride, _lib.coeff_array(Q5), 5, 1e-7, c, wp, need, None)
    assert st == _lib.MUON_OK
    torch.cuda.synchronize()
    extra = 4e-3 if out_dtype == torch.bfloat16 else 0.0
    for b in range(batch):
        o = out[b * stride:b * stride + rows * cols].reshape(rows, cols)
        ref = oracle.orthogonalize(to64(x[b]), Q5)
        assert oracle.relative_frobenius_error(to64(o), ref) <= tol(compute) + extra, b
        if pad:  # the gap between matrices is not written
            assert torch.all(out[b * stride + rows * cols:(b + 1) * stride] == 7.0)


@pytest.mark.parametrize("tall", [False, True], ids=["wide", "tall"])
def test_gram_by_qaq_log_spectrum(tall):
    # 2048 x 8192 is the smallest shape whose steps 1 and 3 form the Gram
    # matrix as Q A Q (bf16, N >= 4M, M >= 2048); a log-uniform spectrum over
    # four decades is where that rounding shows most (emulated: 7.5e-3 against
    # 5.3e-3 for the Gram of X itself at 512 x 2048)
    import dataclasses
    announce("gram by QAQ, log spectrum 2048x8192", "tall" if tall else "wide")
    w = dataclasses.replace(wl.STRESS_4096x16384, shapes=((8192, 2048) if tall else (2048, 8192),))
    g = wl.make_grad(w, 0, device=DEV)
    o = mn.orthogonalize(g, Q5, compute="bf16", out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.orthogonalize(to64(g), Q5)
    err = oracle.relative_frobenius_error(to64(o), ref)
    print("  rel err", err, flush=True)
    assert err <= tol("bf16")
    check_tiles(to64(o), ref, tol("bf16"), "qaq log spectrum")


def test_gram_by_qaq_per_step_table():
    # Q = a_{k-1} I + B_{k-1} takes the previous step's a: with a table whose
    # consecutive a differ (quintic, cubic, ...) a wrong step index would show
    announce("gram by QAQ, per-step table, 2048x8192")
    table = [wl.QUINTIC, wl.CUBIC, wl.QUINTIC, wl.CUBIC, wl.QUINTIC]
    g = wl.gaussian_matrix(2048, 8192, seed=41, device=DEV).to(torch.bfloat16)
    o = mn.orthogonalize(g, table, compute="bf16", out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.orthogonalize(to64(g), table)
    err = oracle.relative_frobenius_error(to64(o), ref)
    print("  rel err", err, flush=True)
    assert err <= tol("bf16")
    check_tiles(to64(o), ref, tol("bf16"), "qaq per-step table")

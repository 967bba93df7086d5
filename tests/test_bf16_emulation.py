"""An emulation of the bf16 path's rounding, used only to derive tolerances
and to check two design choices; it is never the parity reference (that is
the fp64 oracle).

The emulated arithmetic follows the library's bf16 path step by step:
  * X_0 is the fp32 input u carried as hi = bf16(u) and a signed byte lo,
    u - hi in 1/256 of hi's bf16 spacing (lo8 below); the Frobenius norm is
    folded in as 1/(||u|| + eps) (squared into the first Gram matrix, once
    into the first update);
  * every product takes bf16 operands (X's hi plane, A, B, or T), multiplies
    exactly and accumulates in fp32;
  * A and B are stored as bf16 (round to nearest even), X between steps as
    hi + lo of the fp32 update a X + B X, in the same 3-byte form;
  * in Q A Q Gram steps (wide groups with N >= 4M, M >= 2048 on the GPU), A
    is formed from the previous step as T = a' (A + A_lo) + B A, then
    A = a' T + T B, with A_lo A's bf16 residual.
Products are evaluated with exact (fp64) sums rounded once to fp32; the
hardware's fp32 accumulation differs from that only at the 1e-7 level,
far below the bf16 roundings that set the error.

With every rounding switched off the emulation must be the oracle's
iteration (pinned first below), so its algebra is the method's."""
import numpy as np
import pytest

import oracle
import workloads as wl
from gpu_helpers import (BF16_SMALL_TOL, BF16_TOL, DEGENERATE_BF16_TOL, DEGENERATE_SHAPES,
                         SMALL_DIM)

Q5 = [(3.4445, -4.7750, 2.0315)] * 5


def bf16(x):
    """Round fp32 values to bf16 (nearest, ties to even), returned as fp32."""
    x = np.ascontiguousarray(x, np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    r = ((b + (((b >> 16) & 1) + 0x7FFF)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def f32(x):
    return np.asarray(x, np.float64).astype(np.float32)


def lo8(x):
    """x as (hi, lo) with hi = bf16(x) and lo = q * 2^(e - 16), q the signed
    byte round((x - hi) * 2^(16 - e)) (to nearest even) clamped to
    [-128, 127], where hi = f * 2^e with f in [0.5, 1) (frexp), so 2^(e - 16)
    is 1/256 of hi's bf16 spacing.  The decode takes the unit from hi's
    exponent bits: lo = 0 for a zero or subnormal hi, NaN for a non-finite
    one.  Both returned as fp32 values."""
    x = f32(x)
    hi = bf16(x)
    finite = np.isfinite(hi)
    _, e = np.frexp(np.where(finite, hi, 0.0).astype(np.float64))
    unit = np.ldexp(1.0, e.astype(np.int64) - 16)
    with np.errstate(invalid="ignore"):
        q = np.clip(np.rint((x.astype(np.float64) - hi) / unit), -128, 127)
    normal = np.abs(hi.astype(np.float64)) >= 2.0 ** -126
    lo = np.where(normal, q * unit, 0.0)
    return hi, f32(np.where(finite, lo, np.nan))


def emulate(u, coeffs, xstate="lo8", qaq_steps=(), exact=False):
    """O for the fp32 input u as the bf16 path computes it.

    xstate "lo8": X kept as hi + a one-byte lo between steps (the library);
    "hilo": hi + lo as two bf16 values (the same 16 bits in 4 bytes); "bf16":
    X kept as bf16 alone (the rejected design).  qaq_steps: steps whose Gram
    matrix is formed as Q A Q (never step 0 or the last step).  exact: no
    rounding at all, fp64 throughout (must equal the oracle)."""
    rnd = (lambda x: np.asarray(x, np.float64)) if exact else bf16
    fl = (lambda x: np.asarray(x, np.float64)) if exact else f32

    def mm(a, b):
        return fl(np.asarray(a, np.float64) @ np.asarray(b, np.float64))

    u = fl(u)
    tall = u.shape[0] > u.shape[1]
    if tall:
        u = u.T.copy()
    s = float(np.sum(np.asarray(u, np.float64) ** 2))
    inv = 1.0 / (np.sqrt(s) + oracle.DEFAULT_EPS)
    inv = float(inv) if exact else np.float32(inv)
    def split(x):
        if exact:
            return x, np.zeros_like(x)
        if xstate == "lo8":
            return lo8(x)
        hi = rnd(x)
        return hi, (rnd(fl(x - hi)) if xstate == "hilo" else np.zeros_like(x))

    hi, lo = split(u)
    A = B = Alo = None
    n_steps = len(coeffs)
    for k, (a, b, c) in enumerate(coeffs):
        a, b, c = (float(a), float(b), float(c)) if exact else map(np.float32, (a, b, c))
        if 0 < k <= n_steps - 2 and k in qaq_steps:
            ap = coeffs[k - 1][0] if exact else np.float32(coeffs[k - 1][0])
            T = rnd(fl(ap * fl(A + Alo) + mm(B, A)))
            A = rnd(fl(ap * T + mm(T, B)))
        else:
            acc = mm(hi, hi.T)
            if k == 0:
                acc = fl(acc * (inv * inv))
            A = rnd(acc)
            Alo = rnd(fl(acc - A))
        B = rnd(fl(b * A + c * mm(A, A.T)))
        x = fl(a * fl(hi + lo) + mm(B, hi))
        if k == 0:
            x = fl(inv * x)
        if k == n_steps - 1:
            out = np.asarray(x, np.float64)
            return out.T if tall else out
        hi, lo = split(x)


def emulated_errors(shape, draws, seed):
    rng = np.random.default_rng(seed)
    errs = []
    for _ in range(draws):
        u = rng.standard_normal(shape).astype(np.float32)
        ref = oracle.orthogonalize(u.astype(np.float64), Q5)
        errs.append(oracle.relative_frobenius_error(emulate(u, Q5), ref))
    return np.array(errs)


# ------------------------------------------------ the emulator is the method
@pytest.mark.parametrize("shape", [(1, 1), (2, 8), (8, 2), (5, 5), (16, 40), (40, 16)])
@pytest.mark.parametrize("qaq", [(), (1, 3)])
def test_emulation_without_rounding_is_the_oracle(shape, qaq):
    u = np.random.default_rng(3).standard_normal(shape)
    got = emulate(u, Q5, qaq_steps=qaq, exact=True)
    assert oracle.relative_frobenius_error(got, oracle.orthogonalize(u, Q5)) <= 1e-12


def test_bf16_rounding_helper():
    # round to nearest even at the 16th bit: 1 + 2^-8 is a tie between 1 and
    # 1 + 2^-7 and goes to the even one (1); 1 + 3*2^-9 rounds up
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -9, -2.7435, 3.0e38], np.float32)
    assert list(bf16(x)) == [1.0, 1.0, 1.0 + 2.0 ** -7, -2.75, np.float32(1.765625 * 2.0 ** 127)]


# ------------------------------- tolerances of the small shapes, derived
DRAWS, SEED = 1000, 20261203


@pytest.mark.parametrize("oriented", sorted(BF16_SMALL_TOL), ids=lambda s: f"{s[0]}x{s[1]}")
def test_small_shape_bound_is_derived_from_the_emulation(oriented):
    """Each bound of the table is at least the emulated maximum over 1000
    Gaussian draws and at most 1.25 times it."""
    e = emulated_errors(oriented, DRAWS, SEED)
    bound = BF16_SMALL_TOL[oriented]
    print(oriented, "median %.3e max %.3e bound %.3g" % (np.median(e), e.max(), bound))
    assert e.max() <= bound <= 1.25 * e.max()


@pytest.mark.parametrize("shape", [(64, 64), (64, 128), (100, 300), (128, 128)])
def test_from_64_rows_on_the_plain_bar_holds(shape):
    """From min(rows, cols) = 64 on the bf16 bar of 2e-2 applies as it is:
    the emulated maximum stays below it with room to spare."""
    assert min(shape) >= SMALL_DIM
    e = emulated_errors(shape, 100, SEED)
    assert e.max() <= 0.95 * BF16_TOL, e.max()


# ------------------------------- degenerate inputs, bounds derived
@pytest.mark.parametrize("kind", wl.DEGENERATE_KINDS)
def test_degenerate_bounds_are_derived(kind):
    """A degenerate kind keeps the plain bar when the emulated bf16 path stays
    within 0.8 of it on every shape the GPU test uses; otherwise its bound is
    between 1.1 and 1.25 times the emulated maximum."""
    e = []
    for shape in DEGENERATE_SHAPES:
        x = wl.degenerate_matrix(kind, *shape).numpy()
        ref = oracle.orthogonalize(x.astype(np.float64), Q5)
        e.append(oracle.relative_frobenius_error(emulate(x, Q5), ref))
    worst = max(e)
    print(kind, ["%.3e" % v for v in e])
    if kind in DEGENERATE_BF16_TOL:
        assert worst > 0.8 * BF16_TOL
        assert 1.1 * worst <= DEGENERATE_BF16_TOL[kind] <= 1.25 * worst
    else:
        assert worst <= 0.8 * BF16_TOL


# -------------------------------------------- the two design choices
def _inputs(kind, m, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "lowrank":   # rank 16 + noise, the d1280 recipe's structure
        p, q = rng.standard_normal((m, 16)), rng.standard_normal((n, 16))
        g = (p @ q.T) * (1e-3 / 4.0) + 1e-4 * rng.standard_normal((m, n))
    else:                   # log-uniform singular values in [1e-4, 1]
        u, _ = np.linalg.qr(rng.standard_normal((m, m)))
        v, _ = np.linalg.qr(rng.standard_normal((n, m)))
        s = np.exp(np.log(1e-4) * rng.random(m))
        g = (u * s) @ v.T
    return g.astype(np.float32)


@pytest.mark.parametrize("kind", ["lowrank", "logspec"])
def test_x_state_needs_more_than_bf16(kind):
    """X carried between steps as bf16 alone misses the 2e-2 bar on
    structured inputs; with 16 significant bits it stays far inside, and the
    one-byte lo gives the error of a second bf16 value within 3%."""
    g = _inputs(kind, 256, 1024, 11)
    ref = oracle.orthogonalize(g.astype(np.float64), Q5)
    e_lo8 = oracle.relative_frobenius_error(emulate(g, Q5), ref)
    e_hilo = oracle.relative_frobenius_error(emulate(g, Q5, xstate="hilo"), ref)
    e_bf16 = oracle.relative_frobenius_error(emulate(g, Q5, xstate="bf16"), ref)
    assert e_lo8 <= 0.5 * BF16_TOL and e_bf16 > BF16_TOL, (e_lo8, e_bf16)
    assert abs(e_lo8 / e_hilo - 1.0) <= 0.03, (e_lo8, e_hilo)


def test_lo8_holds_sixteen_bits():
    """hi + lo of the one-byte form is within 1/512 of hi's bf16 spacing of
    x (2^-16 relative) over fp32's normal range, 2^-126 to 2^126, except where
    x - hi is within 1/512 of that spacing below +1/2 of it: there q = 128 is
    clamped to 127 and the error is at most 1/256.  Zero stays zero; a
    non-finite x comes back as NaN."""
    rng = np.random.default_rng(5)
    mant = rng.uniform(1.0, 2.0, 4000) * rng.choice([-1.0, 1.0], 4000)
    x = f32(mant * np.exp2(rng.integers(-126, 127, 4000)))
    hi, lo = lo8(x)
    e = ((hi.view(np.uint32) >> 23) & 0xFF).astype(np.int64)
    ulp = np.exp2((e - 134).astype(np.float64))
    d = x.astype(np.float64) - hi
    err = np.abs(d - lo)
    clamped = d > ulp * (127.5 / 256)
    assert 0 < clamped.sum() < 0.01 * x.size
    assert np.all(err[~clamped] <= ulp[~clamped] / 512)
    assert np.all(err[clamped] <= ulp[clamped] / 256)
    assert np.all(np.abs(d) <= ulp / 2)
    z_hi, z_lo = lo8(np.zeros(3, np.float32))
    assert not z_hi.any() and not z_lo.any()
    s_hi, s_lo = lo8(np.array([np.inf, -np.inf, np.nan], np.float32))
    assert np.isnan(s_hi + s_lo).all()


@pytest.mark.parametrize("kind", ["lowrank", "logspec"])
def test_qaq_gram_steps_one_and_three_only(kind):
    """Q A Q Gram matrices at steps 1 and 3 keep the error within the bar;
    at steps 1, 2 and 3 (three in a row) they do not."""
    g = _inputs(kind, 256, 1024, 12)
    ref = oracle.orthogonalize(g.astype(np.float64), Q5)
    e13 = oracle.relative_frobenius_error(emulate(g, Q5, qaq_steps=(1, 3)), ref)
    e123 = oracle.relative_frobenius_error(emulate(g, Q5, qaq_steps=(1, 2, 3)), ref)
    assert e13 <= 0.5 * BF16_TOL and e123 > BF16_TOL, (e13, e123)


@pytest.mark.parametrize("kind", ["gauss", "logspec"])
@pytest.mark.parametrize("qaq", [(), (1, 3)])
def test_tile_errors_track_the_matrix_error(kind, qaq):
    """Every 256 x 256 tile of the emulated result is within 1.1x of the
    whole matrix's error (the GPU tests allow 1.25x, gpu_helpers.check_tiles),
    so a per-tile bound catches faults confined to part of a matrix."""
    from gpu_helpers import TILE_SPREAD, tile_errors
    g = (np.random.default_rng(3).standard_normal((512, 2048)).astype(np.float32)
         if kind == "gauss" else _inputs(kind, 512, 2048, 13))
    ref = oracle.orthogonalize(g.astype(np.float64), Q5)
    o = emulate(g, Q5, qaq_steps=qaq)
    whole = oracle.relative_frobenius_error(o, ref)
    e = tile_errors(o, ref)
    assert len(e) == 16 and e.max() <= 1.1 * whole and 1.1 < TILE_SPREAD
    # a 10% error in one 32 x 256 block passes the whole-matrix bar but not
    # the per-tile bound
    bad = o.copy()
    noise = np.sign(np.random.default_rng(4).standard_normal((32, 256)))
    bad[64:96, :256] += 0.1 * ref[64:96, :256] * noise
    assert oracle.relative_frobenius_error(bad, ref) <= BF16_TOL
    assert tile_errors(bad, ref).max() > BF16_TOL

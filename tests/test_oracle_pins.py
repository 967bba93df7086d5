"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: the SVD
closed form, convergence of the cubic map to U V^T, exact rational
arithmetic, invariances and scalar closed forms.  A dropped term, a wrong sign,
a swapped coefficient or a transposed operand anywhere in the oracle fails at
least one of them (see ``test_planted_mistakes_are_caught``).
"""
from fractions import Fraction
import math
import os

import numpy as np
import pytest

import oracle
from oracle import muon_oracle as mo
import workloads as wl

QUINTIC = [wl.QUINTIC] * 5


def scalar_map(x: float, coeffs) -> float:
    """Composition of x -> a x + b x^3 + c x^5 in plain Python floats."""
    for a, b, c in coeffs:
        x = a * x + b * x ** 3 + c * x ** 5
    return x


def spectral_closed_form(g, coeffs, eps=mo.DEFAULT_EPS):
    """U phi(Sigma / (||G||_F + eps)) V^T: the iteration acts on singular values
    by the scalar polynomial (polynomial functional calculus)."""
    g = np.asarray(g, np.float64)
    u, s, vt = np.linalg.svd(g, full_matrices=False)
    fro = math.sqrt(float(np.sum(s * s)))
    sig = s / (fro + eps)
    for a, b, c in coeffs:
        sig = a * sig + b * sig ** 3 + c * sig ** 5
    return (u * sig) @ vt


def rng(seed):
    return np.random.default_rng(seed)


def with_spectrum(rows, cols, smin, smax, seed):
    r = rng(seed)
    k = min(rows, cols)
    u, _ = np.linalg.qr(r.standard_normal((rows, k)))
    v, _ = np.linalg.qr(r.standard_normal((cols, k)))
    s = np.exp(r.uniform(math.log(smin), math.log(smax), size=k))
    return (u * s) @ v.T


# ---------------------------------------------------------------- P3 closed form
@pytest.mark.parametrize("shape", [(1, 1), (2, 8), (8, 2), (5, 5), (16, 8),
                                   (8, 16), (64, 64), (256, 128), (96, 300)])
@pytest.mark.parametrize("steps", [1, 5])
def test_ns_matches_spectral_closed_form(shape, steps):
    g = rng(hash(shape) % 1000 + steps).standard_normal(shape)
    coeffs = [wl.QUINTIC] * steps
    o = oracle.orthogonalize(g, coeffs)
    ref = spectral_closed_form(g, coeffs)
    assert np.max(np.abs(o - ref)) <= 1e-10 * max(1.0, np.max(np.abs(ref)))


def test_ns_closed_form_ill_conditioned():
    # log-uniform spectrum in [1e-4, 1] like the conditioning stress workload
    g = with_spectrum(96, 384, 1e-4, 1.0, 7)
    for coeffs in ([wl.QUINTIC] * 5, [wl.CUBIC] * 30):
        o = oracle.orthogonalize(g, coeffs)
        ref = spectral_closed_form(g, coeffs)
        assert oracle.relative_frobenius_error(o, ref) <= 1e-10


def test_ns_per_step_table_order():
    # different (a, b, c) per step: the closed form fixes their order of use
    table = [(3.4445, -4.7750, 2.0315), (1.5, -0.5, 0.0), (2.0, -1.5, 0.5),
             (1.875, -1.25, 0.375)]
    g = rng(3).standard_normal((24, 40))
    o = oracle.orthogonalize(g, table)
    ref = spectral_closed_form(g, table)
    assert oracle.relative_frobenius_error(o, ref) <= 1e-12
    o_rev = oracle.orthogonalize(g, table[::-1])
    assert oracle.relative_frobenius_error(o_rev, ref) > 1e-3


# ---------------------------------------------------------- P2 cubic -> U V^T
@pytest.mark.parametrize("shape", [(1, 1), (2, 8), (8, 2), (3, 4), (4, 3),
                                   (5, 5), (16, 8), (8, 16)])
def test_cubic_converges_to_polar_factor(shape):
    rows, cols = shape
    g = with_spectrum(rows, cols, 1e-2, 1.0, rows * 100 + cols)
    o = oracle.orthogonalize(g, [wl.CUBIC] * 40)
    u, _, vt = np.linalg.svd(g, full_matrices=False)
    assert np.max(np.abs(o - u @ vt)) <= 1e-6


def test_cubic_gaussian_polar_factor():
    g = rng(11).standard_normal((16, 8))
    o = oracle.orthogonalize(g, [wl.CUBIC] * 40)
    u, _, vt = np.linalg.svd(g, full_matrices=False)
    assert np.max(np.abs(o - u @ vt)) <= 1e-6
    # polar factor: O^T O = I for a tall full-rank matrix
    assert np.max(np.abs(o.T @ o - np.eye(8))) <= 1e-6


# ------------------------------------------------------- P1 tall/wide forms
@pytest.mark.parametrize("shape", [(300, 120), (17, 5), (8, 2)])
def test_tall_equals_transposed_wide(shape):
    g = rng(5).standard_normal(shape)
    o_tall = oracle.orthogonalize(g, QUINTIC)           # tall form
    o_wide_t = oracle.orthogonalize(g.T, QUINTIC).T     # wide form on G^T
    assert np.max(np.abs(o_tall - o_wide_t)) <= 1e-13 * max(1, np.abs(o_tall).max()) * 10
    # forcing the other form on the same matrix: X (X^T X)^k = (X X^T)^k X
    o_forced = oracle.orthogonalize(g, QUINTIC, form="wide")
    assert np.max(np.abs(o_tall - o_forced)) <= 1e-12


def test_square_uses_wide_and_agrees_with_tall():
    g = rng(6).standard_normal((33, 33))
    assert np.max(np.abs(oracle.orthogonalize(g, QUINTIC)
                         - oracle.orthogonalize(g, QUINTIC, form="tall"))) <= 1e-12


# ------------------------------------------------ P4 quintic singular-value band
def test_quintic_band_on_single_256x128():
    w = wl.SINGLE_256x128
    g = wl.make_grad(w, 0).double().numpy()
    _, u = oracle.nesterov_momentum(g, np.zeros_like(g), w.mu)
    o = oracle.orthogonalize(u, w.coeff_table)
    sv = np.linalg.svd(o, compute_uv=False)
    assert sv.min() >= 0.5 and sv.max() <= 1.5


def test_quintic_scalar_map_facts():
    # p(1) = a + b + c; phi5 is bounded by 1.21 on [0, 1] and >= 0.5 above 1.0671e-3
    a, b, c = wl.QUINTIC
    assert abs(scalar_map(1.0, [wl.QUINTIC]) - (a + b + c)) < 1e-15
    xs = np.linspace(0.0, 1.0, 200001)
    ys = np.array([scalar_map(x, QUINTIC) for x in xs[::50]])
    assert ys.max() < 1.21
    assert scalar_map(1.0671e-3, QUINTIC) >= 0.5 > scalar_map(1.0660e-3, QUINTIC)


# --------------------------------------------------------- P5 special cases
def test_scalar_one_by_one():
    for gval in (3.0, -0.25, 1e-3):
        o = oracle.orthogonalize(np.array([[gval]]), QUINTIC)
        x0 = abs(gval) / (abs(gval) + mo.DEFAULT_EPS)
        assert abs(o[0, 0] - math.copysign(scalar_map(x0, QUINTIC), gval)) <= 1e-13
    o = oracle.orthogonalize(np.array([[-2.0]]), [wl.CUBIC] * 40)
    assert abs(o[0, 0] + 1.0) <= 1e-12


def test_orthonormal_columns_scale():
    q, _ = np.linalg.qr(rng(8).standard_normal((256, 128)))
    o = oracle.orthogonalize(q, QUINTIC)
    expect = scalar_map(1.0 / (math.sqrt(128) + mo.DEFAULT_EPS), QUINTIC)
    assert abs(expect - 0.72276216) < 1e-6
    assert np.max(np.abs(o - expect * q)) <= 1e-12


def test_permutation_matrix_scale():
    p = np.eye(768)[rng(9).permutation(768)]
    o = oracle.orthogonalize(p, QUINTIC)
    expect = scalar_map(1.0 / (math.sqrt(768) + mo.DEFAULT_EPS), QUINTIC)
    assert abs(expect - 1.08359457) < 1e-6
    assert np.max(np.abs(o - expect * p)) <= 1e-12


def test_rectangular_diagonal_elementwise():
    d = np.array([3.0, -1.0, 0.5, -0.01])
    g = np.zeros((4, 7))
    g[np.arange(4), np.arange(4)] = d
    o = oracle.orthogonalize(g, QUINTIC)
    fro = math.sqrt(float(np.sum(d * d))) + mo.DEFAULT_EPS
    expect = np.zeros_like(g)
    for i, di in enumerate(d):
        expect[i, i] = math.copysign(scalar_map(abs(di) / fro, QUINTIC), di)
    assert np.max(np.abs(o - expect)) <= 1e-13


def test_zero_gradient_gives_zero():
    o = oracle.orthogonalize(np.zeros((5, 9)), QUINTIC)
    assert np.all(o == 0.0)


# --------------------------------------- exact rational arithmetic (brute force)
def _exact_ns(g_rows, norm, coeffs):
    """Newton-Schulz in exact rationals with pure-Python loops (eps = 0).
    ``norm`` is the exact integer Frobenius norm of the integer matrix."""
    x = [[Fraction(v, norm) for v in row] for row in g_rows]
    rows, cols = len(x), len(x[0])
    fc = [(Fraction(a), Fraction(b), Fraction(c)) for a, b, c in coeffs]

    def mm(p, q):
        return [[sum(p[i][k] * q[k][j] for k in range(len(q)))
                 for j in range(len(q[0]))] for i in range(len(p))]

    def tr(p):
        return [list(r) for r in zip(*p)]

    for a, b, c in fc:
        if rows > cols:
            A = mm(tr(x), x)
            A2 = mm(A, A)
            poly = [[b * A[i][j] + c * A2[i][j] for j in range(cols)] for i in range(cols)]
            xp = mm(x, poly)
        else:
            A = mm(x, tr(x))
            A2 = mm(A, A)
            poly = [[b * A[i][j] + c * A2[i][j] for j in range(rows)] for i in range(rows)]
            xp = mm(poly, x)
        x = [[a * x[i][j] + xp[i][j] for j in range(cols)] for i in range(rows)]
    return np.array([[float(v) for v in row] for row in x])


@pytest.mark.parametrize("g,norm", [
    ([[1, 2, 2], [0, 4, 0]], 5),          # wide 2x3, ||G||_F = 5
    ([[1, 0], [2, 4], [2, 0]], 5),        # tall 3x2
    ([[2, 3, 6]], 7),                     # one row
    ([[1, 2], [2, 4]], 5),                # square, rank one
])
@pytest.mark.parametrize("steps", [1, 3])
def test_exact_rational_brute_force(g, norm, steps):
    coeffs = [wl.QUINTIC] * steps
    exact = _exact_ns(g, norm, coeffs)
    got = oracle.orthogonalize(np.array(g, float), coeffs, eps=0.0)
    assert np.max(np.abs(got - exact)) <= 1e-12


# ------------------------------------------------------ P8 / P9 invariances
def test_orthogonal_invariance():
    r = rng(12)
    g = r.standard_normal((20, 50))
    q1, _ = np.linalg.qr(r.standard_normal((20, 20)))
    q2, _ = np.linalg.qr(r.standard_normal((50, 50)))
    lhs = oracle.orthogonalize(q1 @ g @ q2, QUINTIC)
    rhs = q1 @ oracle.orthogonalize(g, QUINTIC) @ q2
    assert np.max(np.abs(lhs - rhs)) <= 1e-12


def test_permutation_invariance():
    r = rng(13)
    g = r.standard_normal((30, 12))
    pr, pc = r.permutation(30), r.permutation(12)
    lhs = oracle.orthogonalize(g[pr][:, pc], QUINTIC)
    rhs = oracle.orthogonalize(g, QUINTIC)[pr][:, pc]
    assert np.max(np.abs(lhs - rhs)) <= 1e-13


@pytest.mark.parametrize("alpha", [1e-3, 1.0, 1e3, -1.0])
def test_scale_and_sign_invariance(alpha):
    g = rng(14).standard_normal((16, 8))
    lhs = oracle.orthogonalize(alpha * g, QUINTIC)
    rhs = math.copysign(1.0, alpha) * oracle.orthogonalize(g, QUINTIC)
    assert oracle.relative_frobenius_error(lhs, rhs) <= 1e-4


# ------------------------------------------------ P6 / P7 momentum and update
def test_nesterov_closed_form():
    r = rng(15)
    g, buf = r.standard_normal((7, 9)), r.standard_normal((7, 9))
    mu = 0.95
    new_buf, u = oracle.nesterov_momentum(g, buf, mu)
    assert np.max(np.abs(u - ((1 + mu) * g + mu * mu * buf))) <= 1e-14
    assert np.max(np.abs(new_buf - (g + mu * buf))) <= 1e-15
    _, u0 = oracle.nesterov_momentum(g, np.zeros_like(g), mu)
    assert np.max(np.abs(u0 - 1.95 * g)) <= 1e-15


def test_muon_step_update_closed_form():
    r = rng(16)
    w, g, buf = (r.standard_normal((12, 5)) for _ in range(3))
    new_w, new_buf, o = oracle.muon_step(w, g, buf, 0.9, 0.02, 1.7, QUINTIC)
    assert np.max(np.abs((new_w - w) - (-0.02 * 1.7) * o)) <= 1e-15
    # the step orthogonalises the momentum-corrected gradient, not g itself
    u = 1.9 * g + 0.81 * buf
    assert np.max(np.abs(o - spectral_closed_form(u, QUINTIC))) <= 1e-10
    assert np.max(np.abs(new_buf - (0.9 * buf + g))) <= 1e-15


# ------- 3.8B shape list ("Training a 3.8B LLM to CORE 0.384 for $998", parameter table)
def _golden_table():
    path = os.path.join(os.path.dirname(__file__), "golden", "page5_parameter_table.txt")
    out = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v, step = line.split()
            out[k] = (float(v), float(step))
    return out


def test_3p8b_matrix_set_matches_page_parameter_table():
    t = _golden_table()
    w = wl.GPT_3P8B
    assert len(w.shapes) == 168
    d_model, n_layers = 3072, 28
    kv_dim = int(t["kv_heads"][0]) * 128
    assert kv_dim == 1024 and int(t["query_heads"][0]) * 128 == d_model
    mat = sum(r * c for r, c in w.shapes)
    assert mat == 2_818_572_288
    # two RMSNorm gain vectors per layer complete the decoder-layer count
    layers = mat + n_layers * 2 * d_model
    v, step = t["decoder_layers_28"]
    assert abs(layers / 1e6 - v) <= step / 2
    vocab = int(t["vocab_padded"][0])
    v, step = t["token_embedding"]
    assert abs(vocab * d_model / 1e6 - v) <= step / 2
    v, step = t["value_embeddings_14_tables"]
    assert abs(14 * vocab * kv_dim / 1e6 - v) <= step / 2
    assert w.oriented_groups() == {(3072, 3072): 56, (1024, 3072): 56, (3072, 12288): 56}


def test_counted_flops_of_workloads():
    assert abs(wl.GPT_3P8B.ns_flops_counted() / 1e12 - 199.03) < 0.01
    assert abs(wl.GPT_D768.ns_flops_counted() / 1e12 - 1.087) < 0.001
    assert abs(wl.GPT_D1280.ns_flops_counted() / 1e12 - 12.58) < 0.01


# ---------------------------------- the pins catch plausible oracle mistakes
def _mutants():
    """Plausible slips in the Newton-Schulz step; each must fail a pin."""
    ns = mo.newton_schulz  # the unpatched iteration

    def run(x, coeffs, update):
        x = np.asarray(x, float)
        for a, b, c in coeffs:
            x = update(x, a, b, c)
        return x

    def dropped_c(x, coeffs, form=None):
        return ns(x, [(a, b, 0.0) for a, b, c in coeffs], form)

    def swapped_bc(x, coeffs, form=None):
        return ns(x, [(a, c, b) for a, b, c in coeffs], form)

    def wrong_sign_b(x, coeffs, form=None):
        return ns(x, [(a, -b, c) for a, b, c in coeffs], form)

    def a_not_a_squared(x, coeffs, form=None):
        def upd(x, a, b, c):
            A = x @ x.T
            return a * x + (b * A + c * A) @ x
        return run(x, coeffs, upd)

    def wrong_side(x, coeffs, form=None):
        def upd(x, a, b, c):
            A = x @ x.T
            return a * x + x @ (b * A + c * A @ A)
        return run(x, coeffs, upd)

    def transposed_operand(x, coeffs, form=None):
        def upd(x, a, b, c):
            A = x @ x.T
            return a * x + ((b * A + c * A @ A) @ x.T).T
        return run(x, coeffs, upd)

    return [dropped_c, swapped_bc, wrong_sign_b, a_not_a_squared, wrong_side,
            transposed_operand]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_planted_mistakes_are_caught(mutant, monkeypatch):
    monkeypatch.setattr(mo, "newton_schulz", mutant)
    caught = False
    for shape in [(5, 5), (16, 8), (8, 16)]:
        g = rng(21).standard_normal(shape)
        try:
            o = mo.orthogonalize(g, QUINTIC)
        except ValueError:
            caught = True
            break
        if np.max(np.abs(o - spectral_closed_form(g, QUINTIC))) > 1e-8:
            caught = True
            break
    assert caught


def test_planted_normalisation_mistake_is_caught(monkeypatch):
    def no_sqrt(u, eps=mo.DEFAULT_EPS):
        u = np.asarray(u, float)
        s = float(np.sum(u * u))
        return u / (s + eps), s
    monkeypatch.setattr(mo, "frobenius_normalize", no_sqrt)
    g = rng(22).standard_normal((16, 8))
    o = mo.orthogonalize(g, QUINTIC)
    assert np.max(np.abs(o - spectral_closed_form(g, QUINTIC))) > 1e-3


# ------------------------------ the comparison every parity check rests on
def _rfe_pins(rfe):
    """True if ``rfe`` passes every hand-computed case of the relative
    Frobenius error ||y - y_ref||_F / ||y_ref||_F."""
    cases = [
        # diff (3, -1): sqrt(10) / ||(0, 5)|| = sqrt(10) / 5
        ([[3.0, 4.0]], [[0.0, 5.0]], math.sqrt(10.0) / 5.0),
        # diff (0, 0, 0, 4): 4 / ||ref|| = 4 / 3, where ||y|| = 5 and the
        # largest entries are 4 (diff) and 2 (ref)
        ([[1.0, 2.0], [2.0, 4.0]], [[1.0, 2.0], [2.0, 0.0]], 4.0 / 3.0),
        # an error of 0.14, whose square (0.0196) would pass a 2e-2 bar
        ([[1.0, 0.14]], [[1.0, 0.0]], 0.14),
        # many small errors: ||(0.1, ..., 0.1)|| over 100 entries = 1, ref norm 10
        (np.full((10, 10), 1.1), np.ones((10, 10)), 0.1),
        # both zero: no error; a zero reference with a non-zero result: infinite
        ([[0.0, 0.0]], [[0.0, 0.0]], 0.0),
        ([[1e-30, 0.0]], [[0.0, 0.0]], float("inf")),
    ]
    for y, ref, want in cases:
        got = rfe(y, ref)
        if math.isinf(want):
            if not math.isinf(got):
                return False
        elif abs(got - want) > 1e-12 * max(1.0, want):
            return False
    return True


def test_relative_frobenius_error_hand_computed():
    assert _rfe_pins(oracle.relative_frobenius_error)


def _rfe_slips():
    def squared_ratio(y, ref):
        y, ref = np.asarray(y, float), np.asarray(ref, float)
        d = float(np.sum(ref * ref))
        return 0.0 if d == 0 else float(np.sum((y - ref) ** 2)) / d

    def result_in_denominator(y, ref):
        y, ref = np.asarray(y, float), np.asarray(ref, float)
        d = float(np.linalg.norm(y))
        return 0.0 if d == 0 else float(np.linalg.norm(y - ref)) / d

    def max_abs(y, ref):
        y, ref = np.asarray(y, float), np.asarray(ref, float)
        d = float(np.max(np.abs(ref)))
        return 0.0 if d == 0 else float(np.max(np.abs(y - ref))) / d

    def absolute(y, ref):
        return float(np.linalg.norm(np.asarray(y, float) - np.asarray(ref, float)))

    return [squared_ratio, result_in_denominator, max_abs, absolute]


@pytest.mark.parametrize("slip", _rfe_slips(), ids=lambda f: f.__name__)
def test_relative_frobenius_error_slips_fail_the_pins(slip):
    assert not _rfe_pins(slip)


# -------------------- the closed form the full-size GPU tests compare with
def test_gram_closed_form_matches_the_oracle():
    """tests/gpu_helpers.gram_closed_form computes U phi(S) V^T from the
    eigendecomposition of X X^T (so it runs at any size); on small cases it
    must equal the step-by-step oracle, for the quintic and the 30-step cubic
    on ill-conditioned inputs, rank-deficient ones and per-step tables."""
    from gpu_helpers import gram_closed_form, normalise
    cases = [
        (rng(40).standard_normal((48, 160)), QUINTIC, 1e-10),
        (with_spectrum(64, 256, 1e-4, 1.0, 41), QUINTIC, 1e-10),
        (with_spectrum(64, 256, 1e-4, 1.0, 42), [wl.CUBIC] * 30, 1e-8),
        (rng(43).standard_normal((32, 8)) @ rng(44).standard_normal((8, 96)), QUINTIC, 1e-10),
        (rng(45).standard_normal((40, 120)), [wl.QUINTIC, wl.CUBIC] * 3, 1e-10),
    ]
    for g, coeffs, bound in cases:
        ref = oracle.orthogonalize(g, coeffs)
        cf = gram_closed_form(normalise(g), coeffs)
        assert oracle.relative_frobenius_error(cf, ref) <= bound


def test_gram_closed_form_planted_mistake_fails():
    # taking phi(l) instead of phi(sqrt l) / sqrt l would be a plausible slip
    from gpu_helpers import gram_eig, normalise
    g = rng(46).standard_normal((24, 80))
    x0 = normalise(g)
    lam, v = gram_eig(x0)
    s = np.sqrt(np.maximum(lam, 0.0))
    wrong = (v * np.array([scalar_map(x, QUINTIC) for x in s])) @ (v.T @ x0)
    ref = oracle.orthogonalize(g, QUINTIC)
    assert oracle.relative_frobenius_error(wrong, ref) > 0.5


# --------------------------------------------------- non-finite values
def test_nan_gradient_element_propagates():
    """One NaN in a gradient: the momentum is NaN at that element only, and
    the normalisation spreads it to every element of O and of the new
    weights (the header's promise: non-finite values propagate)."""
    g = rng(47).standard_normal((6, 10))
    g[2, 3] = np.nan
    buf = rng(48).standard_normal((6, 10)) * 1e-3
    w = rng(49).standard_normal((6, 10)) * 0.02
    new_w, new_buf, o = oracle.muon_step(w, g, buf, 0.95, 0.02, 1.0, QUINTIC)
    assert np.isnan(new_buf[2, 3]) and np.isfinite(np.delete(new_buf.ravel(), 2 * 10 + 3)).all()
    assert np.isnan(o).all() and np.isnan(new_w).all()


def test_infinite_weight_element_stays_local():
    """An infinite weight does not enter the direction: only its own element
    of the new weights is non-finite."""
    g = rng(50).standard_normal((6, 10))
    w = rng(51).standard_normal((6, 10)) * 0.02
    w[4, 1] = np.inf
    new_w, _, o = oracle.muon_step(w, g, np.zeros_like(g), 0.95, 0.02, 1.0, QUINTIC)
    assert np.isfinite(o).all()
    assert new_w[4, 1] == np.inf
    assert np.isfinite(np.delete(new_w.ravel(), 4 * 10 + 1)).all()

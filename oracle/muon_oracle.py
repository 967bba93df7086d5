"""Plain fp64 CPU oracle of the Muon step for a GPT's 2-D weight matrices.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it.

Sources.  "Page 1" is the web3.cnoyu.systems review of karpathy/autoresearch's
``train.py`` (Japanese), in its paragraph on the Muon half of the MuonAdamW
optimizer: Muon takes the gradient, applies Nesterov momentum, and runs a
5-step Newton-Schulz iteration towards the orthogonal factor U of the polar
decomposition G = U*S; a tall matrix (more rows than columns) uses
A = X^T X, X <- aX + X(bA + cA^2), a wide one A = X X^T,
X <- aX + (bA + cA^2)X; the per-step coefficients are a precomputed table;
the orthogonal factor is used as the update direction; the momentum buffer
has the parameter's shape.

Readings where the page is silent (each one is listed with its reason in the
design notes of the repository):
  * Nesterov form: buf' = mu*buf + g, u = g + mu*buf'.
  * Before the iteration u is divided by (||u||_F + eps), eps = 1e-7.
  * A square matrix takes the wide form (both forms agree in exact arithmetic).
  * The weight update is W' = W - lr*scale*O with a per-matrix scale.

Everything is computed in float64 with numpy; inputs of lower precision
(bf16 or fp32 values) are upcast exactly before the first operation.

Parity pins: every function here is pinned by the tests in
``tests/test_oracle_pins.py`` (SVD closed form, convergence of the cubic
iteration to U V^T, exact rational arithmetic on small integer matrices,
tall/wide equivalence, orthogonal and scale invariance, closed forms for the
momentum and update; for NorMuon the closed form on orthonormal rows, the
RMS normalisation at beta2 = 0, the two-step EMA and transpose equivariance;
for the cautious decay a hand-derived example and its special cases).  No
function is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

DEFAULT_EPS = 1e-7


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def nesterov_momentum(grad, buf, mu: float):
    """Nesterov momentum of page 1 (Muon paragraph): returns (buf', u).

    buf' = mu*buf + g; u = g + mu*buf'.  ``buf`` is the element-wise momentum
    buffer of the parameter's shape.
    """
    g = _f64(grad)
    b = _f64(buf)
    new_buf = mu * b + g
    u = g + mu * new_buf
    return new_buf, u


def frobenius_normalize(u, eps: float = DEFAULT_EPS):
    """Divide by the Frobenius norm plus eps; returns (X0, ||u||_F)."""
    u = _f64(u)
    s = float(np.sqrt(np.sum(u * u)))
    return u / (s + eps), s


def newton_schulz(x, coeffs, form: str | None = None):
    """The Newton-Schulz iteration of page 1, one step per (a, b, c) row.

    Tall (rows > cols): A = X^T X, X <- aX + X (bA + cA^2).
    Wide or square:     A = X X^T, X <- aX + (bA + cA^2) X.
    ``form`` forces "tall" or "wide" (used to pin the equivalence of the two).
    """
    x = _f64(x)
    rows, cols = x.shape
    if form is None:
        form = "tall" if rows > cols else "wide"
    if form not in ("tall", "wide"):
        raise ValueError(f"unknown form {form!r}")
    for a, b, c in coeffs:
        if form == "tall":
            A = x.T @ x
            x = a * x + x @ (b * A + c * (A @ A))
        else:
            A = x @ x.T
            x = a * x + (b * A + c * (A @ A)) @ x
    return x


def orthogonalize(g, coeffs, eps: float = DEFAULT_EPS, form: str | None = None):
    """Frobenius-normalise ``g`` and run the Newton-Schulz iteration: O."""
    x0, _ = frobenius_normalize(g, eps)
    return newton_schulz(x0, coeffs, form)


def weight_update(w, o, lr: float, scale: float):
    """W' = W - lr*scale*O: the orthogonal factor used as the update direction."""
    return _f64(w) - lr * scale * _f64(o)


def muon_step(w, grad, buf, mu: float, lr: float, scale: float, coeffs,
              eps: float = DEFAULT_EPS):
    """One Muon step on one matrix.  Returns (W', buf', O).

    Order of page 1: momentum, orthogonalisation (normalise + iterate),
    then the weight update.
    """
    new_buf, u = nesterov_momentum(grad, buf, mu)
    o = orthogonalize(u, coeffs, eps)
    return weight_update(w, o, lr, scale), new_buf, o


# ---------------------------------------------------------------------------
# Page 1, the paragraph after the Muon one, adds two things on top of the
# plain step.  NorMuon: after orthogonalisation, per-row (or, by the aspect
# ratio, per-column) second-moment estimates of the update, kept as an
# exponential moving average, give every output dimension its own step size
# (Adam's adaptivity applied in the orthogonalised coordinates).  Cautious
# weight decay: only parameters whose update direction agrees in sign with
# the parameter decay, mask = (update * param) >= 0.
#
# Readings where the page is silent (listed with reasons in the design
# notes of the repository):
#   * the statistics sit on the shorter side of the matrix: per row of a wide
#     or square matrix, per column of a tall one (one value per row of the
#     oriented matrix); the second moment is the mean of O^2 along the longer
#     side;
#   * v' = beta2*v + (1 - beta2)*mean(O^2), no bias correction; beta2 and the
#     eps added to sqrt(v') are the caller's;
#   * O' = O / (sqrt(v') + eps) broadcast along the longer side;
#   * decoupled decay on the parameter before the update:
#     W' = W - lr*scale*O' - lr*wd*mask*W, mask = (O'*W >= 0) when cautious,
#     1 otherwise.


def normuon_scale(o, v, beta2: float, eps: float):
    """NorMuon scaling of an orthogonalised update O: returns (O', v').

    ``v`` holds min(rows, cols) second moments, one per row of a wide or
    square O, one per column of a tall O.
    """
    o = _f64(o)
    v = _f64(v)
    rows, cols = o.shape
    axis = 0 if rows > cols else 1          # reduce along the longer side
    msq = np.mean(o * o, axis=axis)
    new_v = beta2 * v + (1.0 - beta2) * msq
    d = np.sqrt(new_v) + eps
    o_new = o / (d[None, :] if axis == 0 else d[:, None])
    return o_new, new_v


def decayed_weight_update(w, o, lr: float, scale: float, weight_decay: float,
                          cautious: bool):
    """W' = W - lr*scale*O - lr*weight_decay*mask*W, mask = (O*W >= 0) when
    ``cautious`` (page 1's cautious weight decay), else 1 (plain decoupled
    decay)."""
    w = _f64(w)
    o = _f64(o)
    mask = (o * w >= 0.0) if cautious else np.ones_like(w, dtype=bool)
    return w - lr * scale * o - lr * weight_decay * np.where(mask, w, 0.0)


def muon_step_ex(w, grad, buf, mu: float, lr: float, scale: float, coeffs,
                 eps: float = DEFAULT_EPS, weight_decay: float = 0.0,
                 cautious: bool = True, second_moment=None, beta2: float = 0.0,
                 normuon_eps: float = 0.0):
    """The Muon step with page 1's additions: momentum, orthogonalisation,
    NorMuon scaling (when ``second_moment`` is given), then the weight update
    with (cautious) decoupled weight decay.  Returns a dict with ``w``,
    ``buf``, ``o`` (the update direction applied) and ``v`` (the new second
    moments, or None)."""
    new_buf, u = nesterov_momentum(grad, buf, mu)
    o = orthogonalize(u, coeffs, eps)
    new_v = None
    if second_moment is not None:
        o, new_v = normuon_scale(o, second_moment, beta2, normuon_eps)
    new_w = decayed_weight_update(w, o, lr, scale, weight_decay, cautious)
    return {"w": new_w, "buf": new_buf, "o": o, "v": new_v}


def relative_frobenius_error(y, y_ref) -> float:
    """||y - y_ref||_F / ||y_ref||_F (0 when both are zero)."""
    y = _f64(y)
    y_ref = _f64(y_ref)
    den = float(np.linalg.norm(y_ref))
    num = float(np.linalg.norm(y - y_ref))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den

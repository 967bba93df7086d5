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
momentum and update).  No function is "parity unpinned".
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


def relative_frobenius_error(y, y_ref) -> float:
    """||y - y_ref||_F / ||y_ref||_F (0 when both are zero)."""
    y = _f64(y)
    y_ref = _f64(y_ref)
    den = float(np.linalg.norm(y_ref))
    num = float(np.linalg.norm(y - y_ref))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den

"""Seeded synthetic workloads for the Muon matrix step.

This module holds shapes and random-number recipes only: none of the
optimizer's arithmetic.  Both sides of a parity test (the fp64 oracle and the
HIP library) take their inputs from here; neither side's code lives here.

Every matrix gets its own ``torch.Generator`` per tensor (grad, momentum,
weight), seeded from (workload seed, matrix index, stream id), so any subset of
a workload can be generated without generating the rest.  The generator runs
on the device the tensors are made on; CPU and GPU streams differ, so a test
always hands the *same* tensors (copied to the host) to the oracle.

Shapes follow the two pages that describe them:
  * the 3.8B GPT of "Training a 3.8B LLM to CORE 0.384 for $998"
    (hackernews.jp), architecture sentence and component/parameter table:
    28 decoder layers, GQA with 24 query / 8 KV heads of dim 128 at
    d_model 3072, relu^2 MLP;
  * the GPT trained by autoresearch (page 1, web3.cnoyu.systems review of
    ``train.py``): Muon owns the attention projections and MLP weights.
Matrix order is layer-major, then q, k, v, o, up, down.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

# Quintic coefficient triple used at every step by all five workloads.
QUINTIC = (3.4445, -4.7750, 2.0315)
# Cubic Newton-Schulz map x -> 1.5x - 0.5x^3 (converges to the polar factor).
CUBIC = (1.5, -0.5, 0.0)


@dataclass(frozen=True)
class Workload:
    name: str
    shapes: tuple            # ((rows, cols), ...) in step order
    grad_dtype: torch.dtype  # dtype of the gradients handed to the step
    grad_kind: str           # "gauss" | "lowrank" | "logspec"
    grad_std: float          # std of the Gaussian part
    buf_kind: str            # "zero" | "gauss"
    buf_std: float
    w_std: float             # weights ~ N(0, w_std), fp32 master copy
    mu: float
    lr: float
    n_steps: int
    coeffs: tuple            # one (a, b, c) triple, used at every step
    seed: int
    unit_scale: bool         # scale 1 for every matrix, else sqrt(max(1, rows/cols))
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def coeff_table(self):
        return [self.coeffs] * self.n_steps

    def scale(self, rows: int, cols: int) -> float:
        if self.unit_scale:
            return 1.0
        return math.sqrt(max(1.0, rows / cols))

    def oriented_groups(self):
        """{(m, n): count} with m = min(rows, cols), n = max(rows, cols)."""
        out: dict = {}
        for r, c in self.shapes:
            key = (min(r, c), max(r, c))
            out[key] = out.get(key, 0) + 1
        return out

    def ns_flops_counted(self) -> float:
        """Counted Newton-Schulz flops per step: sum over matrices of
        n_steps * (4 m^2 n + 2 m^3), m = min dim, n = max dim."""
        tot = 0.0
        for r, c in self.shapes:
            m, n = min(r, c), max(r, c)
            tot += 4.0 * m * m * n + 2.0 * m ** 3
        return tot * self.n_steps

    def n_elements(self) -> int:
        return sum(r * c for r, c in self.shapes)


def _gpt_layer_shapes(d_model: int, kv_dim: int, d_ff: int):
    # q, k, v, o as (out_features, in_features); up (d_ff x d), down (d x d_ff)
    return [(d_model, d_model), (kv_dim, d_model), (kv_dim, d_model),
            (d_model, d_model), (d_ff, d_model), (d_model, d_ff)]


def _gpt_shapes(n_layers, d_model, kv_dim, d_ff):
    return tuple(s for _ in range(n_layers)
                 for s in _gpt_layer_shapes(d_model, kv_dim, d_ff))


SINGLE_256x128 = Workload(
    name="single_256x128_fp32", shapes=((256, 128),),
    grad_dtype=torch.float32, grad_kind="gauss", grad_std=1.0,
    buf_kind="zero", buf_std=0.0, w_std=0.02, mu=0.95, lr=0.02,
    n_steps=5, coeffs=QUINTIC, seed=0, unit_scale=True)

GPT_D768 = Workload(
    name="gpt_d768_8layers", shapes=_gpt_shapes(8, 768, 768, 3072),
    grad_dtype=torch.bfloat16, grad_kind="gauss", grad_std=1e-3,
    buf_kind="gauss", buf_std=1e-3, w_std=0.02, mu=0.95, lr=0.02,
    n_steps=5, coeffs=QUINTIC, seed=2, unit_scale=False)

GPT_D1280 = Workload(
    name="gpt_d1280_20layers", shapes=_gpt_shapes(20, 1280, 1280, 5120),
    grad_dtype=torch.bfloat16, grad_kind="lowrank", grad_std=1e-4,
    buf_kind="zero", buf_std=0.0, w_std=0.02, mu=0.95, lr=0.02,
    n_steps=5, coeffs=QUINTIC, seed=3, unit_scale=False,
    extra={"rank": 64, "lowrank_entry_std": 1e-3})

GPT_3P8B = Workload(
    name="gpt_3.8b_28layers", shapes=_gpt_shapes(28, 3072, 1024, 12288),
    grad_dtype=torch.bfloat16, grad_kind="gauss", grad_std=1e-3,
    buf_kind="gauss", buf_std=1e-3, w_std=0.02, mu=0.95, lr=0.02,
    n_steps=5, coeffs=QUINTIC, seed=4, unit_scale=False)

STRESS_4096x16384 = Workload(
    name="stress_4096x16384_logspec",
    shapes=tuple([(4096, 16384)] * 64 + [(16384, 4096)] * 64),
    grad_dtype=torch.bfloat16, grad_kind="logspec", grad_std=0.0,
    buf_kind="zero", buf_std=0.0, w_std=0.02, mu=0.95, lr=0.02,
    n_steps=5, coeffs=QUINTIC, seed=5, unit_scale=False,
    extra={"s_min": 1e-4, "s_max": 1.0, "cubic_steps": 30})

WORKLOADS = {w.name: w for w in
             (SINGLE_256x128, GPT_D768, GPT_D1280, GPT_3P8B, STRESS_4096x16384)}

# Stream ids for the per-matrix generators.
_GRAD, _BUF, _W, _AUX, _V = 0, 1, 2, 3, 4


def _gen(device, seed: int, index: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + index * 16 + stream) % (2 ** 62))
    return g


def _randn(shape, gen, device, std=1.0):
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def haar_orthonormal(rows: int, cols: int, gen, device) -> torch.Tensor:
    """rows x cols (rows >= cols) with orthonormal columns, Haar-distributed:
    QR of a Gaussian matrix with the signs of diag(R) folded into Q."""
    assert rows >= cols
    z = torch.randn((rows, cols), generator=gen, device=device, dtype=torch.float32)
    q, r = torch.linalg.qr(z, mode="reduced")
    d = torch.sign(torch.diagonal(r))
    d[d == 0] = 1.0
    return q * d


def make_grad(w: Workload, index: int, device="cpu") -> torch.Tensor:
    rows, cols = w.shapes[index]
    g = _gen(device, w.seed, index, _GRAD)
    if w.grad_kind == "gauss":
        t = _randn((rows, cols), g, device, w.grad_std)
    elif w.grad_kind == "lowrank":
        k = w.extra["rank"]
        p = _randn((rows, k), g, device)
        q = _randn((cols, k), g, device)
        # entry std of the low-rank part = lowrank_entry_std
        t = (p @ q.T) * (w.extra["lowrank_entry_std"] / math.sqrt(k))
        t += _randn((rows, cols), g, device, w.grad_std)
    elif w.grad_kind == "logspec":
        m, n = min(rows, cols), max(rows, cols)
        u = haar_orthonormal(m, m, g, device)
        v = haar_orthonormal(n, m, g, device)
        lo, hi = math.log(w.extra["s_min"]), math.log(w.extra["s_max"])
        s = torch.exp(lo + (hi - lo) * torch.rand((m,), generator=g, device=device))
        t = (u * s) @ v.T                    # m x n
        if rows > cols:
            t = t.T.contiguous()
    else:
        raise ValueError(w.grad_kind)
    return t.to(w.grad_dtype).contiguous()


def make_buf(w: Workload, index: int, device="cpu") -> torch.Tensor:
    rows, cols = w.shapes[index]
    if w.buf_kind == "zero":
        return torch.zeros((rows, cols), device=device, dtype=torch.float32)
    return _randn((rows, cols), _gen(device, w.seed, index, _BUF), device, w.buf_std)


def make_weight(w: Workload, index: int, device="cpu") -> torch.Tensor:
    rows, cols = w.shapes[index]
    return _randn((rows, cols), _gen(device, w.seed, index, _W), device, w.w_std)


def make_inputs(w: Workload, device="cpu", indices=None):
    """Tensors for the matrices ``indices`` (default: all) of workload ``w``.

    Returns dict with lists ``params`` (fp32), ``grads`` (w.grad_dtype),
    ``bufs`` (fp32) and ``scales`` (python floats), plus ``indices``.
    """
    if indices is None:
        indices = range(len(w.shapes))
    indices = list(indices)
    out = {"params": [], "grads": [], "bufs": [], "scales": [], "indices": indices}
    for i in indices:
        r, c = w.shapes[i]
        out["grads"].append(make_grad(w, i, device))
        out["bufs"].append(make_buf(w, i, device))
        out["params"].append(make_weight(w, i, device))
        out["scales"].append(w.scale(r, c))
    return out


def make_second_moment(w: Workload, index: int, device="cpu") -> torch.Tensor:
    """A seeded NorMuon second-moment state for matrix ``index``:
    min(rows, cols) fp32 values, uniform in [0, 2/max(rows, cols)] (around
    the mean square 1/max(rows, cols) of an orthonormal-row update), so that
    one step already exercises the moving average."""
    rows, cols = w.shapes[index]
    g = _gen(device, w.seed, index, _V)
    u = torch.rand((min(rows, cols),), generator=g, device=device, dtype=torch.float32)
    return u * (2.0 / max(rows, cols))


def sample_indices(w: Workload, per_group: int):
    """First ``per_group`` matrices of every distinct raw (rows, cols) shape."""
    seen: dict = {}
    out = []
    for i, s in enumerate(w.shapes):
        if seen.get(s, 0) < per_group:
            seen[s] = seen.get(s, 0) + 1
            out.append(i)
    return out


def owner_indices(w: Workload, n_ranks: int, rank: int = 0):
    """Matrices that ``rank`` owns when the step is sharded by whole matrix
    over ``n_ranks`` GPUs: within every oriented shape (min and max of rows
    and cols), every ``n_ranks``-th matrix in list order, starting at
    ``rank``.  Each rank then runs the same oriented groups, 1/n_ranks as
    large (the 3.8B set's groups of 56 give 7 per rank on 8)."""
    if n_ranks < 1 or not 0 <= rank < n_ranks:
        raise ValueError("need n_ranks >= 1 and 0 <= rank < n_ranks")
    pos: dict = {}
    out = []
    for i, (r, c) in enumerate(w.shapes):
        key = (min(r, c), max(r, c))
        k = pos.get(key, 0)
        pos[key] = k + 1
        if k % n_ranks == rank:
            out.append(i)
    return out


def gaussian_matrix(rows: int, cols: int, seed: int, device="cpu",
                    dtype=torch.float32, std: float = 1.0) -> torch.Tensor:
    """A seeded N(0, std) matrix for the ragged/edge-shape parity cases."""
    g = _gen(device, seed, 0, _AUX)
    return _randn((rows, cols), g, device, std).to(dtype)


def gaussian_batch(batch: int, rows: int, cols: int, seed: int, device="cpu",
                   dtype=torch.float32, std: float = 1.0) -> torch.Tensor:
    """A (batch, rows, cols) stack of independent seeded N(0, std) matrices."""
    return torch.stack([
        _randn((rows, cols), _gen(device, seed, i, _AUX), device, std)
        for i in range(batch)]).to(dtype)


# Degenerate inputs for the edge-case parity tests: each a seeded fp32 matrix
# made on the host (numpy's PCG64), so that the GPU test and the CPU-side
# bf16 emulation see the same values.
DEGENERATE_KINDS = ("rank1", "one_element", "zero_rows", "dup_rows", "constant",
                    "col_scales", "row_scales")


def degenerate_matrix(kind: str, rows: int, cols: int, seed: int = 7,
                      device="cpu") -> torch.Tensor:
    """rank1: an outer product of two Gaussian vectors; one_element: a single
    non-zero entry; zero_rows: Gaussian with every other row zero; dup_rows:
    8 Gaussian rows, each repeated rows/8 times (rank 8); constant: all ones;
    col_scales / row_scales: Gaussian with columns / rows scaled by 10^u, u
    uniform in [-3, 3] (singular values spread over six decades)."""
    import numpy as np
    rng = np.random.default_rng([seed, DEGENERATE_KINDS.index(kind)])
    if kind == "rank1":
        x = np.outer(rng.standard_normal(rows), rng.standard_normal(cols))
    elif kind == "one_element":
        x = np.zeros((rows, cols))
        x[int(rng.integers(rows)), int(rng.integers(cols))] = -3.3  # not a bf16 value
    elif kind == "zero_rows":
        x = rng.standard_normal((rows, cols)) * (np.arange(rows)[:, None] % 2)
    elif kind == "dup_rows":
        assert rows % 8 == 0
        x = np.repeat(rng.standard_normal((8, cols)), rows // 8, axis=0)
    elif kind == "constant":
        x = np.ones((rows, cols))
    elif kind == "col_scales":
        x = rng.standard_normal((rows, cols)) * (10.0 ** rng.uniform(-3, 3, cols))[None, :]
    elif kind == "row_scales":
        x = rng.standard_normal((rows, cols)) * (10.0 ** rng.uniform(-3, 3, rows))[:, None]
    else:
        raise ValueError(kind)
    return torch.from_numpy(x.astype(np.float32)).to(device)

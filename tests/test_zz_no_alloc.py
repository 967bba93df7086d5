"""muon_step_static (no workspace argument, nothing allocated: the scratch is
the library's fixed per-GPU area) against muon_step with a caller workspace,
through the C ABI.  Both run the same kernels on the same inputs, so the
weights and momentum must agree bit for bit; two calls in a row, the second
on a smaller set, since the fixed area keeps the first call's contents."""
import dataclasses

import pytest
import torch

import muon_newton_schulz_step_amd as mn
import workloads as wl
from gpu_helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def clone_inputs(inputs):
    return {k: ([t.clone() for t in v] if k in ("params", "grads", "bufs") else v)
            for k, v in inputs.items()}


def both_ways(w, compute):
    a = wl.make_inputs(w, device=DEV)
    b = clone_inputs(a)
    mn.step(a["params"], a["grads"], a["bufs"], mu=w.mu, lr=w.lr, scales=a["scales"],
            coeffs=w.coeff_table, compute=compute, workspace=mn.Workspace())
    mn.step_static(b["params"], b["grads"], b["bufs"], mu=w.mu, lr=w.lr, scales=b["scales"],
                   coeffs=w.coeff_table, compute=compute)
    torch.cuda.synchronize()
    for k in range(len(w.shapes)):
        assert torch.equal(a["params"][k], b["params"][k]), (w.name, compute, k)
        assert torch.equal(a["bufs"][k], b["bufs"][k]), (w.name, compute, k)
    # the step did change the weights (not two untouched copies)
    w0 = wl.make_weight(w, 0, device=DEV)
    assert not torch.equal(b["params"][0], w0)


def static_need(shapes, compute):
    """Scratch of muon_step_static: its chunks run one after the other, so
    the largest chunk's workspace (one chunk = up to 64 matrices of one
    oriented shape)."""
    groups = {}
    for r, c in shapes:
        key = (min(r, c), max(r, c))
        groups[key] = groups.get(key, 0) + 1
    return max(mn.orthogonalize_workspace_bytes(min(cnt, 64), m, n, compute)
               for (m, n), cnt in groups.items())


def largest_d768_prefix(compute):
    """The most whole layers of the d768 GPT set whose step fits the fixed
    scratch area (all 8 on the bf16 path; fp32 carries X in 12 bytes per
    element and fits fewer)."""
    per_layer = 6
    for layers in range(8, 0, -1):
        shapes = wl.GPT_D768.shapes[:layers * per_layer]
        if static_need(shapes, compute) <= mn.MUON_STATIC_SCRATCH_BYTES:
            return dataclasses.replace(wl.GPT_D768, shapes=shapes)
    raise AssertionError("not even one d768 layer fits")


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_static_scratch_two_calls_match_workspace_step(compute):
    # first as many d768 layers as fit the fixed area (all 8 at bf16), then a
    # smaller mixed set with ragged, tall and wide shapes
    w = largest_d768_prefix(compute)
    announce("static scratch: d768 set,", len(w.shapes), "matrices", compute)
    if compute == "bf16":
        assert len(w.shapes) == len(wl.GPT_D768.shapes)
    both_ways(w, compute)
    announce("static scratch: small mixed set", compute)
    small = dataclasses.replace(wl.GPT_D768, shapes=((96, 256), (256, 96), (128, 128), (5, 3)))
    both_ways(small, compute)


def test_static_scratch_refuses_too_large_step():
    announce("static scratch: too large")
    p = torch.zeros(4096, 16384, device=DEV)
    g = torch.ones(4096, 16384, dtype=torch.bfloat16, device=DEV)
    b = torch.zeros(4096, 16384, device=DEV)
    with pytest.raises(mn.MuonError, match="WORKSPACE"):
        mn.step_static([p], [g], [b], mu=0.95, lr=0.02)
    torch.cuda.synchronize()
    assert torch.count_nonzero(p) == 0 and torch.count_nonzero(b) == 0

"""muon_step under stream capture: the library enqueues only kernel launches
on the caller's stream (no allocation, memset or synchronisation), so a
captured step replays as a graph.  Each replay must equal the same step run
eagerly, bitwise (the kernels are deterministic); replays reuse the captured
arguments (lr, mu, scales, coefficients)."""
import dataclasses

import pytest
import torch

import muon_newton_schulz_step_amd as mn
import workloads as wl
from gpu_helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_captured_step_replays_match_eager(compute):
    announce("graph capture", compute)
    w = dataclasses.replace(wl.GPT_D768, shapes=((96, 256), (256, 96), (128, 128), (300, 700),
                                                 (768, 768)))
    a = wl.make_inputs(w, device=DEV)  # replayed
    b = wl.make_inputs(w, device=DEV)  # eager, same seeded values
    need = mn.step_workspace_bytes(w.shapes, compute)
    ws_a = torch.empty(need, dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(need, dtype=torch.uint8, device=DEV)
    kw = dict(mu=w.mu, lr=w.lr, coeffs=w.coeff_table, compute=compute)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mn.step(a["params"], a["grads"], a["bufs"], scales=a["scales"], workspace=ws_a, **kw)
    torch.cuda.synchronize()
    for x, y in zip(a["params"] + a["bufs"], b["params"] + b["bufs"]):
        assert torch.equal(x, y)  # capturing ran nothing
    for replay in range(3):
        g.replay()
        mn.step(b["params"], b["grads"], b["bufs"], scales=b["scales"], workspace=ws_b, **kw)
        torch.cuda.synchronize()
        for x, y in zip(a["params"] + a["bufs"], b["params"] + b["bufs"]):
            assert torch.equal(x, y), replay
        # unrelated eager work between replays
        torch.randn(1 << 20, device=DEV).square().sum().item()
    del g

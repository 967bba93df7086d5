"""muon_step under stream capture: the library enqueues only kernel launches
on the caller's stream (no allocation, memset or synchronisation), so a
captured step replays as a graph.  Each replay must equal the same step run
eagerly, bitwise (the kernels are deterministic); replays reuse the captured
arguments (lr, mu, scales, coefficients).  Two sets: small chunks that run
concurrently on library lanes (forked off the captured stream and joined
back to it), and a large chunk beside a small one, which run in turn on the
captured stream; muon_step_ex with NorMuon and cautious decay, whose
row-statistics and weight passes are captured the same way; and the
allocation-free muon_step_static beside muon_orthogonalize in one graph."""
import dataclasses

import pytest
import torch

import muon_newton_schulz_step_amd as mn
import workloads as wl
from gpu_helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


SETS = {
    "concurrent": ((96, 256), (256, 96), (128, 128), (300, 700), (768, 768)),
    # 2 x 4096 x 16384 is a large chunk (2 x 4096^2 x 16384 multiply-adds per
    # update), so the step runs its two chunks in turn
    "in_turn": ((4096, 16384), (16384, 4096), (256, 512)),
}


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
@pytest.mark.parametrize("which", sorted(SETS))
def test_captured_step_replays_match_eager(compute, which):
    announce("graph capture", compute, which)
    w = dataclasses.replace(wl.GPT_D768, shapes=SETS[which])
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


@pytest.mark.parametrize("compute", ["bf16", "fp32"])
def test_captured_step_ex_replays_match_eager(compute):
    # NorMuon with cautious decay: the row-statistics and weight passes are
    # launches too, so the captured step replays like the plain one
    import ctypes
    from muon_newton_schulz_step_amd import _lib
    announce("graph capture step_ex", compute)
    w = dataclasses.replace(wl.GPT_D768, shapes=SETS["concurrent"])
    a = wl.make_inputs(w, device=DEV)
    b = wl.make_inputs(w, device=DEV)
    va = [wl.make_second_moment(w, i, device=DEV) for i in range(len(w.shapes))]
    vb = [v.clone() for v in va]
    opt = dict(weight_decay=0.1, cautious=True, beta2=0.95, normuon_eps=1e-8)
    o = _lib.MuonOptions(0.1, 1, 1, 0.95, 1e-8)
    need = mn.lib().muon_step_ex_workspace_bytes(
        len(w.shapes), _lib.int_array([r for r, _ in w.shapes]),
        _lib.int_array([c for _, c in w.shapes]), 0 if compute == "bf16" else 1, ctypes.byref(o))
    assert need > 0
    ws_a = torch.empty(need, dtype=torch.uint8, device=DEV)
    ws_b = torch.empty(need, dtype=torch.uint8, device=DEV)
    kw = dict(mu=w.mu, lr=w.lr, coeffs=w.coeff_table, compute=compute, **opt)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mn.step_ex(a["params"], a["grads"], a["bufs"], scales=a["scales"], second_moments=va,
                   workspace=ws_a, **kw)
    torch.cuda.synchronize()
    for x, y in zip(a["params"] + a["bufs"] + va, b["params"] + b["bufs"] + vb):
        assert torch.equal(x, y)  # capturing ran nothing
    for replay in range(3):
        g.replay()
        mn.step_ex(b["params"], b["grads"], b["bufs"], scales=b["scales"], second_moments=vb,
                   workspace=ws_b, **kw)
        torch.cuda.synchronize()
        for x, y in zip(a["params"] + a["bufs"] + va, b["params"] + b["bufs"] + vb):
            assert torch.equal(x, y), replay
        torch.randn(1 << 20, device=DEV).square().sum().item()
    del g


def test_captured_static_step_and_orthogonalize_replay():
    # the allocation-free entry point (its scratch is the library's own) and
    # orthogonalize with a caller workspace, captured and replayed likewise
    announce("graph capture static step and orthogonalize")
    w = dataclasses.replace(wl.GPT_D768, shapes=SETS["concurrent"])
    a = wl.make_inputs(w, device=DEV)
    b = wl.make_inputs(w, device=DEV)
    x = wl.gaussian_batch(3, 300, 700, seed=12, device=DEV)
    oa = torch.empty_like(x)
    ws = torch.empty(mn.orthogonalize_workspace_bytes(3, 300, 700, "bf16"), dtype=torch.uint8,
                     device=DEV)
    kw = dict(mu=w.mu, lr=w.lr, coeffs=w.coeff_table, compute="bf16")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mn.step_static(a["params"], a["grads"], a["bufs"], scales=a["scales"], **kw)
        mn.orthogonalize(x, w.coeff_table, compute="bf16", out=oa, workspace=ws)
    torch.cuda.synchronize()
    for replay in range(3):
        g.replay()
        mn.step_static(b["params"], b["grads"], b["bufs"], scales=b["scales"], **kw)
        ob = mn.orthogonalize(x, w.coeff_table, compute="bf16")
        torch.cuda.synchronize()
        for p, q in zip(a["params"] + a["bufs"], b["params"] + b["bufs"]):
            assert torch.equal(p, q), replay
        assert torch.equal(oa, ob), replay
        torch.randn(1 << 20, device=DEV).square().sum().item()
    del g

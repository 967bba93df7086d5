"""The library's choice of GEMM tile per launch, seen from outside: the
flops its launches execute (recorded per launch from its tile counts) and
its number of final launches must equal what bench.py's model of that
choice predicts, since the counter summaries and the executed-flop figures
are matched against that model."""
import dataclasses

import pytest
import torch

import bench
import muon_newton_schulz_step_amd as mn
import workloads as wl
from gpu_helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GEMM_KINDS = ("gram", "gramq", "poly", "update", "final")

CASES = {
    "d768": wl.GPT_D768,
    "d1280": wl.GPT_D1280,
    "3.8b": wl.GPT_3P8B,
    # one chunk each, around the points where the choice changes
    "sets": dataclasses.replace(
        wl.GPT_D768, shapes=((1280, 1280),) * 12 + ((1280, 1280 + 1),) * 16
        + ((1024, 1024),) * 24 + ((2048, 8192),) * 2 + ((8192, 2048),) * 2
        + ((768, 3072),) * 3 + ((3072, 768),) * 2),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_executed_flops_and_finals_match_the_model(case):
    w = CASES[case]
    announce("tile choice", case, len(w.shapes))
    inp = wl.make_inputs(w, device=DEV)
    mn.timing_enable(True)
    mn.timing_read()
    try:
        mn.step(inp["params"], inp["grads"], inp["bufs"], mu=w.mu, lr=w.lr,
                scales=inp["scales"], coeffs=w.coeff_table)
        torch.cuda.synchronize()
    finally:
        mn.timing_enable(False)
    recs = mn.timing_read()
    executed = sum(r["exec_flops"] for r in recs if r["kind"] in GEMM_KINDS)
    assert executed == pytest.approx(bench.ns_flops_executed(w), rel=1e-12)
    finals = sum(1 for r in recs if r["kind"] == "final")
    assert finals == sum(1 for k, _, _ in bench.launch_sequence(w) if k == "final")

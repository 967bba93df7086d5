"""The streaming kernel variants (nontemporal X-state, weight, gradient and
momentum accesses, taken for chunks whose X state exceeds the last-level
cache) change only where data is cached, never a value: a step run with
them forced (MUON_STREAM=1, read once per process, so in a child process)
must equal the default run of the same small, cached-variant step bitwise,
for muon_step and for muon_step_ex with NorMuon and cautious decay."""
import dataclasses
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import muon_newton_schulz_step_amd as mn
import workloads as wl
from gpu_helpers import announce

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SHAPES = ((96, 256), (256, 96), (300, 700), (700, 300), (512, 2048))
OPT = dict(weight_decay=0.1, cautious=True, beta2=0.95, normuon_eps=1e-8)


def run_steps(device="cuda:0"):
    """Both entry points on the same seeded inputs; everything they write,
    as host arrays."""
    w = dataclasses.replace(wl.GPT_D768, shapes=SHAPES)
    out = {}
    for ex in (False, True):
        inp = wl.make_inputs(w, device=device)
        kw = dict(mu=w.mu, lr=w.lr, scales=inp["scales"], coeffs=w.coeff_table, compute="bf16")
        if ex:
            vs = [wl.make_second_moment(w, i, device=device) for i in range(len(SHAPES))]
            mn.step_ex(inp["params"], inp["grads"], inp["bufs"], second_moments=vs, **kw, **OPT)
        else:
            vs = []
            mn.step(inp["params"], inp["grads"], inp["bufs"], **kw)
        torch.cuda.synchronize()
        tag = "ex" if ex else "plain"
        for name, ts in (("w", inp["params"]), ("buf", inp["bufs"]), ("v", vs)):
            for k, t in enumerate(ts):
                out[f"{tag}_{name}{k}"] = t.cpu().numpy()
    return out


def test_streaming_variants_match_cached_bitwise(tmp_path):
    announce("streaming vs cached variants", SHAPES)
    path = tmp_path / "stream.npz"
    code = ("import sys, numpy as np; sys.path[:0] = [%r, %r]; "
            "import test_gpu_stream as t; np.savez(%r, **t.run_steps())"
            % (ROOT, os.path.join(ROOT, "tests"), str(path)))
    env = dict(os.environ, MUON_STREAM="1")
    proc = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT,
                          capture_output=True, text=True, timeout=300)
    assert proc.returncode == 0, proc.stdout[-2000:] + proc.stderr[-2000:]
    cached = run_steps()
    streamed = np.load(path)
    assert sorted(streamed.files) == sorted(cached)
    for key, val in cached.items():
        assert np.array_equal(streamed[key], val), key

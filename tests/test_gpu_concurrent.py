"""Small steps run their chunks concurrently, each on a stream lane of its
own and in its own workspace region, forked off the caller's stream and
joined back to it.  That changes when kernels run, never a value:

  * the same concurrent step repeated from the same inputs is bitwise the
    same every time (a regression test: with another kernel beside it on a
    CU, a wave's LDS operand reads of a k-tile stage could still be queued
    when the workgroup refilled that stage, and results varied from run to
    run until the waves waited for their own reads before the hand-over);
  * it equals, bitwise, the same step with the chunks run one after the
    other (MUON_CONCURRENT=0, read once per process, so in a child process),
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
# the d768 GPT set plus two more oriented shapes: four chunks, four lanes
SHAPES = wl.GPT_D768.shapes + ((512, 2048), (2048, 512), (96, 256), (256, 96), (96, 256))
OPT = dict(weight_decay=0.1, cautious=True, beta2=0.95, normuon_eps=1e-8)


def run_steps(repeats=1, device="cuda:0"):
    """Both entry points on the same seeded inputs, each `repeats` times from
    fresh copies; everything they write, as host arrays (one dict per run)."""
    w = dataclasses.replace(wl.GPT_D768, shapes=SHAPES)
    base = wl.make_inputs(w, device=device)
    vs0 = [wl.make_second_moment(w, i, device=device) for i in range(len(SHAPES))]
    runs = []
    for _ in range(repeats):
        out = {}
        for ex in (False, True):
            inp = {k: ([t.clone() for t in v] if k in ("params", "grads", "bufs") else v)
                   for k, v in base.items()}
            kw = dict(mu=w.mu, lr=w.lr, scales=inp["scales"], coeffs=w.coeff_table,
                      compute="bf16")
            if ex:
                vs = [v.clone() for v in vs0]
                mn.step_ex(inp["params"], inp["grads"], inp["bufs"], second_moments=vs, **kw,
                           **OPT)
            else:
                vs = []
                mn.step(inp["params"], inp["grads"], inp["bufs"], **kw)
            torch.cuda.synchronize()
            tag = "ex" if ex else "plain"
            for name, ts in (("w", inp["params"]), ("buf", inp["bufs"]), ("v", vs)):
                for k, t in enumerate(ts):
                    out[f"{tag}_{name}{k}"] = t.cpu().numpy()
        runs.append(out)
    return runs


def test_concurrent_step_repeats_bitwise():
    announce("concurrent chunks, 4 repeats", len(SHAPES), "matrices")
    assert len(mn.plan_groups(SHAPES)[1]) == 4
    runs = run_steps(repeats=4)
    for r in runs[1:]:
        for key, val in runs[0].items():
            assert np.array_equal(r[key], val), key


def test_concurrent_equals_sequential_bitwise(tmp_path):
    announce("concurrent vs sequential chunks", len(SHAPES), "matrices")
    path = tmp_path / "seq.npz"
    code = ("import sys, numpy as np; sys.path[:0] = [%r, %r]; "
            "import test_gpu_concurrent as t; np.savez(%r, **t.run_steps()[0])"
            % (ROOT, os.path.join(ROOT, "tests"), str(path)))
    env = dict(os.environ, MUON_CONCURRENT="0")
    proc = subprocess.run([sys.executable, "-c", code], env=env, cwd=ROOT,
                          capture_output=True, text=True, timeout=300)
    assert proc.returncode == 0, proc.stdout[-2000:] + proc.stderr[-2000:]
    conc = run_steps()[0]
    seq = np.load(path)
    assert sorted(seq.files) == sorted(conc)
    for key, val in conc.items():
        assert np.array_equal(seq[key], val), key


def test_two_streams_with_default_workspaces():
    """Two steps at once on two streams, both with the binding's default
    workspace: each (device, stream) gets its own, so they share no scratch
    and each equals, bitwise, the same step run alone."""
    announce("two streams, default workspaces")
    w = dataclasses.replace(wl.GPT_D768, shapes=((384, 1536), (1536, 384), (384, 384)) * 4)
    alone, together = [], []
    for seed_shift in (0, 1):
        ws = dataclasses.replace(w, seed=w.seed + 10 * seed_shift)
        inp = wl.make_inputs(ws, device="cuda:0")
        mn.step(inp["params"], inp["grads"], inp["bufs"], mu=w.mu, lr=w.lr,
                scales=inp["scales"], coeffs=w.coeff_table, workspace=mn.Workspace())
        torch.cuda.synchronize()
        alone.append([p.clone() for p in inp["params"]])
        together.append((ws, wl.make_inputs(ws, device="cuda:0")))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for (ws, inp), s in zip(together, streams):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            mn.step(inp["params"], inp["grads"], inp["bufs"], mu=w.mu, lr=w.lr,
                    scales=inp["scales"], coeffs=w.coeff_table)
    torch.cuda.synchronize()
    for a, (_, inp) in zip(alone, together):
        for x, y in zip(a, inp["params"]):
            assert torch.equal(x, y)
    keys = [k for k in mn._default_ws if k[0] == "cuda:0"]
    assert len({k[1] for k in keys}) >= 2


def test_host_threads_stepping_at_once():
    """Four host threads, each with its own stream and workspace, step
    small sets whose chunks run on the library's shared stream lanes (the
    ctypes calls release the interpreter lock, so the library's entry points
    run at the same time): every result equals, bitwise, the same step run
    alone."""
    import threading
    announce("four host threads")
    w = dataclasses.replace(wl.GPT_D768, shapes=((96, 256), (256, 96), (128, 128), (300, 700)))
    sets = [wl.make_inputs(dataclasses.replace(w, seed=w.seed + 7 * t), device="cuda:0")
            for t in range(4)]
    need = mn.step_workspace_bytes(w.shapes, "bf16")
    expect = []
    for inp in sets:
        p = [x.clone() for x in inp["params"]]
        b = [x.clone() for x in inp["bufs"]]
        for _ in range(3):
            mn.step(p, inp["grads"], b, mu=w.mu, lr=w.lr, scales=inp["scales"],
                    coeffs=w.coeff_table, workspace=torch.empty(need, dtype=torch.uint8,
                                                                device="cuda:0"))
        torch.cuda.synchronize()
        expect.append(p + b)
    streams = [torch.cuda.Stream() for _ in sets]
    wss = [torch.empty(need, dtype=torch.uint8, device="cuda:0") for _ in sets]
    torch.cuda.synchronize()
    errors = []

    def worker(t):
        try:
            inp, s = sets[t], streams[t]
            with torch.cuda.stream(s):
                for _ in range(3):
                    mn.step(inp["params"], inp["grads"], inp["bufs"], mu=w.mu, lr=w.lr,
                            scales=inp["scales"], coeffs=w.coeff_table, workspace=wss[t])
            s.synchronize()
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(e)
    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads)
    assert not errors, errors
    torch.cuda.synchronize()
    for inp, exp in zip(sets, expect):
        for x, y in zip(inp["params"] + inp["bufs"], exp):
            assert torch.equal(x, y)

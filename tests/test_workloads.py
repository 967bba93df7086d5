"""Seeded synthetic inputs: determinism, shapes, dtypes and distributions."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import workloads as wl


def test_shapes_and_groups():
    assert wl.GPT_D768.oriented_groups() == {(768, 768): 32, (768, 3072): 16}
    assert wl.GPT_D1280.oriented_groups() == {(1280, 1280): 80, (1280, 5120): 40}
    assert wl.STRESS_4096x16384.oriented_groups() == {(4096, 16384): 128}
    assert len(wl.GPT_D768.shapes) == 48 and len(wl.GPT_D1280.shapes) == 120
    # layer-major then q, k, v, o, up, down
    assert wl.GPT_3P8B.shapes[:6] == ((3072, 3072), (1024, 3072), (1024, 3072),
                                      (3072, 3072), (12288, 3072), (3072, 12288))


def test_deterministic_and_subsettable():
    w = wl.GPT_D768
    a = wl.make_inputs(w, indices=[0, 5])
    b = wl.make_inputs(w, indices=[5])
    assert torch.equal(a["grads"][1], b["grads"][0])
    assert torch.equal(a["bufs"][1], b["bufs"][0])
    assert torch.equal(a["params"][1], b["params"][0])
    assert a["grads"][0].dtype == torch.bfloat16
    assert a["bufs"][0].dtype == torch.float32
    # different streams differ
    assert not torch.equal(a["bufs"][0], a["params"][0])


def test_single_workload_distribution():
    w = wl.SINGLE_256x128
    x = wl.make_inputs(w)
    g = x["grads"][0]
    assert g.dtype == torch.float32 and g.shape == (256, 128)
    assert abs(float(g.std()) - 1.0) < 0.02
    assert abs(float(x["params"][0].std()) - 0.02) < 0.001
    assert float(x["bufs"][0].abs().max()) == 0.0
    assert x["scales"] == [1.0]


def test_scale_rule():
    w = wl.GPT_3P8B
    assert w.scale(12288, 3072) == 2.0
    assert w.scale(3072, 12288) == 1.0
    assert w.scale(3072, 3072) == 1.0


def test_lowrank_grad_spectrum():
    w = dataclasses.replace(wl.GPT_D1280, shapes=((160, 640),))
    g = wl.make_grad(w, 0).double().numpy()
    s = np.linalg.svd(g, compute_uv=False)
    # rank-64 part dominates; noise floor ~ 1e-4 * (sqrt(640) + sqrt(160))
    assert s[63] > 3 * s[64]
    assert s[64] < 1e-4 * (math.sqrt(640) + math.sqrt(160)) * 1.3


def test_logspec_grad_spectrum():
    w = dataclasses.replace(wl.STRESS_4096x16384, shapes=((64, 256), (256, 64)))
    for i in range(2):
        g = wl.make_grad(w, i).double().numpy()
        s = np.linalg.svd(g, compute_uv=False)
        assert s.max() <= 1.02 and s.min() >= 1e-4 * 0.5
        assert s.max() / s.min() > 100


def test_ragged_helpers():
    a = wl.gaussian_batch(3, 5, 7, seed=1)
    assert a.shape == (3, 5, 7)
    assert torch.equal(a[0], wl.gaussian_batch(1, 5, 7, seed=1)[0])
    assert wl.sample_indices(wl.GPT_3P8B, 2) == [0, 1, 2, 3, 4, 5, 10, 11]


def test_owner_indices_partition_every_oriented_group():
    """Sharding by whole matrix: over n ranks every matrix has exactly one
    owner, and each rank holds 1/n of every oriented group (the 3.8B set's
    groups of 56: 7 each on 8 ranks)."""
    w = wl.GPT_3P8B
    owners = {}
    for rank in range(8):
        idx = wl.owner_indices(w, 8, rank)
        groups = {}
        for i in idx:
            assert i not in owners
            owners[i] = rank
            r, c = w.shapes[i]
            groups[(min(r, c), max(r, c))] = groups.get((min(r, c), max(r, c)), 0) + 1
        assert groups == {(3072, 3072): 7, (1024, 3072): 7, (3072, 12288): 7}
    assert sorted(owners) == list(range(len(w.shapes)))
    assert wl.owner_indices(w, 1) == list(range(len(w.shapes)))
    for bad in ((0, 0), (8, 8), (8, -1)):
        with pytest.raises(ValueError):
            wl.owner_indices(w, *bad)

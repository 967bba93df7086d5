"""C ABI checks that need no GPU: symbols, argument validation, workspace
sizing and the grouping planner.  Every rejected call returns before any HIP
call is made, so these run on a machine without a GPU."""
import ctypes
import os
import re

import pytest

import muon_newton_schulz_step_amd as mn
from muon_newton_schulz_step_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
Q = [(3.4445, -4.7750, 2.0315)] * 5
FAKE = 0x10000  # 16- and 256-byte aligned; never dereferenced by rejected calls


def header_functions():
    src = open(os.path.join(ROOT, "include", "muon.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(muon_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = mn.lib()
    declared = header_functions()
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings():
    for st in (0, -1, -2, -3, -4):
        assert mn.status_string(st).startswith("MUON_")
    assert "unknown" in mn.status_string(7)


def orth(in_ptr=FAKE, in_dtype=0, out_ptr=FAKE * 2, out_dtype=1, batch=1, rows=8, cols=16,
         stride=None, coeffs=Q, n_steps=None, eps=1e-7, compute=0, ws=FAKE * 1024,
         ws_bytes=None):
    lib = mn.lib()
    if stride is None:
        stride = rows * cols
    if n_steps is None:
        n_steps = len(coeffs)
    if ws_bytes is None:
        ws_bytes = lib.muon_orthogonalize_workspace_bytes(max(batch, 1), rows, cols, compute)
    table = _lib.coeff_array(coeffs) if coeffs is not None else None
    return lib.muon_orthogonalize(
        ctypes.c_void_p(in_ptr), in_dtype, ctypes.c_void_p(out_ptr), out_dtype, batch, rows,
        cols, stride, table, n_steps, eps, compute, ctypes.c_void_p(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(batch=-1), mn.MUON_ERR_INVALID_ARG),
    (dict(batch=0), mn.MUON_OK),                       # nothing enqueued
    (dict(in_ptr=0), mn.MUON_ERR_INVALID_ARG),
    (dict(out_ptr=0), mn.MUON_ERR_INVALID_ARG),
    (dict(rows=0), mn.MUON_ERR_INVALID_ARG),
    (dict(cols=-3), mn.MUON_ERR_INVALID_ARG),
    (dict(in_dtype=5), mn.MUON_ERR_INVALID_ARG),
    (dict(out_dtype=-1), mn.MUON_ERR_INVALID_ARG),
    (dict(compute=2), mn.MUON_ERR_INVALID_ARG),
    (dict(n_steps=0), mn.MUON_ERR_INVALID_ARG),
    (dict(coeffs=Q * 13, n_steps=65), mn.MUON_ERR_INVALID_ARG),
    (dict(coeffs=None, n_steps=5), mn.MUON_ERR_INVALID_ARG),
    (dict(coeffs=[(float("nan"), 0.0, 0.0)]), mn.MUON_ERR_INVALID_ARG),
    (dict(eps=-1.0), mn.MUON_ERR_INVALID_ARG),
    (dict(eps=float("inf")), mn.MUON_ERR_INVALID_ARG),
    (dict(stride=8 * 16 - 1), mn.MUON_ERR_INVALID_ARG),
    (dict(in_ptr=FAKE + 2), mn.MUON_ERR_INVALID_ARG),   # misaligned
    (dict(out_ptr=FAKE + 8), mn.MUON_ERR_INVALID_ARG),  # overlaps input, not equal
    # the same pointer but a wider output type: the output of matrix i
    # would overwrite inputs of later matrices (or chunks) before they are read
    (dict(out_ptr=FAKE, in_dtype=0, out_dtype=1), mn.MUON_ERR_INVALID_ARG),
    (dict(out_ptr=FAKE, in_dtype=1, out_dtype=0, batch=100), mn.MUON_ERR_INVALID_ARG),
    (dict(rows=1 << 16, cols=1 << 16), mn.MUON_ERR_INVALID_ARG),  # too many elements
    (dict(ws=0), mn.MUON_ERR_WORKSPACE),
    (dict(ws_bytes=1024), mn.MUON_ERR_WORKSPACE),
    (dict(ws=FAKE * 1024 + 16), mn.MUON_ERR_WORKSPACE),  # workspace misaligned
    (dict(ws=FAKE), mn.MUON_ERR_INVALID_ARG),            # workspace overlaps input
])
def test_orthogonalize_rejects_before_enqueue(kw, expect):
    assert orth(**kw) == expect


def step_call(n=2, rows=(8, 16), cols=(16, 8), params=None, grads=None, bufs=None,
              param_dtype=1, grad_dtype=0, mu=0.95, lr=0.02, scales=(1.0, 1.0), coeffs=Q,
              n_steps=None, eps=1e-7, compute=0, ws=FAKE * 4096, ws_bytes=None):
    lib = mn.lib()
    params = params if params is not None else [FAKE * (i + 1) * 64 for i in range(n)]
    grads = grads if grads is not None else [FAKE * (i + 1) * 64 + 4096 for i in range(n)]
    bufs = bufs if bufs is not None else [FAKE * (i + 1) * 64 + 8192 for i in range(n)]
    r, c = _lib.int_array(rows), _lib.int_array(cols)
    if ws_bytes is None:
        ws_bytes = lib.muon_step_workspace_bytes(n, r, c, compute) if n > 0 else 0
    if n_steps is None:
        n_steps = len(coeffs)
    return lib.muon_step(
        n, r, c, _lib.ptr_array(params), param_dtype, _lib.ptr_array(grads), grad_dtype,
        _lib.ptr_array(bufs), mu, lr, _lib.float_array(scales), _lib.coeff_array(coeffs),
        n_steps, eps, compute, ctypes.c_void_p(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(n=-1), mn.MUON_ERR_INVALID_ARG),
    (dict(n=0), mn.MUON_OK),
    (dict(rows=(8, 0)), mn.MUON_ERR_INVALID_ARG),
    (dict(params=[FAKE * 64, 0]), mn.MUON_ERR_INVALID_ARG),
    (dict(grads=[FAKE * 64 + 4096, FAKE * 128 + 4098]), mn.MUON_ERR_INVALID_ARG),
    (dict(bufs=[FAKE * 64, FAKE * 128 + 8192]), mn.MUON_ERR_INVALID_ARG),  # buf aliases param
    (dict(param_dtype=0), mn.MUON_ERR_UNSUPPORTED),
    (dict(grad_dtype=3), mn.MUON_ERR_INVALID_ARG),
    (dict(mu=float("nan")), mn.MUON_ERR_INVALID_ARG),
    (dict(lr=float("inf")), mn.MUON_ERR_INVALID_ARG),
    (dict(scales=(1.0, float("nan"))), mn.MUON_ERR_INVALID_ARG),
    (dict(n_steps=65, coeffs=Q * 13), mn.MUON_ERR_INVALID_ARG),
    (dict(ws=0), mn.MUON_ERR_WORKSPACE),
    (dict(ws_bytes=100), mn.MUON_ERR_WORKSPACE),
    (dict(ws=FAKE * 64), mn.MUON_ERR_INVALID_ARG),           # workspace overlaps a weight
    (dict(ws=FAKE * 128 + 4096), mn.MUON_ERR_INVALID_ARG),   # ... a gradient
    (dict(ws=FAKE * 64 + 8192 - 256), mn.MUON_ERR_INVALID_ARG),  # ... a momentum buffer
    # across matrices: two weights in one buffer, a weight over the other
    # matrix's (bf16) gradient, momentum buffers that overlap by four elements,
    # a momentum buffer over the other matrix's gradient
    (dict(params=[FAKE * 64, FAKE * 64]), mn.MUON_ERR_INVALID_ARG),
    (dict(params=[FAKE * 64, FAKE * 64 + 4096 + 240]), mn.MUON_ERR_INVALID_ARG),
    (dict(bufs=[FAKE * 64 + 8192, FAKE * 64 + 8192 + 496]), mn.MUON_ERR_INVALID_ARG),
    (dict(bufs=[FAKE * 64 + 8192, FAKE * 64 + 4096]), mn.MUON_ERR_INVALID_ARG),
])
def test_step_rejects_before_enqueue(kw, expect):
    assert step_call(**kw) == expect


def step_ex_call(n=2, rows=(8, 16), cols=(16, 8), vs=None, opt=None, ws=FAKE * 4096,
                 ws_bytes=None, no_opt=False, no_vs=False):
    lib = mn.lib()
    params = [FAKE * (i + 1) * 64 for i in range(n)]
    grads = [FAKE * (i + 1) * 64 + 4096 for i in range(n)]
    bufs = [FAKE * (i + 1) * 64 + 8192 for i in range(n)]
    if vs is None:
        vs = [FAKE * (i + 1) * 64 + 16384 for i in range(n)]
    if opt is None:
        opt = dict(weight_decay=0.1, cautious=1, normuon=1, beta2=0.95, normuon_eps=1e-8)
    o = _lib.MuonOptions(**opt)
    r, c = _lib.int_array(rows), _lib.int_array(cols)
    if ws_bytes is None:
        ws_bytes = lib.muon_step_ex_workspace_bytes(n, r, c, 0, ctypes.byref(o)) if n > 0 else 0
    return lib.muon_step_ex(
        n, r, c, _lib.ptr_array(params), 1, _lib.ptr_array(grads), 0, _lib.ptr_array(bufs),
        None if no_vs else _lib.ptr_array(vs), 0.95, 0.02, _lib.float_array([1.0] * n),
        _lib.coeff_array(Q), 5, 1e-7, 0, None if no_opt else ctypes.byref(o),
        ctypes.c_void_p(ws), ws_bytes, None)


OPT = dict(weight_decay=0.1, cautious=1, normuon=1, beta2=0.95, normuon_eps=1e-8)


@pytest.mark.parametrize("kw,expect", [
    (dict(n=0), mn.MUON_OK),
    (dict(opt={**OPT, "weight_decay": -0.1}), mn.MUON_ERR_INVALID_ARG),
    (dict(opt={**OPT, "weight_decay": float("nan")}), mn.MUON_ERR_INVALID_ARG),
    (dict(opt={**OPT, "cautious": 2}), mn.MUON_ERR_INVALID_ARG),
    (dict(opt={**OPT, "normuon": -1}), mn.MUON_ERR_INVALID_ARG),
    (dict(opt={**OPT, "beta2": 1.5}), mn.MUON_ERR_INVALID_ARG),
    (dict(opt={**OPT, "beta2": float("nan")}), mn.MUON_ERR_INVALID_ARG),
    (dict(opt={**OPT, "normuon_eps": -1.0}), mn.MUON_ERR_INVALID_ARG),
    (dict(opt={**OPT, "normuon_eps": float("inf")}), mn.MUON_ERR_INVALID_ARG),
    (dict(no_vs=True), mn.MUON_ERR_INVALID_ARG),                    # NorMuon without buffers
    (dict(vs=[FAKE * 64 + 16384, 0]), mn.MUON_ERR_INVALID_ARG),     # one missing
    (dict(vs=[FAKE * 64 + 16386, FAKE * 128 + 16384]), mn.MUON_ERR_INVALID_ARG),  # misaligned
    (dict(vs=[FAKE * 64 + 8, FAKE * 128 + 16384]), mn.MUON_ERR_INVALID_ARG),      # overlaps W
    (dict(ws=0), mn.MUON_ERR_WORKSPACE),
    (dict(vs=[FAKE * 4096 + 256, FAKE * 128 + 16384]), mn.MUON_ERR_INVALID_ARG),  # in workspace
    # the two (8, 16) and (16, 8) matrices keep 8 floats of second moment
    # each: sharing one buffer, or overlapping the other matrix's weight
    (dict(vs=[FAKE * 64 + 16384, FAKE * 64 + 16384]), mn.MUON_ERR_INVALID_ARG),
    (dict(vs=[FAKE * 64 + 16384, FAKE * 64 + 16384 + 28]), mn.MUON_ERR_INVALID_ARG),
    (dict(vs=[FAKE * 64 + 16384, FAKE * 64 + 508]), mn.MUON_ERR_INVALID_ARG),
])
def test_step_ex_rejects_before_enqueue(kw, expect):
    assert step_ex_call(**kw) == expect


def test_step_ex_workspace_sizes():
    lib = mn.lib()
    rows, cols = (3072, 12288), (12288, 3072)   # one chunk: 2 x (3072, 12288)
    r, c = _lib.int_array(rows), _lib.int_array(cols)
    plain = lib.muon_step_workspace_bytes(2, r, c, 0)
    assert lib.muon_step_ex_workspace_bytes(2, r, c, 0, None) == plain
    wd_only = _lib.MuonOptions(0.1, 1, 0, 0.0, 0.0)
    assert lib.muon_step_ex_workspace_bytes(2, r, c, 0, ctypes.byref(wd_only)) == plain
    nm = _lib.MuonOptions(0.0, 1, 1, 0.9, 1e-8)
    # NorMuon adds, for 2 x (3072, 12288) (one wide, one tall): the per-row
    # scales (3072 floats each) and, on the bf16 path, the last update's row
    # sums (12288 / 64 blocks of 3072 floats each)
    assert lib.muon_step_ex_workspace_bytes(2, r, c, 0, ctypes.byref(nm)) == (
        plain + 2 * 3072 * 4 + 2 * (12288 // 64) * 3072 * 4)
    plain32 = lib.muon_step_workspace_bytes(2, r, c, 1)
    assert lib.muon_step_ex_workspace_bytes(2, r, c, 1, ctypes.byref(nm)) == plain32 + 2 * 3072 * 4
    bad = _lib.MuonOptions(-1.0, 1, 0, 0.0, 0.0)
    assert lib.muon_step_ex_workspace_bytes(2, r, c, 0, ctypes.byref(bad)) == 0
    # with NorMuon the plain size is too small
    assert step_ex_call(ws_bytes=lib.muon_step_workspace_bytes(
        2, _lib.int_array((8, 16)), _lib.int_array((16, 8)), 0)) == mn.MUON_ERR_WORKSPACE


def test_workspace_sizes():
    lib = mn.lib()
    small = lib.muon_orthogonalize_workspace_bytes(1, 256, 128, 0)
    assert small > 0 and small % 256 == 0
    # transposed shapes share the oriented layout
    assert small == lib.muon_orthogonalize_workspace_bytes(1, 128, 256, 0)
    # fp32 compute needs more than bf16
    assert lib.muon_orthogonalize_workspace_bytes(1, 256, 128, 1) > small
    # batches are processed in chunks of at most 64 matrices
    assert (lib.muon_orthogonalize_workspace_bytes(200, 256, 128, 0)
            == lib.muon_orthogonalize_workspace_bytes(64, 256, 128, 0))
    assert lib.muon_orthogonalize_workspace_bytes(0, 256, 128, 0) == 0
    assert lib.muon_orthogonalize_workspace_bytes(1, 0, 128, 0) == 0
    # 3.8B matrix set: the largest group is 56 x (3072, 12288)
    shapes = [(3072, 3072), (1024, 3072), (1024, 3072), (3072, 3072),
              (12288, 3072), (3072, 12288)] * 28
    ws = mn.step_workspace_bytes(shapes)
    assert ws == lib.muon_orthogonalize_workspace_bytes(56, 3072, 12288, 0)
    # bf16: X as hi (twice, 2 bytes each) and lo (1 byte) planes, A and B
    # (bf16), A's residual and the product T of the Q A Q steps (bf16; this
    # group has N = 4M and M >= 2048), the fp32 norm partials of 64 x 64 tiles
    # and the per-matrix 1/norm
    need = 56 * (5 * 3072 * 12288 + 4 * 3072 * 3072 * 2
                 + (3072 // 64) * (12288 // 64) * 4 + 4)
    assert need <= ws < need + 8 * 256


def test_plan_groups_by_oriented_shape():
    shapes = [(768, 768), (768, 3072), (3072, 768), (768, 768), (5, 3), (3, 5), (4, 4)]
    gof, groups = mn.plan_groups(shapes)
    assert gof == [0, 1, 1, 0, 2, 2, 3]
    assert groups == [(768, 768, 2), (768, 3072, 2), (3, 5, 2), (4, 4, 1)]
    gof, groups = mn.plan_groups([])
    assert gof == [] and groups == []
    shapes = [(3072, 3072), (1024, 3072), (1024, 3072), (3072, 3072),
              (12288, 3072), (3072, 12288)] * 28
    _, groups = mn.plan_groups(shapes)
    assert groups == [(3072, 3072, 56), (1024, 3072, 56), (3072, 12288, 56)]


def test_timing_log_empty_without_launches():
    prev = mn.timing_enable(True)
    assert mn.timing_read() == []
    mn.timing_enable(prev)


def test_binding_refuses_host_tensors():
    # the library takes raw device pointers: host tensors never reach it
    import torch
    p, g, b = torch.zeros(8, 16), torch.zeros(8, 16, dtype=torch.bfloat16), torch.zeros(8, 16)
    with pytest.raises(ValueError, match="GPU"):
        mn.step([p], [g], [b], mu=0.95, lr=0.02)
    with pytest.raises(ValueError, match="GPU"):
        mn.step_ex([p], [g], [b], mu=0.95, lr=0.02, weight_decay=0.1,
                   second_moments=[torch.zeros(8)], beta2=0.95, normuon_eps=1e-8)
    with pytest.raises(ValueError, match="GPU"):
        mn.orthogonalize(torch.zeros(8, 16))


def static_call(n=2, rows=(8, 16), cols=(16, 8), params=None, grads=None, bufs=None,
                param_dtype=1, grad_dtype=0, mu=0.95, lr=0.02, scales=None, coeffs=Q,
                n_steps=None, eps=1e-7, compute=0):
    lib = mn.lib()
    params = params if params is not None else [FAKE * (i + 1) * 64 for i in range(n)]
    grads = grads if grads is not None else [FAKE * (i + 1) * 64 + 4096 for i in range(n)]
    bufs = bufs if bufs is not None else [FAKE * (i + 1) * 64 + 8192 for i in range(n)]
    scales = scales if scales is not None else [1.0] * n
    if n_steps is None:
        n_steps = len(coeffs)
    return lib.muon_step_static(
        n, _lib.int_array(rows), _lib.int_array(cols), _lib.ptr_array(params), param_dtype,
        _lib.ptr_array(grads), grad_dtype, _lib.ptr_array(bufs), mu, lr,
        _lib.float_array(scales), _lib.coeff_array(coeffs), n_steps, eps, compute, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(n=-1), mn.MUON_ERR_INVALID_ARG),
    (dict(n=0), mn.MUON_OK),
    (dict(rows=(8, 0)), mn.MUON_ERR_INVALID_ARG),
    (dict(params=[FAKE * 64, 0]), mn.MUON_ERR_INVALID_ARG),
    (dict(bufs=[FAKE * 64, FAKE * 128 + 8192]), mn.MUON_ERR_INVALID_ARG),
    (dict(params=[FAKE * 64, FAKE * 64]), mn.MUON_ERR_INVALID_ARG),
    (dict(param_dtype=0), mn.MUON_ERR_UNSUPPORTED),
    (dict(mu=float("nan")), mn.MUON_ERR_INVALID_ARG),
    (dict(n_steps=65, coeffs=Q * 13), mn.MUON_ERR_INVALID_ARG),
    # one 4096 x 16384 matrix needs more than the fixed scratch area: refused
    # before anything touches the GPU
    (dict(n=1, rows=(4096,), cols=(16384,), params=[1 << 40], grads=[2 << 40],
          bufs=[3 << 40]), mn.MUON_ERR_WORKSPACE),
])
def test_step_static_rejects_before_enqueue(kw, expect):
    assert static_call(**kw) == expect


def test_static_scratch_size_matches_header():
    src = open(os.path.join(ROOT, "include", "muon.h")).read()
    m = re.search(r"#define MUON_STATIC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", src)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.MUON_STATIC_SCRATCH_BYTES
    lib = mn.lib()
    # the limit applies to the largest chunk (the static entry point runs its
    # chunks one after the other): the 8-layer d768 GPT set fits, one
    # (4096, 16384) matrix does not
    largest = max(mn.orthogonalize_workspace_bytes(32, 768, 768),
                  mn.orthogonalize_workspace_bytes(16, 768, 3072))
    assert 0 < largest <= _lib.MUON_STATIC_SCRATCH_BYTES
    big = lib.muon_step_workspace_bytes(1, _lib.int_array([4096]), _lib.int_array([16384]), 0)
    assert big > _lib.MUON_STATIC_SCRATCH_BYTES


@pytest.mark.parametrize("blocks,iters,sink,expect", [
    (0, 10, FAKE, mn.MUON_ERR_INVALID_ARG),
    (4, 0, FAKE, mn.MUON_ERR_INVALID_ARG),
    (4, 10, 0, mn.MUON_ERR_INVALID_ARG),
    (4, 10, FAKE + 2, mn.MUON_ERR_INVALID_ARG),
])
def test_probe_mfma_rejects(blocks, iters, sink, expect):
    assert mn.lib().muon_probe_mfma_bf16(blocks, iters, ctypes.c_void_p(sink), None) == expect


@pytest.mark.parametrize("src,dst,nbytes,blocks", [
    (0, FAKE * 4, 1024, 8),
    (FAKE, 0, 1024, 8),
    (FAKE, FAKE * 4, 1000, 8),        # not a multiple of 16
    (FAKE + 8, FAKE * 4, 1024, 8),    # misaligned
    (FAKE, FAKE + 512, 1024, 8),      # overlapping
    (FAKE, FAKE * 4, 1024, 0),
    (FAKE, FAKE * 4, 0, 8),
])
def test_probe_copy_rejects(src, dst, nbytes, blocks):
    assert mn.lib().muon_probe_copy(ctypes.c_void_p(src), ctypes.c_void_p(dst), nbytes, blocks,
                                    None) == mn.MUON_ERR_INVALID_ARG


def test_small_steps_size_a_region_per_chunk():
    """Small steps run their chunks concurrently, each in its own workspace
    region: the size is the sum of the chunks' layouts; large steps run them
    in turn and need only the largest."""
    d768 = [(768, 768)] * 4 + [(3072, 768), (768, 3072)]
    d768 = d768 * 8
    a = mn.orthogonalize_workspace_bytes(32, 768, 768)
    b = mn.orthogonalize_workspace_bytes(16, 768, 3072)
    assert mn.step_workspace_bytes(d768) == a + b
    big = [(3072, 3072), (3072, 12288)] * 8
    assert mn.step_workspace_bytes(big) == max(
        mn.orthogonalize_workspace_bytes(8, 3072, 3072),
        mn.orthogonalize_workspace_bytes(8, 3072, 12288))
    # the 3.8B set runs its groups in turn, the d1280 set concurrently
    shapes = [(3072, 3072), (1024, 3072), (1024, 3072), (3072, 3072),
              (12288, 3072), (3072, 12288)] * 28
    assert mn.step_workspace_bytes(shapes) == mn.orthogonalize_workspace_bytes(56, 3072, 12288)
    d1280 = ([(1280, 1280)] * 4 + [(5120, 1280), (1280, 5120)]) * 20
    assert mn.step_workspace_bytes(d1280) == (
        mn.orthogonalize_workspace_bytes(64, 1280, 1280)
        + mn.orthogonalize_workspace_bytes(16, 1280, 1280)
        + mn.orthogonalize_workspace_bytes(40, 1280, 5120))
    # one chunk: nothing to run beside it
    assert mn.step_workspace_bytes([(768, 768)] * 3) == mn.orthogonalize_workspace_bytes(3, 768, 768)

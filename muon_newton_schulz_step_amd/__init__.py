"""MI355X-native Muon step: Python binding of libmuon.so.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI (``include/muon.h``).  PyTorch provides device
memory (tensors, the workspace) and the stream (the current HIP stream,
which PyTorch-ROCm exposes as ``torch.cuda.current_stream().cuda_stream``).

    orthogonalize(x, coeffs)                       -> O for one matrix or a batch
    step(params, grads, bufs, mu=, lr=, scales=, coeffs=)   in place
    step_ex(..., weight_decay=, cautious=, second_moments=, beta2=, normuon_eps=)
    step_static(params, grads, bufs, ...)          step with no workspace (fixed scratch)
"""
from __future__ import annotations

import ctypes

from . import _lib
from ._lib import (  # noqa: F401
    EXPORTS, KERNEL_KINDS, MUON_BF16, MUON_FP32, MUON_MAX_STEPS, MUON_OK, MUON_ERR_HIP,
    MUON_ERR_INVALID_ARG, MUON_ERR_UNSUPPORTED, MUON_ERR_WORKSPACE, MUON_STATIC_SCRATCH_BYTES,
)

DEFAULT_EPS = 1e-7
QUINTIC = (3.4445, -4.7750, 2.0315)


class MuonError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib.load().muon_status_string(status).decode()
        super().__init__(f"{where}: {msg}")


def lib():
    return _lib.load()


def status_string(status: int) -> str:
    return lib().muon_status_string(status).decode()


def _torch():
    import torch
    return torch


def _dtype_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.bfloat16:
        return MUON_BF16
    if dtype == torch.float32:
        return MUON_FP32
    raise TypeError(f"unsupported dtype {dtype} (bfloat16 or float32)")


def _compute_code(compute) -> int:
    if compute in ("bf16", "bfloat16", MUON_BF16):
        return MUON_BF16
    if compute in ("fp32", "float32", MUON_FP32):
        return MUON_FP32
    raise ValueError(f"compute must be 'bf16' or 'fp32', not {compute!r}")


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _coeffs(coeffs, n_steps=None):
    if isinstance(coeffs[0], (int, float)):
        if n_steps is None:
            raise ValueError("a single (a, b, c) triple needs n_steps")
        coeffs = [tuple(coeffs)] * n_steps
    coeffs = [tuple(c) for c in coeffs]
    if n_steps is not None and len(coeffs) != n_steps:
        raise ValueError("len(coeffs) != n_steps")
    return _lib.coeff_array(coeffs), len(coeffs)


class Workspace:
    """A reusable device buffer; grows to the largest request seen.

    The library's kernels read and write it as they run, so one Workspace
    must not serve two calls that can run at the same time (two streams):
    their kernels would share scratch.  Calls on one stream are ordered and
    may share it.  When it is used on a stream other than the one it was
    allocated on, the buffer is marked as in use there, so that PyTorch's
    caching allocator does not hand its memory out again (after it grows)
    before that stream's work is done."""

    def __init__(self, device=None):
        self.device = device
        self.buf = None

    def get(self, nbytes: int, device):
        torch = _torch()
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != device:
            self.buf = None
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._stream = torch.cuda.current_stream(device)
        cur = torch.cuda.current_stream(device)
        if cur != self._stream:
            self.buf.record_stream(cur)
        return self.buf


# Default workspaces, one per (device, stream): calls on different streams
# never share scratch.
_default_ws: dict = {}


def _check_device(device, **tensors):
    """Every tensor must live on `device`, a GPU: the library is handed raw
    device pointers, so host or other-device tensors are refused here."""
    if device.type != "cuda":
        raise ValueError("tensors must be GPU tensors")
    for name, ts in tensors.items():
        for t in ts:
            if t is not None and t.device != device:
                raise ValueError(f"{name}: every tensor must be on {device}, found {t.device}")


def _workspace(nbytes: int, device, workspace):
    if workspace is None:
        key = (str(device), _torch().cuda.current_stream(device).cuda_stream)
        workspace = _default_ws.setdefault(key, Workspace())
    if isinstance(workspace, Workspace):
        buf = workspace.get(nbytes, device)
        return buf.data_ptr(), buf.numel()
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def orthogonalize_workspace_bytes(batch: int, rows: int, cols: int, compute="bf16") -> int:
    return int(lib().muon_orthogonalize_workspace_bytes(batch, rows, cols, _compute_code(compute)))


def step_workspace_bytes(shapes, compute="bf16") -> int:
    rows = _lib.int_array(r for r, _ in shapes)
    cols = _lib.int_array(c for _, c in shapes)
    return int(lib().muon_step_workspace_bytes(len(shapes), rows, cols, _compute_code(compute)))


def plan_groups(shapes):
    """Oriented-shape grouping muon_step uses: (group_of, [(m, n, count), ...])."""
    n = len(shapes)
    rows = _lib.int_array(r for r, _ in shapes)
    cols = _lib.int_array(c for _, c in shapes)
    gof, gm, gn, gc = (_lib.int_array([0] * n) for _ in range(4))
    ng = ctypes.c_int(0)
    st = lib().muon_plan_groups(n, rows, cols, gof, gm, gn, gc, ctypes.byref(ng))
    if st != MUON_OK:
        raise MuonError(st, "muon_plan_groups")
    return [gof[i] for i in range(n)], [(gm[g], gn[g], gc[g]) for g in range(ng.value)]


def orthogonalize(x, coeffs=QUINTIC, n_steps=None, *, eps=DEFAULT_EPS, compute="bf16",
                  out=None, out_dtype=None, workspace=None):
    """Newton-Schulz orthogonalisation of a matrix (rows, cols) or a batch
    (batch, rows, cols) on the GPU.  ``coeffs`` is a table of (a, b, c) rows or
    one triple with ``n_steps``.  Returns ``out`` (a new tensor by default,
    dtype ``out_dtype`` or x.dtype)."""
    torch = _torch()
    if n_steps is None and isinstance(coeffs[0], (int, float)):
        n_steps = 5
    table, n_steps = _coeffs(coeffs, n_steps)
    _check_device(x.device, out=[out], workspace=[
        workspace if workspace is not None and not isinstance(workspace, Workspace) else None])
    squeeze = x.dim() == 2
    xb = x.unsqueeze(0) if squeeze else x
    if xb.dim() != 3:
        raise ValueError("x must be (rows, cols) or (batch, rows, cols)")
    xb = xb.contiguous()
    batch, rows, cols = xb.shape
    if out is None:
        out = torch.empty_like(xb, dtype=out_dtype or x.dtype)
    else:
        out = out.view(batch, rows, cols)
        if not out.is_contiguous():
            raise ValueError("out must be contiguous")
    c = _compute_code(compute)
    need = orthogonalize_workspace_bytes(max(batch, 1), rows, cols, compute)
    with torch.cuda.device(x.device):
        wptr, wbytes = _workspace(need, x.device, workspace)
        st = lib().muon_orthogonalize(
            ctypes.c_void_p(xb.data_ptr()), _dtype_code(xb.dtype),
            ctypes.c_void_p(out.data_ptr()), _dtype_code(out.dtype),
            batch, rows, cols, rows * cols, table, n_steps, float(eps), c,
            ctypes.c_void_p(wptr), wbytes, _stream(x.device))
    if st != MUON_OK:
        raise MuonError(st, "muon_orthogonalize")
    return out[0] if squeeze else out


def step(params, grads, bufs, *, mu, lr, scales=None, coeffs=QUINTIC, n_steps=None,
         eps=DEFAULT_EPS, compute="bf16", workspace=None):
    """One Muon step, in place on ``params`` (fp32) and ``bufs`` (fp32
    momentum), for lists of 2-D GPU tensors of any mix of shapes."""
    _step(params, grads, bufs, None, None, mu=mu, lr=lr, scales=scales, coeffs=coeffs,
          n_steps=n_steps, eps=eps, compute=compute, workspace=workspace)


def step_ex(params, grads, bufs, *, mu, lr, scales=None, coeffs=QUINTIC, n_steps=None,
            eps=DEFAULT_EPS, compute="bf16", workspace=None, weight_decay=0.0,
            cautious=True, second_moments=None, beta2=None, normuon_eps=None):
    """``step`` with the additions of the web3.cnoyu.systems review of
    karpathy/autoresearch's train.py, paragraph after the Muon one
    (muon_step_ex): decoupled weight decay
    (cautious: only where update * param >= 0) and, when ``second_moments``
    (fp32 vectors of min(rows, cols) elements, in place) are given, NorMuon
    scaling with ``beta2`` and ``normuon_eps`` (no defaults: the page gives
    none)."""
    normuon = second_moments is not None
    if normuon and (beta2 is None or normuon_eps is None):
        raise ValueError("NorMuon needs beta2 and normuon_eps")
    opt = _lib.MuonOptions(float(weight_decay), 1 if cautious else 0, 1 if normuon else 0,
                           float(beta2) if normuon else 0.0,
                           float(normuon_eps) if normuon else 0.0)
    if normuon:
        if len(second_moments) != len(params):
            raise ValueError("one second-moment vector per matrix")
        for p, v in zip(params, second_moments):
            if (v.dtype != _torch().float32 or not v.is_contiguous()
                    or v.numel() != min(p.shape)):
                raise ValueError("second moments: contiguous fp32, min(rows, cols) elements")
    _step(params, grads, bufs, second_moments, opt, mu=mu, lr=lr, scales=scales,
          coeffs=coeffs, n_steps=n_steps, eps=eps, compute=compute, workspace=workspace)


def _step(params, grads, bufs, second_moments, opt, *, mu, lr, scales, coeffs, n_steps, eps,
          compute, workspace):
    n = len(params)
    if not (len(grads) == len(bufs) == n):
        raise ValueError("params, grads and bufs must have the same length")
    if n == 0:
        return
    if n_steps is None and isinstance(coeffs[0], (int, float)):
        n_steps = 5
    table, n_steps = _coeffs(coeffs, n_steps)
    if scales is None:
        scales = [1.0] * n
    grad_dtype = _dtype_code(grads[0].dtype)
    for p, g, b in zip(params, grads, bufs):
        if p.dim() != 2 or g.shape != p.shape or b.shape != p.shape:
            raise ValueError("params, grads and bufs must be matching 2-D tensors")
        if not (p.is_contiguous() and g.is_contiguous() and b.is_contiguous()):
            raise ValueError("tensors must be contiguous")
        if _dtype_code(g.dtype) != grad_dtype:
            raise ValueError("all grads must share one dtype")
    device = params[0].device
    _check_device(device, params=params, grads=grads, bufs=bufs,
                  second_moments=second_moments or [],
                  workspace=[workspace if workspace is not None
                             and not isinstance(workspace, Workspace) else None])
    shapes = [tuple(p.shape) for p in params]
    rows = _lib.int_array(r for r, _ in shapes)
    cols = _lib.int_array(c for _, c in shapes)
    c = _compute_code(compute)
    common = (_lib.ptr_array(p.data_ptr() for p in params), _dtype_code(params[0].dtype),
              _lib.ptr_array(g.data_ptr() for g in grads), grad_dtype,
              _lib.ptr_array(b.data_ptr() for b in bufs))
    with _torch().cuda.device(device):
        if opt is None:
            need = int(lib().muon_step_workspace_bytes(n, rows, cols, c))
            wptr, wbytes = _workspace(need, device, workspace)
            st = lib().muon_step(
                n, rows, cols, *common,
                float(mu), float(lr), _lib.float_array(scales), table, n_steps, float(eps), c,
                ctypes.c_void_p(wptr), wbytes, _stream(device))
            where = "muon_step"
        else:
            need = int(lib().muon_step_ex_workspace_bytes(n, rows, cols, c, ctypes.byref(opt)))
            wptr, wbytes = _workspace(need, device, workspace)
            vptrs = (_lib.ptr_array(v.data_ptr() for v in second_moments)
                     if second_moments is not None else None)
            st = lib().muon_step_ex(
                n, rows, cols, *common, vptrs,
                float(mu), float(lr), _lib.float_array(scales), table, n_steps, float(eps), c,
                ctypes.byref(opt), ctypes.c_void_p(wptr), wbytes, _stream(device))
            where = "muon_step_ex"
    if st != MUON_OK:
        raise MuonError(st, where)


def step_static(params, grads, bufs, *, mu, lr, scales=None, coeffs=QUINTIC, n_steps=None,
                eps=DEFAULT_EPS, compute="bf16"):
    """``step`` through muon_step_static: no workspace, nothing allocated; the
    scratch is the library's fixed area on the current GPU
    (MUON_STATIC_SCRATCH_BYTES), so calls that overlap in time on one GPU
    race."""
    n = len(params)
    if not (len(grads) == len(bufs) == n):
        raise ValueError("params, grads and bufs must have the same length")
    if n == 0:
        return
    if n_steps is None and isinstance(coeffs[0], (int, float)):
        n_steps = 5
    table, n_steps = _coeffs(coeffs, n_steps)
    if scales is None:
        scales = [1.0] * n
    grad_dtype = _dtype_code(grads[0].dtype)
    for p, g, b in zip(params, grads, bufs):
        if p.dim() != 2 or g.shape != p.shape or b.shape != p.shape:
            raise ValueError("params, grads and bufs must be matching 2-D tensors")
        if not (p.is_contiguous() and g.is_contiguous() and b.is_contiguous()):
            raise ValueError("tensors must be contiguous")
        if _dtype_code(g.dtype) != grad_dtype:
            raise ValueError("all grads must share one dtype")
    device = params[0].device
    _check_device(device, params=params, grads=grads, bufs=bufs)
    rows = _lib.int_array(p.shape[0] for p in params)
    cols = _lib.int_array(p.shape[1] for p in params)
    with _torch().cuda.device(device):
        st = lib().muon_step_static(
            n, rows, cols, _lib.ptr_array(p.data_ptr() for p in params),
            _dtype_code(params[0].dtype), _lib.ptr_array(g.data_ptr() for g in grads), grad_dtype,
            _lib.ptr_array(b.data_ptr() for b in bufs), float(mu), float(lr),
            _lib.float_array(scales), table, n_steps, float(eps), _compute_code(compute),
            _stream(device))
    if st != MUON_OK:
        raise MuonError(st, "muon_step_static")


def probe_mfma_bf16(sink, blocks: int, iters: int) -> float:
    """Enqueue the MFMA rate probe on the current stream; returns the flops the
    launch performs (time it with events on the same stream)."""
    st = lib().muon_probe_mfma_bf16(blocks, iters, ctypes.c_void_p(sink.data_ptr()),
                                    _stream(sink.device))
    if st != MUON_OK:
        raise MuonError(st, "muon_probe_mfma_bf16")
    return float(blocks) * 8 * iters * 4 * 32768


def probe_copy(src, dst, blocks: int) -> float:
    """Enqueue the plain copy probe src -> dst (same size, bytes a multiple of
    16) on the current stream; returns the HBM bytes it moves (read + write)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size")
    st = lib().muon_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()),
                               nbytes, blocks, _stream(src.device))
    if st != MUON_OK:
        raise MuonError(st, "muon_probe_copy")
    return 2.0 * nbytes


def timing_enable(on: bool = True) -> bool:
    return bool(lib().muon_timing_enable(1 if on else 0))


def timing_read(cap: int = 1 << 16):
    """Per-launch timing records since the last read (dicts)."""
    arr = (_lib.MuonTimingRecord * cap)()
    n = ctypes.c_int(0)
    st = lib().muon_timing_read(arr, cap, ctypes.byref(n))
    if st != MUON_OK:
        raise MuonError(st, "muon_timing_read")
    return [dict(kind=KERNEL_KINDS[r.kind], m=r.m, n=r.n, batch=r.batch, step=r.step,
                 ms=r.ms, flops=r.flops, bytes=r.bytes, exec_flops=r.exec_flops)
            for r in arr[:n.value]]

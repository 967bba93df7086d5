"""Build libmuon.so in-tree with hipcc for gfx950.

``python -m muon_newton_schulz_step_amd.build`` or ``build()`` compiles the HIP
kernels and the host runtime into ``muon_newton_schulz_step_amd/libmuon.so``.
Every translation unit is compiled to an object in parallel (the GEMM
epilogue families are separate units), then linked; the library is replaced
atomically.  It always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmuon.so")
SOURCES = ["gemm_update.hip", "gemm_final_w.hip", "gemm_final_out.hip", "gemm_gram.hip",
           "gemm_poly.hip", "gemm_fp32.hip", "muon_kernels.hip", "muon_peaks.hip",
           "muon_static.hip",
           "muon_api.cpp"]
ARCH = os.environ.get("MUON_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmuon.so)")


def compile_command(src: str, obj: str):
    return [
        hipcc(), "-O3", "-std=c++17", "-fPIC", "-c",
        f"--offload-arch={ARCH}",
        # no packed-fp32 instructions anywhere in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC,
        os.path.join(CSRC, src), "-o", obj,
    ]


def link_command(objs, out: str):
    return [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,--no-undefined",
            *objs, "-o", out]


# hipcc's host pass does not know the device-only feature; drop that noise
_NOISE = "is not a recognized feature for this target"


def _run(cmd):
    proc = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in proc.stderr.splitlines() if _NOISE not in l)
    return proc.returncode, err


def build(verbose: bool = False, jobs: int | None = None) -> str:
    jobs = jobs or min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
    with tempfile.TemporaryDirectory(prefix="muon_build_") as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [compile_command(s, o) for s, o in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for src, (rc, err) in zip(SOURCES, results):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src} ({rc}):\n{err}")
            if verbose and err.strip():
                print(err, file=sys.stderr)
        tmp = LIB + f".tmp{os.getpid()}"
        cmd = link_command(objs, tmp)
        if verbose:
            print(" ".join(cmd), flush=True)
        rc, err = _run(cmd)
        if rc != 0:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise RuntimeError(f"link failed ({rc}):\n{err}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

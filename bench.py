"""Benchmark of the Muon step on the 3.8B GPT matrix set (one MI355X).

A step is one muon_step call over all 168 matrices (momentum, Frobenius
normalisation, 5 Newton-Schulz steps, weight update), inputs resident in HBM.
Prints one JSON line:  metric / value (ms per step) / NS TFLOP/s and its
fraction of the dense bf16 MFMA peak / roofline of the dominant kernel /
the fp64 oracle timed on the host cores as a CPU baseline.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--compute bf16|fp32]
                    [--variant plain|cwd|normuon_cwd] [--graph] [--no-peaks]

--variant times muon_step_ex instead: the cautious weight decay (cwd, decay
0.1) of the web3.cnoyu.systems review of karpathy/autoresearch's train.py,
or NorMuon (beta2 0.95, eps 1e-8) with it (normuon_cwd).  The
default, plain, is the benchmark's Muon step.  --graph times replays of one
captured step instead of eager calls (the small workloads are bound by the
host cost of their launches).

The headline time is taken with the library's per-launch timing off; the
per-kernel table (and the roofline of the dominant kernel) comes from a second
pass of the same number of steps right after it, with HIP events recorded by
the library around every launch on the launch stream.  The measured-peaks leg
then times two probe kernels of the library on the same GPU: back-to-back bf16
MFMAs (the sustained matrix rate) and a plain 16-byte copy (the sustained HBM
bandwidth), so every fraction is reported against the datasheet peak and
against what the chip sustained in the same run.
"""
import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK = {"bf16": 2500.0, "fp32": 157.3}   # dense MFMA TFLOP/s, MI355X datasheet
HBM_PEAK_GBS = 8000.0
METRIC = "Muon step ms, 3.8B matrix set; NS TFLOP/s and % of bf16 MFMA peak"
# muon_step_ex options of the non-default variants (the page gives no values)
VARIANTS = {
    "plain": None,
    "cwd": dict(weight_decay=0.1, cautious=True),
    "normuon_cwd": dict(weight_decay=0.1, cautious=True, beta2=0.95, normuon_eps=1e-8),
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="gpt_3.8b_28layers")
    p.add_argument("--compute", default="bf16", choices=["bf16", "fp32"])
    p.add_argument("--variant", default="plain", choices=list(VARIANTS))
    p.add_argument("--coeffs", choices=["quintic", "cubic"], default=None,
                   help="coefficient triple at every step (default: the workload's quintic)")
    p.add_argument("--ns-steps", type=int, default=None,
                   help="Newton-Schulz steps (default: the workload's 5)")
    p.add_argument("--matrices", type=int, default=None,
                   help="time a bounded sample: the first N matrices of each raw shape of "
                        "the workload")
    p.add_argument("--owner-share", type=int, default=None, metavar="N",
                   help="time the matrices one rank owns in an N-way step sharded by whole "
                        "matrix (every N-th matrix of each oriented shape)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="time replays of one captured step (a HIP graph: no per-launch host "
                        "cost); the per-kernel times then come from an eager pass after it")
    p.add_argument("--cpu-sample-seconds", type=float, default=12.0,
                   help="seconds of oracle work for the CPU baseline sample")
    p.add_argument("--calibrate", "--calibrate-copy", dest="calibrate", action="store_true",
                   help="before the step, run the library's MFMA probe and one plain 1 GiB "
                        "copy (the known work that counter passes are scaled by)")
    p.add_argument("--no-peaks", action="store_true",
                   help="skip the measured-peaks leg (MFMA and copy probes)")
    p.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of a "
                        "'--steps 1 --warmup 0 --calibrate' run into profiles/traffic.json")
    p.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                   help="print a markdown table of a rocprofv3 --kernel-trace CSV: the "
                        "library's kernels by instantiation and grid, calls, average and "
                        "total time")
    p.add_argument("--tile-sweep", action="store_true",
                   help="time one step over each of a list of same-shape sets (one chunk "
                        "each, alone) and print per-kernel launch times, one JSON line per "
                        "set; run with MUON_GEMM_TILE=128, =256 and unset to compare the "
                        "tiles with the library's choice")
    p.add_argument("--tile-table", nargs=3, metavar=("AT128", "AT256", "CHOSEN"),
                   help="markdown table of three --tile-sweep outputs")
    p.add_argument("--overlap-probe", action="store_true",
                   help="run the library's MFMA probe and copy probe alone and side by side "
                        "on two streams (one long launch each) and print what each sustains")
    p.add_argument("--batch-sweep", action="store_true",
                   help="time each GEMM kind of one orthogonalisation against the batch size "
                        "(launch time against tile count: rounds of the CUs or a straight line)")
    p.add_argument("--write-mfma", metavar="MFMA_CSV",
                   help="turn a rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 "
                        "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE counter CSV of a "
                        "'--steps 1 --warmup 0 --calibrate' run into profiles/mfma.json")
    return p.parse_args()


def kernel_summary(records, steps):
    """Aggregate the per-launch HIP-event log by (kind, m, n)."""
    agg = {}
    for r in records:
        key = (r["kind"], r["m"], r["n"])
        a = agg.setdefault(key, {"kind": r["kind"], "m": r["m"], "n": r["n"], "launches": 0,
                                 "ms": 0.0, "flops": 0.0, "exec_flops": 0.0, "bytes": 0.0,
                                 "batch": r["batch"]})
        a["launches"] += 1
        a["ms"] += r["ms"]
        a["flops"] += r["flops"]
        a["exec_flops"] += r["exec_flops"]
        a["bytes"] += r["bytes"]
    out = sorted(agg.values(), key=lambda a: -a["ms"])
    for a in out:
        a["ms_per_step"] = a["ms"] / steps
        a["avg_launch_ms"] = a["ms"] / a["launches"]
        sec = a["ms"] * 1e-3
        # tflops: the flops the launches execute; tflops_counted: the method's
        # 4m^2n + 2m^3 count, which the triangle and Q A Q launches undercut
        a["tflops"] = a["exec_flops"] / sec / 1e12 if sec > 0 else 0.0
        a["tflops_counted"] = a["flops"] / sec / 1e12 if sec > 0 else 0.0
        a["gbs"] = a["bytes"] / sec / 1e9 if sec > 0 else 0.0
    return out


CSRC = os.path.join(ROOT, "muon_newton_schulz_step_amd", "csrc")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
MFMA_JSON = os.path.join(ROOT, "profiles", "mfma.json")
COPY_BYTES = 1 << 30
# the calibration MFMA probe of --calibrate: 256 workgroups x 2000 rounds
CAL_MFMA = (256, 2000)


def kernel_source_digest():
    """SHA-256 over the device sources (kernels and the headers they include),
    in name order: counter summaries are valid for exactly this code."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def profile_entry(path, kernel_key):
    """A kernel's entry of a committed counter summary (profiles/*.json), or
    None if there is none for the current kernel source."""
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)
        if data.get("kernel_source_sha256") != kernel_source_digest():
            return None
        return data["kernels"].get(kernel_key)
    except Exception:
        return None


def traffic_from_profiles(kernel_key):
    """HBM bytes per launch of a kernel from the committed counter summary."""
    k = profile_entry(TRAFFIC_JSON, kernel_key)
    return None if k is None else k["traffic_bytes"]


def pick_tile(t256, batch, use, compute="bf16"):
    """The GEMM tile the library takes for a launch of `batch` matrices with
    t256 tiles each at 256 x 256, as its host runtime decides it.  use:
    "full" (update, final), "tri" (polynomial, Q A Q products: the lower
    triangle of t256 x t256 tiles) or "gram" (the Gram's lower triangle).
    Rounds of the 256 CUs, one 256-tile workgroup or two 128-tile ones per
    CU; 256 when 1.6 (the Gram: 1.4) x rounds(256) <= rounds(128).
    MUON_GEMM_TILE=128|256 forces the tile, as in the library."""
    if compute != "bf16":
        return 128
    pref = os.environ.get("MUON_GEMM_TILE", "")
    if pref in ("128", "256"):
        return int(pref)
    tri = use != "full"
    t = t256 * (t256 + 1) // 2 if tri else t256
    t128 = (2 * t256) * (2 * t256 + 1) // 2 if tri else 4 * t256
    w256, w128 = t * batch, t128 * batch
    ratio5 = 7 if use == "gram" else 8
    return 256 if ratio5 * -(-w256 // 256) <= 5 * -(-w128 // 512) else 128


def launch_sequence(w):
    """(kind, m, n) of every library launch of one bf16 step, in launch order:
    per oriented group (first appearance) and chunk of at most 64 matrices,
    prep, norm, then gram, poly, update per Newton-Schulz step, the last
    update being one final launch for the chunk's wide matrices and one for
    its tall ones (a single one for both when the larger part alone would take
    128 x 128 tiles).  Groups with padded N >= 4M and M >= 2048 form the Gram
    matrix of steps 1 and 3 (not the last) in two gramq launches instead."""
    def pad(d):
        return (d + 255) // 256 * 256
    groups = {}
    for r, c in w.shapes:
        groups.setdefault((min(r, c), max(r, c)), []).append(r > c)
    seq = []
    for (m, n), talls in groups.items():
        qaq = pad(n) >= 4 * pad(m) and pad(m) >= 2048
        for b0 in range(0, len(talls), 64):
            chunk = talls[b0:b0 + 64]
            nt = sum(chunk)
            nw = len(chunk) - nt
            # one launch for both parts when the larger would take 128-tiles
            t256 = (pad(m) // 256) * (pad(n) // 256)
            mixed = nw > 0 and nt > 0 and pick_tile(t256, max(nw, nt), "full") == 128
            finals = [("final", m, n)] * (1 if mixed else (nw > 0) + (nt > 0))
            seq += [("prep", m, n), ("norm", m, n)]
            for k in range(w.n_steps):
                if qaq and k in (1, 3) and k <= w.n_steps - 2:
                    seq += [("gramq", m, n), ("gramq", m, n), ("poly", m, n)]
                else:
                    seq += [("gram", m, n), ("poly", m, n)]
                seq += [("update", m, n)] if k < w.n_steps - 1 else finals
    return seq


def ns_flops_executed(w, compute="bf16"):
    """Flops the GEMM launches of one step execute (MFMA work over the padded
    tiles they run), against the method's counted 4m^2n + 2m^3 per matrix
    and step: GRAM and POLY run lower-triangle tiles only, and on the bf16
    path the Gram matrix of steps 1 and 3 of groups with padded N >= 4M and
    M >= 2048 is formed as Q A Q (two M x M x M triangle launches)."""
    def pad(d):
        return (d + 255) // 256 * 256
    groups = {}
    for r, c in w.shapes:
        key = (min(r, c), max(r, c))
        groups[key] = groups.get(key, 0) + 1
    tot = 0.0
    for (m, n), count in groups.items():
        M, N = pad(m), pad(n)
        for b0 in range(0, count, 64):
            cnt = min(64, count - b0)
            t256 = M // 256
            def tri(tile):  # C elements the triangle launches compute
                return (M // tile) * (M // tile + 1) // 2 * tile * tile * cnt
            tri_g = tri(pick_tile(t256, cnt, "gram", compute))
            tri_p = tri(pick_tile(t256, cnt, "tri", compute))
            qaq = compute == "bf16" and N >= 4 * M and M >= 2048
            for k in range(w.n_steps):
                if qaq and k in (1, 3) and k <= w.n_steps - 2:
                    tot += 2 * (2.0 * tri_p * M)       # two Q A Q products
                else:
                    tot += 2.0 * tri_g * N             # GRAM
                tot += 2.0 * tri_p * M                 # POLY
                tot += 2.0 * M * N * M * cnt           # UPDATE / FINAL (full tiles)
    return tot


_EPI_NAMES = {0: "GRAM", 1: "POLY", 2: "UPDATE", 3: "FINAL_W", 4: "FINAL_OUT", 5: "FINAL_W_T",
              6: "FINAL_OUT_T", 7: "GRAM_LO", 8: "POLY_LO", 9: "UPDATE_ROWS", 10: "FINAL_W_MIX"}


def kernel_label(name):
    """A readable label for a library kernel name as rocprofv3 prints it
    (mangled, or demangled; its demangler renders the bf16 POLY instance as
    '<bool _Accum, int, E, ...>')."""
    import re
    m = re.search(r"gemm_kernelI(DF16b|f)Li(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)ELi(\d+)"
                  r"ELb(\d)ELb(\d)ELb(\d)E", name)
    if m:
        t, epi, bm, bn, wgm, wgn, st, qrow, buf, strm = m.groups()
        flags = [x for x, on in (("rowQ", qrow), ("buf" if st == "2" else "regs", "1"),
                                 ("stream", strm)) if on == "1"]
        if st == "2" and buf == "0":
            flags[flags.index("buf")] = "dma"
        return (f"gemm<{'bf16' if t == 'DF16b' else 'fp32'},{_EPI_NAMES[int(epi)]},{bm}x{bn},"
                f"{int(wgm) * int(wgn)}w,{','.join(flags)}>")
    # rocprofv3's demangler garbles some bf16 instances: POLY (epilogue 1)
    # comes out as '<bool _Accum, int, E, BM, BN, ...>', GRAM_LO (7) as
    # '<bool _Accum, int, ELiBME, BN, ...>'
    m = re.search(r"gemm_kernel<bool _Accum, int, E(?:Li(\d+)E)?, (\d+), (\d+), (\d+), (\d+),"
                  r"(?: (\d+),)? (true|false), (true|false), (true|false)>", name)
    if m:
        lo_bm, a, b, c, d, e, qrow, buf, strm = m.groups()
        if lo_bm:   # GRAM_LO: BM, then BN WGM WGN S
            epi, bm, bn, wgm, wgn = "GRAM_LO", lo_bm, a, b, c
        else:       # POLY: BM BN WGM WGN S
            epi, bm, bn, wgm, wgn = "POLY", a, b, c, d
        return (f"gemm<bf16,{epi},{bm}x{bn},{int(wgm) * int(wgn)}w,"
                f"{'buf' if buf == 'true' else 'dma'}>")
    m = re.search(r"gemm_kernel<float, (\d+), (\d+), (\d+), (\d+), (\d+), (\d+)", name)
    if m:
        epi, bm, bn, wgm, wgn, st = m.groups()
        return f"gemm<fp32,{_EPI_NAMES[int(epi)]},{bm}x{bn},{int(wgm) * int(wgn)}w,regs>"
    m = re.search(r"prep_kernelI(DF16b|f)(DF16b|f)Lb(\d)ELb(\d)E", name)
    if m:
        g, x, mom, strm = m.groups()
        return (f"prep<grad {'bf16' if g == 'DF16b' else 'fp32'},X {'bf16' if x == 'DF16b' else 'fp32'}"
                f"{',momentum' if mom == '1' else ''}{',stream' if strm == '1' else ''}>")
    m = re.search(r"prep_kernel<float, bool _Accum, bool, E, (true|false)>", name)
    if m:   # the demangler's rendering of prep<fp32 grad, bf16 X, momentum>
        return f"prep<grad fp32,X bf16,momentum{',stream' if m.group(1) == 'true' else ''}>"
    for k in ("normuon_rowparts_kernel", "normuon_rows_kernel", "norm_kernel", "apply_kernel",
              "prep_kernel", "gemm_kernel"):
        if k in name:
            garbled = "_Accum" in name or "gemm_kernel" in k or "prep_kernel" in k
            return k.replace("_kernel", "") + (" (name garbled by the profiler's demangler)"
                                               if garbled else "")
    return name[:60]


def summarize_trace(path):
    """Markdown table of the library's kernels in a rocprofv3 kernel trace."""
    import csv
    agg = {}
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"]
        if not is_step_kernel(name):
            continue
        wg = (int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))) * int(r["Grid_Size_Y"])
        key = (kernel_label(name), wg)
        a = agg.setdefault(key, [0, 0])
        a[0] += 1
        a[1] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    total = sum(v[1] for v in agg.values())
    print("| kernel | workgroups | calls | avg us | total ms | % of library time |")
    print("|---|---|---|---|---|---|")
    for (label, wg), (n, ns) in sorted(agg.items(), key=lambda kv: -kv[1][1]):
        print(f"| `{label}` | {wg} | {n} | {ns / n / 1e3:.1f} | {ns / 1e6:.2f} | "
              f"{100.0 * ns / total:.1f} |")


def is_step_kernel(name):
    """A dispatch of the Muon step (the library's kernels minus its probes);
    rocprofv3 leaves some of the bf16 kernels' names mangled (_ZN4muon...)."""
    return "muon" in name and "probe" not in name


def per_dispatch_counters(path, counters):
    """{dispatch id: [kernel name, {counter: summed value}]} of a rocprofv3
    counter-collection CSV, in dispatch order."""
    import csv
    rows = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] not in counters:
            continue
        did = int(r["Dispatch_Id"])
        ent = rows.setdefault(did, [r["Kernel_Name"], {c: 0.0 for c in counters}])
        ent[1][r["Counter_Name"]] += float(r["Counter_Value"])
    return [rows[k] for k in sorted(rows)]


def write_mfma(csv_path, w):
    """MFMA counters of one profiled bf16 step, per launch kind: executed
    flops from SQ_INSTS_VALU_MFMA_MOPS_BF16 and the MFMA-busy fraction
    SQ_VALU_MFMA_BUSY_CYCLES / GRBM_GUI_ACTIVE, both scaled by what the same
    counters read for the library's MFMA probe (--calibrate), whose flop count
    is exact and whose MFMA pipes are busy all the time."""
    ctr = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
    rows = per_dispatch_counters(csv_path, ctr)
    probe = next(v for name, v in rows if "mfma_probe" in name)
    probe_flops = float(CAL_MFMA[0]) * 8 * CAL_MFMA[1] * 4 * 32768
    flops_per_mop = probe_flops / probe[ctr[0]]
    probe_busy = probe[ctr[1]] / probe[ctr[2]]
    steps = [v for name, v in rows if is_step_kernel(name)]
    seq = launch_sequence(w)
    if len(steps) == 0 or len(steps) % len(seq) != 0:
        raise SystemExit(f"{len(steps)} library dispatches in {csv_path}, "
                         f"not a multiple of the {len(seq)} of one step")
    steps = steps[:len(seq)]  # the timed step (the instrumented pass repeats it)
    acc = {}
    for (kind, m, n), v in zip(seq, steps):
        a = acc.setdefault(f"{kind}_{m}x{n}", {"launches": 0, "flops": 0.0, "busy": 0.0,
                                               "active": 0.0})
        a["launches"] += 1
        a["flops"] += v[ctr[0]] * flops_per_mop
        a["busy"] += v[ctr[1]]
        a["active"] += v[ctr[2]]
    out = {"kernel_source_sha256": kernel_source_digest(), "workload": w.name,
           "calibration": {"probe_flops": probe_flops, "flops_per_mop": flops_per_mop,
                           "probe_busy_per_active_cycle": probe_busy},
           "step_flops_from_counters": sum(a["flops"] for a in acc.values()),
           "step_flops_executed_by_tiles": ns_flops_executed(w), "kernels": {}}
    for key, a in acc.items():
        out["kernels"][key] = {"launches": a["launches"],
                               "exec_flops_per_launch": a["flops"] / a["launches"],
                               "mfma_busy_frac": (a["busy"] / a["active"]) / probe_busy
                               if a["active"] > 0 else 0.0}
    with open(MFMA_JSON, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(f"wrote {MFMA_JSON}")


def write_traffic(fetch_csv, write_csv, w):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of one profiled step,
    scaled by what the same counters read for a plain copy kernel of
    COPY_BYTES read + COPY_BYTES written (an elementwise multiply by 1)."""
    import csv

    def per_dispatch(path, counter):
        rows = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            did = int(r["Dispatch_Id"])
            rows.setdefault(did, [r["Kernel_Name"], 0.0])
            rows[did][1] += float(r["Counter_Value"])
        return [rows[k] for k in sorted(rows)]

    out = {"kernel_source_sha256": kernel_source_digest(), "copy_bytes": COPY_BYTES,
           "workload": w.name, "kernels": {}}
    seq = launch_sequence(w)
    for path, counter, field in ((fetch_csv, "FETCH_SIZE", "fetch"),
                                 (write_csv, "WRITE_SIZE", "write")):
        rows = per_dispatch(path, counter)
        copy_kib = next(v for name, v in rows if "copy_probe" in name)
        scale = COPY_BYTES / (copy_kib * 1024.0)
        out[field + "_scale"] = scale
        muon = [v for name, v in rows if is_step_kernel(name)]
        if len(muon) == 0 or len(muon) % len(seq) != 0:
            raise SystemExit(f"{len(muon)} library dispatches in {path}, "
                             f"not a multiple of the {len(seq)} of one step")
        muon = muon[:len(seq)]  # the timed step (the instrumented pass repeats it)
        acc = {}
        for (kind, m, n), v in zip(seq, muon):
            a = acc.setdefault(f"{kind}_{m}x{n}", [0, 0.0])
            a[0] += 1
            a[1] += v * 1024.0 * scale
        for key, (cnt, tot) in acc.items():
            out["kernels"].setdefault(key, {})[field + "_bytes"] = tot / cnt
    for k in out["kernels"].values():
        k["traffic_bytes"] = k["fetch_bytes"] + k["write_bytes"]
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)
    print(f"wrote {TRAFFIC_JSON}")


def host_info():
    """(BLAS library and version, BLAS threads, CPU model) of this host."""
    blas, threads = "unknown", os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = f"{i.get('internal_api')} {i.get('version')} ({i.get('filepath', '')})"
                threads = i.get("num_threads", threads)
                break
    except Exception:
        pass
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return blas, threads, model


def cpu_baseline(w, seconds, variant="plain", dev="cpu", keep=None):
    """The fp64 oracle on a bounded sample of the workload: matrices taken
    round-robin over the oriented groups until about `seconds` of CPU work,
    per-group mean times extrapolated by the group counts.  The inputs are
    made on `dev` and copied to the host; with `keep` (a list), each sampled
    matrix's (index, inputs on dev, second moment or None, oracle weights)
    is appended to it."""
    import oracle
    import workloads as wl
    blas, threads, model = host_info()
    groups = w.oriented_groups()
    members = {}
    for i, (r, c) in enumerate(w.shapes):
        members.setdefault((min(r, c), max(r, c)), []).append(i)
    times = {k: [] for k in groups}
    spent, rnd = 0.0, 0
    while True:
        for key in groups:
            if rnd >= len(members[key]):
                continue
            idx = members[key][rnd]
            x = wl.make_inputs(w, device=dev, indices=[idx])
            g = x["grads"][0].double().cpu().numpy()
            b = x["bufs"][0].double().cpu().numpy()
            p = x["params"][0].double().cpu().numpy()
            opt = VARIANTS[variant]
            vt = (wl.make_second_moment(w, idx, device=dev)
                  if opt is not None and "beta2" in opt else None)
            t0 = time.perf_counter()
            if opt is None:
                new_w = oracle.muon_step(p, g, b, w.mu, w.lr, x["scales"][0], w.coeff_table)[0]
            else:
                v = vt.double().cpu().numpy() if vt is not None else None
                new_w = oracle.muon_step_ex(p, g, b, w.mu, w.lr, x["scales"][0], w.coeff_table,
                                            weight_decay=opt["weight_decay"],
                                            cautious=opt["cautious"], second_moment=v,
                                            beta2=opt.get("beta2", 0.0),
                                            normuon_eps=opt.get("normuon_eps", 0.0))["w"]
            dt = time.perf_counter() - t0
            if keep is not None:
                keep.append((idx, x, vt, p, new_w))
            times[key].append(dt)
            spent += dt
        rnd += 1
        if spent >= seconds or rnd >= max(len(v) for v in members.values()):
            break
    total_ms = sum(1e3 * sum(t) / len(t) * groups[k] for k, t in times.items())
    sample = ", ".join(f"{len(times[k])} x {k[0]}x{k[1]}" for k in groups)
    return {
        "value": round(total_ms, 1),
        "unit": "ms per step (extrapolated from the sample)",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"fp64 numpy Muon step{'' if variant == 'plain' else ' (' + variant + ')'} "
                   f"on {sample} matrices (of {len(w.shapes)}), "
                   f"{spent:.1f} s of CPU work; per-group mean x group count"),
        "blas": blas,
        "cpu_model": model,
    }


def sample_parity(torch, mn, w, kept, variant, compute):
    """The library's step on the CPU baseline's sampled matrices (their own
    step, from the seeded state, the same tensors the oracle was given)
    against the oracle's weights: relative Frobenius error of dW = W' - W per
    matrix."""
    import oracle
    if not kept:
        return None
    params = [x["params"][0].clone() for _, x, _, _, _ in kept]
    grads = [x["grads"][0] for _, x, _, _, _ in kept]
    bufs = [x["bufs"][0].clone() for _, x, _, _, _ in kept]
    scales = [x["scales"][0] for _, x, _, _, _ in kept]
    opt = VARIANTS[variant]
    kw = dict(mu=w.mu, lr=w.lr, scales=scales, coeffs=w.coeff_table, compute=compute)
    if opt is None:
        mn.step(params, grads, bufs, **kw)
    else:
        vs = [vt.clone() for _, _, vt, _, _ in kept] if "beta2" in opt else None
        mn.step_ex(params, grads, bufs, **kw, weight_decay=opt["weight_decay"],
                   cautious=opt["cautious"], second_moments=vs, beta2=opt.get("beta2"),
                   normuon_eps=opt.get("normuon_eps"))
    torch.cuda.synchronize()
    errs = []
    for (idx, _, _, p, new_w), q in zip(kept, params):
        dw = q.double().cpu().numpy() - p
        errs.append(oracle.relative_frobenius_error(dw, new_w - p))
    return {"matrices": len(errs), "max_rel_err_dW": float(f"{max(errs):.3e}"),
            "mean_rel_err_dW": float(f"{sum(errs) / len(errs):.3e}"),
            "bar": 2e-2 if compute == "bf16" else 1e-4,
            "how": "the CPU baseline's sampled matrices as one step of their own from the "
                   "seeded state, dW = W' - W against the fp64 oracle's, relative Frobenius "
                   "error per matrix"}


def measure_peaks(torch, mn, dev):
    """The two probes of the library, timed with events on the stream they run
    on: sustained bf16 MFMA TFLOP/s (1024 workgroups of 8 waves, 4 MFMA
    chains each, no memory traffic) and sustained copy GB/s (2 GiB in 16-byte
    accesses, read + write)."""
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    blocks, iters = 1024, 100000
    sink = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    mn.probe_mfma_bf16(sink, blocks, 1000)  # warm-up
    e0.record(stream)
    fl = sum(mn.probe_mfma_bf16(sink, blocks, iters) for _ in range(3))
    e1.record(stream)
    torch.cuda.synchronize()
    mfma_tflops = fl / (e0.elapsed_time(e1) * 1e-3) / 1e12
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    copy_gbs = 0.0
    for cblocks in (256, 256 * 2, 256 * 4, 256 * 8, 256 * 16, 256 * 32):
        mn.probe_copy(src, dst, cblocks)  # warm-up
        e0.record(stream)
        moved = sum(mn.probe_copy(src, dst, cblocks) for _ in range(10))
        e1.record(stream)
        torch.cuda.synchronize()
        copy_gbs = max(copy_gbs, moved / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst, sink
    return {"mfma_bf16_tflops": round(mfma_tflops, 1), "copy_gbs": round(copy_gbs, 1),
            "how": "library probes on this GPU in this run: back-to-back "
                   "v_mfma_f32_32x32x16_bf16 on registers (1024 x 8 waves x 4 chains x "
                   "1e5 rounds, 3 launches); 2 GiB copy in 16-byte accesses, 4 loads in "
                   "flight per thread (10 launches each at 256-8192 workgroups, the best)"}


def measure_vendor_gemm(torch, dev, w):
    """The vendor's bf16 GEMM (torch.bmm / torch.mm, hipBLASLt underneath) on
    the workload's largest update product, B (M x M) times X (M x N) batched
    over the group (at most 56 matrices), and on one 8192^3 product: what a
    tuned library reaches on these shapes on this GPU, beside the step's own
    kernels.  Contiguous operands only."""
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    groups = w.oriented_groups()
    (m, n), cnt = max(groups.items(), key=lambda kv: kv[0][0] ** 2 * kv[0][1] * kv[1])
    cnt = min(cnt, 56)
    out = {}
    for key, (a_shape, b_shape, fl) in {
            f"bmm_{cnt}x{m}x{m}_by_{m}x{n}": ((cnt, m, m), (cnt, m, n), 2.0 * cnt * m * m * n),
            "mm_8192x8192x8192": ((8192, 8192), (8192, 8192), 2.0 * 8192 ** 3)}.items():
        g = torch.Generator(device=dev).manual_seed(0)
        a = torch.randn(a_shape, generator=g, device=dev, dtype=torch.bfloat16)
        b = torch.randn(b_shape, generator=g, device=dev, dtype=torch.bfloat16)
        mul = torch.bmm if a.dim() == 3 else torch.mm
        c = mul(a, b)  # warm-up (and the library's kernel choice)
        reps = 5
        e0.record(stream)
        for _ in range(reps):
            mul(a, b, out=c)
        e1.record(stream)
        torch.cuda.synchronize()
        out[key + "_tflops"] = round(fl * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12, 1)
        del a, b, c
    out["how"] = ("torch.bmm / torch.mm in bf16 on contiguous random operands, 5 calls after "
                  "one warm-up call, HIP events on the current stream")
    return out


# Same-shape sets of --tile-sweep: (count, rows, cols), square and wide, from
# under one round of 256 x 256 tiles on the 256 CUs to about eight.
TILE_SWEEP_SETS = ([(c, 1280, 1280) for c in (8, 12, 16, 20, 24)]
                   + [(c, 1024, 1024) for c in (16, 24, 32)]
                   + [(c, 768, 768) for c in (32, 48, 64)]
                   + [(c, 1536, 1536) for c in (8, 10, 14)]
                   + [(c, 2048, 2048) for c in (4, 6, 8)]
                   + [(8, 1280, 5120), (20, 1280, 5120), (16, 768, 3072), (8, 1024, 4096),
                      (4, 2048, 8192)])


def tile_sweep(torch, mn, wl, reps=11):
    """One JSON line per set: the median step time over `reps` eager steps and
    the median launch time of each kernel kind (HIP events of the library)."""
    import dataclasses
    dev = "cuda:0"
    for cnt, r, c in TILE_SWEEP_SETS:
        w = dataclasses.replace(wl.GPT_D768, name=f"{cnt}x{r}x{c}", shapes=((r, c),) * cnt)
        inp = wl.make_inputs(w, device=dev)
        ws = torch.empty(mn.step_workspace_bytes(w.shapes, "bf16"), dtype=torch.uint8,
                         device=dev)

        def run():
            mn.step(inp["params"], inp["grads"], inp["bufs"], mu=w.mu, lr=w.lr,
                    scales=inp["scales"], coeffs=w.coeff_table, workspace=ws)
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            run()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        mn.timing_enable(True)
        mn.timing_read()
        for _ in range(5):
            run()
        torch.cuda.synchronize()
        mn.timing_enable(False)
        per = {}
        for rec in mn.timing_read():
            per.setdefault(rec["kind"], []).append(rec["ms"])
        t256, n256 = -(-r // 256), -(-c // 256)
        print(json.dumps({
            "set": w.name, "count": cnt, "rows": r, "cols": c,
            "tile_env": os.environ.get("MUON_GEMM_TILE", ""),
            "tiles": {"gram": pick_tile(t256, cnt, "gram"), "poly": pick_tile(t256, cnt, "tri"),
                      "update": pick_tile(t256 * n256, cnt, "full")},
            "step_ms": round(sorted(ts)[len(ts) // 2], 4),
            "kinds": {k: round(sorted(v)[len(v) // 2], 4) for k, v in per.items()}}), flush=True)
        del inp, ws
        torch.cuda.empty_cache()


# (rows, cols, batches): the 3.8B set's square and wide groups around 56
# matrices (4368 lower-triangle tiles of 256 = 17.06 rounds of the 256 CUs),
# and the d768 set's wide group, whose launches hold a few rounds only.
BATCH_SWEEP_SETS = ((3072, 3072, (48, 52, 54, 55, 56, 57, 58, 60, 64)),
                    (3072, 12288, (52, 55, 56, 57)),
                    (768, 3072, (8, 12, 16, 20, 24, 32)))


def batch_sweep(torch, mn, reps=3):
    """For each set, one JSON line per batch with the median launch time of
    each GEMM kind over `reps` bf16 orthogonalisations (HIP events of the
    library), then one line per kind with two fits of launch time against
    the batch: a straight line (time proportional to the tiles) and a
    multiple of the rounds of 256 workgroups the launch needs (time set by
    whole rounds), each with its largest relative residual."""
    import numpy as np
    dev = "cuda:0"
    for rows, cols, batches in BATCH_SWEEP_SETS:
        per_batch = {}
        for batch in batches:
            g = torch.Generator(device=dev).manual_seed(batch)
            x = (torch.randn(batch, rows, cols, device=dev, generator=g) * 1e-3).to(torch.bfloat16)
            out = torch.empty_like(x)
            mn.orthogonalize(x, out=out)
            torch.cuda.synchronize()
            mn.timing_enable(True)
            mn.timing_read()
            for _ in range(reps):
                mn.orthogonalize(x, out=out)
            torch.cuda.synchronize()
            mn.timing_enable(False)
            per = {}
            for rec in mn.timing_read():
                if rec["kind"] in ("gram", "poly", "update", "gramq"):
                    per.setdefault(rec["kind"], []).append(rec["ms"])
            kinds = {k: round(float(np.median(v)), 4) for k, v in per.items()}
            per_batch[batch] = kinds
            print(json.dumps({"rows": rows, "cols": cols, "batch": batch, "kinds": kinds}),
                  flush=True)
            del x, out
            torch.cuda.empty_cache()
        t256, n256 = -(-rows // 256), -(-cols // 256)
        for kind in sorted({k for v in per_batch.values() for k in v}):
            bs = np.array([b for b in batches if kind in per_batch[b]], dtype=float)
            ms = np.array([per_batch[int(b)][kind] for b in bs])
            full = kind == "update"
            per256 = t256 * n256 if full else t256 * (t256 + 1) // 2
            per128 = 4 * t256 * n256 if full else (2 * t256) * (2 * t256 + 1) // 2
            tiles = bs * per256
            tile = [pick_tile(t256 * n256 if full else t256, int(b),
                              "full" if full else "gram" if kind == "gram" else "tri")
                    for b in bs]
            line = np.polyfit(bs, ms, 1)
            res_line = np.abs(np.polyval(line, bs) - ms) / ms
            # whole rounds: 256 workgroups of 256-tiles, or 512 of 128-tiles
            rounds = np.array([-(-int(b) * per256 // 256) if tl == 256
                               else -(-int(b) * per128 // 512)
                               for b, tl in zip(bs, tile)], dtype=float)
            per_round = float(np.dot(rounds, ms) / np.dot(rounds, rounds))
            res_round = np.abs(rounds * per_round - ms) / ms
            print(json.dumps({"rows": rows, "cols": cols, "kind": kind,
                              "tiles_256": [int(t) for t in tiles], "tile": tile,
                              "line_ms": [round(float(line[1]), 4), round(float(line[0]), 5)],
                              "line_max_rel_residual": round(float(res_line.max()), 4),
                              "ms_per_round": round(per_round, 4),
                              "rounds_max_rel_residual": round(float(res_round.max()), 4)}),
                  flush=True)


def overlap_probe(torch, mn, copy_gib=32, reps=2):
    """The two probes alone, then the copy launched first and the MFMA probe
    right after it on a second stream, so both run on the same CUs: one JSON
    line with each one's rate alone, and while both run.  The copy's rate
    while the MFMA probe runs is estimated from its total time, taking the
    rest of the copy at its solo rate."""
    dev = "cuda:0"
    s_m, s_c = torch.cuda.Stream(dev), torch.cuda.Stream(dev)
    sink = torch.empty(1024 * 512, dtype=torch.float32, device=dev)
    src = torch.empty(copy_gib << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)

    def launch(stream, fn):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            a.record(stream)
            work = fn()
            b.record(stream)
        return a, b, work
    mfma = lambda blocks, iters: launch(s_m, lambda: mn.probe_mfma_bf16(sink, blocks, iters))
    copy = lambda blocks: launch(s_c, lambda: mn.probe_copy(src, dst, blocks))
    mfma(256, 1000)
    copy(256)
    torch.cuda.synchronize()
    out = {}
    a, b, fl = mfma(256, 90000)
    torch.cuda.synchronize()
    out["mfma_alone"] = {"tflops": round(fl / (a.elapsed_time(b) * 1e-3) / 1e12, 1),
                         "ms": round(a.elapsed_time(b), 2)}
    a, b, mv = copy(256)
    torch.cuda.synchronize()
    solo = a.elapsed_time(b)
    out["copy_alone"] = {"gbs": round(mv / (solo * 1e-3) / 1e9, 1), "ms": round(solo, 2)}
    out["both"] = []
    for _ in range(reps):
        ca, cb, mv = copy(256)
        ma, mb, fl = mfma(256, 90000)
        torch.cuda.synchronize()
        tm, tc = ma.elapsed_time(mb), ca.elapsed_time(cb)
        rest = max(0.0, tc - tm)
        during = max(0.0, mv - mv * rest / solo) / (tm * 1e-3) / 1e9
        out["both"].append({"mfma_tflops": round(fl / (tm * 1e-3) / 1e12, 1),
                            "mfma_ms": round(tm, 2), "copy_ms": round(tc, 2),
                            "copy_gbs_while_mfma_runs": round(during, 1)})
    out["how"] = (f"256 workgroups of 8 MFMA waves (2 per SIMD, 4 independent chains each, "
                  f"90000 rounds); a {copy_gib} GiB copy, 256 workgroups of 256 threads, "
                  f"16-byte accesses; HIP events on each stream")
    print(json.dumps(out), flush=True)


def tile_table(paths):
    """Markdown: per set, step and per-kernel times at 128 and 256 tiles and
    with the library's choice (the outputs of three --tile-sweep runs)."""
    runs = []
    for p in paths:
        runs.append({d["set"]: d for d in (json.loads(l) for l in open(p) if l.startswith("{"))})
    print("| set | tiles at 256 (triangle / full) | step ms 128 / 256 / chosen | chosen tiles "
          "(gram / poly / full) | gram | poly | update | final |")
    print("|---|---|---|---|---|---|---|---|")
    for name, ch in runs[2].items():
        a, b = runs[0][name], runs[1][name]
        t, n = -(-ch["rows"] // 256), -(-ch["cols"] // 256)
        cells = []
        for k in ("gram", "poly", "update", "final"):
            pick = ch["tiles"][k if k in ("gram", "poly") else "update"]
            x, y = a["kinds"][k], b["kinds"][k]
            best = "128" if x < y else "256"
            cells.append(f"{x:.3f} / {y:.3f}" + (" ✓" if str(pick) == best else ""))
        print(f"| {name} | {t * (t + 1) // 2 * ch['count']} / {t * n * ch['count']} | "
              f"{a['step_ms']:.3f} / {b['step_ms']:.3f} / {ch['step_ms']:.3f} | "
              f"{ch['tiles']['gram']} / {ch['tiles']['poly']} / {ch['tiles']['update']} | "
              + " | ".join(cells) + " |")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the Muon step shards by whole matrix and "
              f"this library runs one GPU's share; --gpus {args.gpus} is not supported.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import muon_newton_schulz_step_amd as mn
    import workloads as wl

    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.tile_table:
        tile_table(args.tile_table)
        return
    if args.tile_sweep:
        tile_sweep(torch, mn, wl)
        return
    if args.batch_sweep:
        batch_sweep(torch, mn)
        return
    if args.overlap_probe:
        overlap_probe(torch, mn)
        return
    w = wl.WORKLOADS[args.workload]
    full_count = len(w.shapes)
    if args.owner_share is not None and (args.owner_share < 1 or args.matrices):
        print("--owner-share takes N >= 1 and does not combine with --matrices",
              file=sys.stderr)
        sys.exit(2)
    if args.coeffs or args.ns_steps or args.matrices or args.owner_share:
        import dataclasses
        w = dataclasses.replace(
            w, coeffs={"quintic": wl.QUINTIC, "cubic": wl.CUBIC}[args.coeffs or "quintic"]
            if args.coeffs else w.coeffs,
            n_steps=args.ns_steps or w.n_steps,
            shapes=(tuple(w.shapes[i] for i in wl.sample_indices(w, args.matrices))
                    if args.matrices else
                    tuple(w.shapes[i] for i in wl.owner_indices(w, args.owner_share))
                    if args.owner_share else w.shapes))
    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1], w)
        return
    if args.write_mfma:
        write_mfma(args.write_mfma, w)
        return
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inputs = wl.make_inputs(w, device=dev)
    torch.cuda.synchronize()
    ws = mn.Workspace()

    opt = VARIANTS[args.variant]
    vs = None
    if opt is not None and "beta2" in opt:
        vs = [wl.make_second_moment(w, i, device=dev) for i in range(len(w.shapes))]

    def one_step():
        if opt is None:
            mn.step(inputs["params"], inputs["grads"], inputs["bufs"], mu=w.mu, lr=w.lr,
                    scales=inputs["scales"], coeffs=w.coeff_table, compute=args.compute,
                    workspace=ws)
        else:
            mn.step_ex(inputs["params"], inputs["grads"], inputs["bufs"], mu=w.mu, lr=w.lr,
                       scales=inputs["scales"], coeffs=w.coeff_table, compute=args.compute,
                       workspace=ws, second_moments=vs, **opt)

    if args.calibrate:
        # known work for the counter passes: the MFMA probe, then a plain copy
        sink = torch.empty(CAL_MFMA[0] * 512, dtype=torch.float32, device=dev)
        mn.probe_mfma_bf16(sink, *CAL_MFMA)
        src = torch.ones(COPY_BYTES // 4, device=dev)
        dst = torch.empty_like(src)
        mn.probe_copy(src, dst, 256 * 16)
        torch.cuda.synchronize()
        del src, dst, sink
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    stream = torch.cuda.current_stream(dev)
    # an event after every step: the whole region (first to last) gives the
    # mean, the gaps between them the median and the minimum
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    mn.timing_enable(False)
    if args.graph:
        # the workspace was allocated by the warm-up steps: capture allocates nothing
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        graph.replay()
        torch.cuda.synchronize()
        ev[0].record(stream)
        for i in range(args.steps):
            graph.replay()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        del graph
    else:
        ev[0].record(stream)
        for i in range(args.steps):
            one_step()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
    ms_per_step = ev[0].elapsed_time(ev[-1]) / args.steps
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    ms_median = per_step[len(per_step) // 2] if len(per_step) % 2 else \
        0.5 * (per_step[len(per_step) // 2 - 1] + per_step[len(per_step) // 2])
    # the per-kernel pass: the same steps again, each launch between events
    mn.timing_enable(True)
    mn.timing_read()
    for _ in range(args.steps):
        one_step()
    torch.cuda.synchronize()
    mn.timing_enable(False)
    gc.enable()
    records = mn.timing_read()
    kernels = kernel_summary(records, args.steps)
    peaks = None if args.no_peaks else measure_peaks(torch, mn, dev)
    if peaks is not None and args.compute == "bf16":
        try:  # context only: a failure here must not cost the measurement
            peaks["vendor_gemm"] = measure_vendor_gemm(torch, dev, w)
        except Exception as e:  # noqa: BLE001
            peaks["vendor_gemm"] = {"error": f"{type(e).__name__}: {e}"[:200]}
    ns = [k for k in kernels if k["kind"] in ("gram", "gramq", "poly", "update", "final")]
    ns_ms = sum(k["ms"] for k in ns) / args.steps
    flops = w.ns_flops_counted()
    exec_flops = sum(k["exec_flops"] for k in ns) / args.steps
    ns_tflops = flops / (ns_ms * 1e-3) / 1e12
    step_tflops = flops / (ms_per_step * 1e-3) / 1e12
    dom = kernels[0]
    dom_key = f"{dom['kind']}_{dom['m']}x{dom['n']}"
    bound = "mfma" if dom["kind"] in ("gram", "gramq", "poly", "update", "final") else "hbm"
    sec = dom["avg_launch_ms"] * 1e-3
    if bound == "mfma":
        # algorithmic flops of one launch: the method's count for its matrices
        achieved = dom["flops"] / dom["launches"] / sec / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK[args.compute],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK[args.compute], 4),
                "achieved_executed": round(dom["exec_flops"] / dom["launches"] / sec / 1e12, 2)}
        if peaks and args.compute == "bf16":
            roof["measured_peak"] = peaks["mfma_bf16_tflops"]
            roof["frac_of_measured_peak"] = round(achieved / peaks["mfma_bf16_tflops"], 4)
    else:
        achieved = dom["bytes"] / dom["launches"] / sec / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        if peaks:
            roof["measured_peak"] = peaks["copy_gbs"]
            roof["frac_of_measured_peak"] = round(achieved / peaks["copy_gbs"], 4)
    roof["kernel"] = dom_key
    roof["avg_launch_ms"] = round(dom["avg_launch_ms"], 4)
    roof["traffic"] = traffic_from_profiles(dom_key)
    if bound == "mfma":
        # fraction of cycles the matrix pipes were busy in this launch kind,
        # from the committed MFMA counter summary (calibrated on the probe)
        m = profile_entry(MFMA_JSON, dom_key)
        roof["mfma_busy"] = None if m is None else round(m["mfma_busy_frac"], 3)

    # element-wise part: the optimizer state's own bytes per element (gradient
    # read, momentum read and written, weights read and written); prep moves
    # the first three (and writes X_0), the weights move in the FINAL epilogue
    elements = sum(r * c for r, c in w.shapes)
    gbytes = 2 if w.grad_dtype == torch.bfloat16 else 4
    preps = [k for k in kernels if k["kind"] in ("prep", "norm")]
    prep_ms = sum(k["ms"] for k in preps) / args.steps
    prep_moved = sum(k["bytes"] for k in preps) / args.steps
    elementwise = {
        "algorithmic_bytes_per_element": gbytes + 16, "elements": elements,
        "prep_norm_ms_per_step": round(prep_ms, 4),
        "prep_gbs_moved": round(prep_moved / (prep_ms * 1e-3) / 1e9, 1) if prep_ms > 0 else None,
        "prep_frac_of_hbm_peak": round(prep_moved / (prep_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        if prep_ms > 0 else None,
        "note": "weights are read and written inside the last update's epilogue, whose "
                "time is not separable from its GEMM"}
    if peaks and prep_ms > 0:
        elementwise["prep_frac_of_measured_copy"] = round(
            prep_moved / (prep_ms * 1e-3) / 1e9 / peaks["copy_gbs"], 4)

    cpu = parity = None
    if not args.no_cpu_baseline:
        kept = []
        cpu = cpu_baseline(w, args.cpu_sample_seconds, args.variant, dev=dev, keep=kept)
        parity = sample_parity(torch, mn, w, kept, args.variant, args.compute)
        del kept

    groups = w.oriented_groups()
    out = {
        "metric": METRIC if args.variant == "plain" else METRIC + f" ({args.variant})",
        "value": round(ms_per_step, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "ms_per_step_median": round(ms_median, 3),
        "ms_per_step_min": round(per_step[0], 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.compute,
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": w.name, "matrices": len(w.shapes),
                   **({"owner_share": f"rank 0 of {args.owner_share}", "of": full_count}
                      if args.owner_share else
                      {"sample_of": full_count} if len(w.shapes) != full_count else {}),
                   "variant": args.variant,
                   **({"options": opt} if opt else {}),
                   "oriented_groups": {f"{m}x{n}": c for (m, n), c in groups.items()},
                   "ns_steps": w.n_steps, "coeffs": list(w.coeffs),
                   "launch": "hip graph replay" if args.graph else "eager",
                   "parallelism": (f"single GPU: the {len(w.shapes)} matrices that one rank "
                                   f"owns in a {args.owner_share}-way step sharded by whole "
                                   f"matrix" if args.owner_share else
                                   f"single GPU, all {len(w.shapes)} matrices of the set")},
        "ns_tflops": round(ns_tflops, 2),
        "ns_ms_per_step": round(ns_ms, 3),
        "ns_frac_of_peak": round(ns_tflops / PEAK[args.compute], 4),
        "step_tflops": round(step_tflops, 2),
        "counted_ns_tflop_per_step": round(flops / 1e12, 3),
        "executed_ns_tflop_per_step": round(exec_flops / 1e12, 3),
        "ns_tflops_executed": round(exec_flops / (ns_ms * 1e-3) / 1e12, 2),
        "ns_frac_of_peak_executed": round(exec_flops / (ns_ms * 1e-3) / 1e12 / PEAK[args.compute],
                                          4),
        "measured_peaks": peaks,
        "elementwise": elementwise,
        "roofline": roof,
        "cpu_baseline": cpu,
        "parity": parity,
        "kernels": [{k2: (round(v, 4) if isinstance(v, float) else v) for k2, v in k.items()
                     if k2 in ("kind", "m", "n", "batch", "launches", "ms_per_step",
                               "avg_launch_ms", "tflops", "tflops_counted", "gbs")}
                    for k in kernels],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

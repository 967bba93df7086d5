"""Benchmark of the Muon step on the 3.8B GPT matrix set (one MI355X).

A step is one muon_step call over all 168 matrices (momentum, Frobenius
normalisation, 5 Newton-Schulz steps, weight update), inputs resident in HBM.
Prints one JSON line:  metric / value (ms per step) / NS TFLOP/s and its
fraction of the dense bf16 MFMA peak / roofline of the dominant kernel /
the fp64 oracle timed on the host cores as a CPU baseline.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--compute bf16|fp32]
                    [--variant plain|cwd|normuon_cwd] [--graph]

--variant times muon_step_ex instead: page 1's cautious weight decay (cwd,
decay 0.1) or NorMuon (beta2 0.95, eps 1e-8) with it (normuon_cwd).  The
default, plain, is the benchmark's Muon step.  --graph times replays of one
captured step instead of eager calls (the small workloads are bound by the
host cost of their launches); the per-kernel figures then come from an eager
pass after the timed replays.
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
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--graph", action="store_true",
                   help="time replays of one captured step (a HIP graph: no per-launch host "
                        "cost); the per-kernel times then come from an eager pass after it")
    p.add_argument("--cpu-sample-seconds", type=float, default=12.0,
                   help="seconds of oracle work for the CPU baseline sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain 1 GiB device copy (traffic counter calibration)")
    p.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                   help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of a "
                        "'--steps 1 --warmup 0 --calibrate-copy' run into profiles/traffic.json")
    return p.parse_args()


def kernel_summary(records, steps):
    """Aggregate the per-launch HIP-event log by (kind, m, n)."""
    agg = {}
    for r in records:
        key = (r["kind"], r["m"], r["n"])
        a = agg.setdefault(key, {"kind": r["kind"], "m": r["m"], "n": r["n"], "launches": 0,
                                 "ms": 0.0, "flops": 0.0, "bytes": 0.0, "batch": r["batch"]})
        a["launches"] += 1
        a["ms"] += r["ms"]
        a["flops"] += r["flops"]
        a["bytes"] += r["bytes"]
    out = sorted(agg.values(), key=lambda a: -a["ms"])
    for a in out:
        a["ms_per_step"] = a["ms"] / steps
        a["avg_launch_ms"] = a["ms"] / a["launches"]
        a["tflops"] = a["flops"] / (a["ms"] * 1e-3) / 1e12 if a["ms"] > 0 else 0.0
        a["gbs"] = a["bytes"] / (a["ms"] * 1e-3) / 1e9 if a["ms"] > 0 else 0.0
    return out


KERNEL_SRC = os.path.join(ROOT, "muon_newton_schulz_step_amd", "csrc", "muon_kernels.hip")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
COPY_BYTES = 1 << 30


def kernel_source_digest():
    import hashlib
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()


def traffic_from_profiles(kernel_key):
    """HBM bytes per launch of a kernel from the committed counter summary,
    or None if there is none for the current kernel source."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    try:
        with open(TRAFFIC_JSON) as f:
            data = json.load(f)
        if data.get("kernel_source_sha256") != kernel_source_digest():
            return None
        k = data["kernels"].get(kernel_key)
        return None if k is None else k["traffic_bytes"]
    except Exception:
        return None


def launch_sequence(w):
    """(kind, m, n) of every library launch of one bf16 step, in launch order:
    per oriented group (first appearance) and chunk of at most 64 matrices,
    prep, norm, then gram, poly, update per Newton-Schulz step, the last
    update being one final launch for the chunk's wide matrices and one for
    its tall ones.  Groups with padded N >= 4M and M >= 2048 form the Gram
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
            finals = [("final", m, n)] * ((not all(chunk)) + any(chunk))
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
            tile = 256 if compute == "bf16" and t256 * (t256 + 1) // 2 * cnt >= 512 else 128
            tri = (M // tile) * (M // tile + 1) // 2 * tile * tile * cnt  # C elements computed
            qaq = compute == "bf16" and N >= 4 * M and M >= 2048
            for k in range(w.n_steps):
                if qaq and k in (1, 3) and k <= w.n_steps - 2:
                    tot += 2 * (2.0 * tri * M)
                else:
                    tot += 2.0 * tri * N
                tot += 2.0 * tri * M                   # POLY
                tot += 2.0 * M * N * M * cnt           # UPDATE / FINAL (full tiles)
    return tot


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
        first = next(i for i, (name, _) in enumerate(rows) if "muon" in name)
        copy_kib = rows[first - 1][1]  # the calibration copy runs right before the step
        scale = COPY_BYTES / (copy_kib * 1024.0)
        out[field + "_scale"] = scale
        muon = [v for name, v in rows if "muon" in name]
        if len(muon) != len(seq):
            raise SystemExit(f"{len(muon)} library dispatches in {path}, expected {len(seq)}")
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


def cpu_baseline(w, seconds, variant="plain"):
    """The fp64 oracle on a bounded sample of the workload: matrices taken
    round-robin over the oriented groups until about `seconds` of CPU work,
    per-group mean times extrapolated by the group counts."""
    import oracle
    import workloads as wl
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"), default=os.cpu_count())
    except Exception:
        threads = os.cpu_count()
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
            x = wl.make_inputs(w, device="cpu", indices=[idx])
            g = x["grads"][0].double().numpy()
            b = x["bufs"][0].double().numpy()
            p = x["params"][0].double().numpy()
            opt = VARIANTS[variant]
            t0 = time.perf_counter()
            if opt is None:
                oracle.muon_step(p, g, b, w.mu, w.lr, x["scales"][0], w.coeff_table)
            else:
                v = (wl.make_second_moment(w, idx).double().numpy()
                     if "beta2" in opt else None)
                oracle.muon_step_ex(p, g, b, w.mu, w.lr, x["scales"][0], w.coeff_table,
                                    weight_decay=opt["weight_decay"], cautious=opt["cautious"],
                                    second_moment=v, beta2=opt.get("beta2", 0.0),
                                    normuon_eps=opt.get("normuon_eps", 0.0))
            dt = time.perf_counter() - t0
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
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the Muon step shards by whole matrix and "
              f"this build runs one GPU's share; --gpus {args.gpus} is not supported.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import muon_newton_schulz_step_amd as mn
    import workloads as wl

    w = wl.WORKLOADS[args.workload]
    if args.write_traffic:
        write_traffic(args.write_traffic[0], args.write_traffic[1], w)
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

    if args.calibrate_copy:
        src = torch.ones(COPY_BYTES // 4, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)  # one elementwise kernel: reads and writes COPY_BYTES
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        one_step()
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    graph_ms = None
    if args.graph:
        # the workspace was allocated by the warm-up steps: capture allocates nothing
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            one_step()
        graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / args.steps
        del graph
    mn.timing_enable(True)
    mn.timing_read()  # drop warm-up records
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        one_step()
    e1.record(stream)
    torch.cuda.synchronize()
    mn.timing_enable(False)
    gc.enable()
    ms_per_step = graph_ms if args.graph else e0.elapsed_time(e1) / args.steps
    records = mn.timing_read()
    kernels = kernel_summary(records, args.steps)
    ns = [k for k in kernels if k["kind"] in ("gram", "gramq", "poly", "update", "final")]
    ns_ms = sum(k["ms"] for k in ns) / args.steps
    flops = w.ns_flops_counted()
    ns_tflops = flops / (ns_ms * 1e-3) / 1e12
    step_tflops = flops / (ms_per_step * 1e-3) / 1e12
    dom = kernels[0]
    dom_key = f"{dom['kind']}_{dom['m']}x{dom['n']}"
    bound = "mfma" if dom["kind"] in ("gram", "gramq", "poly", "update", "final") else "hbm"
    if bound == "mfma":
        achieved = dom["flops"] / dom["launches"] / (dom["avg_launch_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK[args.compute],
                "unit": "TFLOP/s", "frac": round(achieved / PEAK[args.compute], 4)}
    else:
        achieved = dom["bytes"] / dom["launches"] / (dom["avg_launch_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["kernel"] = dom_key
    roof["avg_launch_ms"] = round(dom["avg_launch_ms"], 4)
    roof["traffic"] = traffic_from_profiles(dom_key)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_sample_seconds, args.variant)

    groups = w.oriented_groups()
    out = {
        "metric": METRIC if args.variant == "plain" else METRIC + f" ({args.variant})",
        "value": round(ms_per_step, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.compute,
        "data": "synthetic (seeded, generated on the GPU)",
        "config": {"workload": w.name, "matrices": len(w.shapes), "variant": args.variant,
                   **({"options": opt} if opt else {}),
                   "oriented_groups": {f"{m}x{n}": c for (m, n), c in groups.items()},
                   "ns_steps": w.n_steps, "coeffs": list(w.coeffs),
                   "launch": "hip graph replay" if args.graph else "eager",
                   "parallelism": "single GPU (one GPU's share of a matrix-sharded step)"},
        "ns_tflops": round(ns_tflops, 2),
        "ns_ms_per_step": round(ns_ms, 3),
        "ns_frac_of_peak": round(ns_tflops / PEAK[args.compute], 4),
        "step_tflops": round(step_tflops, 2),
        "counted_ns_tflop_per_step": round(flops / 1e12, 3),
        "executed_ns_tflop_per_step": round(ns_flops_executed(w, args.compute) / 1e12, 3),
        "ns_tflops_executed": round(ns_flops_executed(w, args.compute) / (ns_ms * 1e-3) / 1e12, 2),
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": [{k2: (round(v, 4) if isinstance(v, float) else v) for k2, v in k.items()
                     if k2 in ("kind", "m", "n", "batch", "launches", "ms_per_step",
                               "avg_launch_ms", "tflops", "gbs")} for k in kernels],
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Host-side logic of bench.py, on the CPU: the refusal of several GPUs,
the launch-sequence model the counter summaries are matched against, the
executed-flop count, and the labels given to kernel names."""
import json
import os
import subprocess
import sys

import bench
import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert out.returncode == 2
    assert "one GPU" in out.stderr and out.stdout == ""


def test_bad_owner_share_is_refused():
    for extra in (["--owner-share", "0"], ["--owner-share", "8", "--matrices", "2"]):
        out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *extra],
                             capture_output=True, text=True, timeout=120, cwd=ROOT)
        assert out.returncode == 2, extra
        assert "--owner-share" in out.stderr and out.stdout == ""


def test_launch_sequence_of_the_3p8b_step():
    seq = bench.launch_sequence(wl.GPT_3P8B)
    groups = {}
    for kind, m, n in seq:
        groups.setdefault((m, n), []).append(kind)
    assert list(groups) == [(3072, 3072), (1024, 3072), (3072, 12288)]
    # square and wide groups: prep, norm, 5 x (gram, poly), 4 updates, 1 final
    for key in ((3072, 3072), (1024, 3072)):
        g = groups[key]
        assert g[:2] == ["prep", "norm"] and g.count("gram") == 5 and g.count("poly") == 5
        assert g.count("update") == 4 and g.count("final") == 1 and len(g) == 17
    # the 3072 x 12288 group: the Gram matrix of steps 1 and 3 formed as
    # Q A Q (two launches counted as gramq each), one final per orientation
    # (28 + 28, each part alone takes 256 x 256 tiles: 63 rounds of the CUs)
    g = groups[(3072, 12288)]
    assert g.count("gram") == 3 and g.count("gramq") == 4 and g.count("poly") == 5
    assert g.count("update") == 4 and g.count("final") == 2


def test_launch_sequence_mixed_final_when_parts_are_small():
    # d768: the (768, 3072) chunk holds 8 wide and 8 tall matrices, 36 tiles
    # of 256 x 256 each: one final launch for both
    seq = bench.launch_sequence(wl.GPT_D768)
    finals = [(m, n) for kind, m, n in seq if kind == "final"]
    assert finals == [(768, 768), (768, 3072)]


def test_tile_choice_model():
    # rounds of the 256 CUs: 256-tiles when 1.6 rounds of 128-tiles (1.4 for
    # the Gram) per round of 256 make up for the larger tile
    pt = bench.pick_tile
    assert pt(12 * 48, 56, "full") == 256   # 3.8B update: 126 vs 252 rounds
    assert pt(12, 56, "gram") == 256        # its Gram: 18 vs 33
    assert pt(12, 56, "tri") == 256         # and polynomial
    assert pt(4, 56, "tri") == 128          # (1024, 3072) polynomial: 3 vs 4
    assert pt(4, 56, "gram") == 128         # its Gram: 1.4 x 3 > 4
    assert pt(4 * 12, 56, "full") == 256    # its update: 3 vs 6
    assert pt(25, 16, "full") == 256        # 16 x 1280^2 update: 2 vs 4
    assert pt(25, 12, "full") == 128        # 12 x 1280^2: 2 vs 3
    assert pt(25, 8, "full") == 256         # 8 x 1280^2: 1 vs 2
    assert pt(5, 20, "gram") == 256         # 20 x 1280^2 Gram: 1.4 x 2 <= 3
    assert pt(5, 20, "tri") == 128          # its polynomial: 1.6 x 2 > 3
    assert pt(5, 8, "tri") == 128           # 8 x 1280^2: 1 vs 1
    assert pt(8, 4, "gram") == 256          # 4 x 2048 x 8192 Gram: 1 vs 2
    assert pt(12 * 48, 56, "full", "fp32") == 128


def test_executed_flops_of_the_3p8b_step():
    # the figure the MFMA counters measured on the GPU (profiles/mfma.json)
    assert bench.ns_flops_executed(wl.GPT_3P8B) == 138854145196032.0
    # counted: the method's 4 m^2 n + 2 m^3 per matrix and step
    assert abs(wl.GPT_3P8B.ns_flops_counted() - 1.99029e14) < 1e9


def test_kernel_labels():
    name = "void muon::gemm_kernel<__bf16, 2, 256, 256, 2, 4, 2, true, true, true>(muon::GemmLaunch)"
    mangled = "_ZN4muon11gemm_kernelIDF16bLi2ELi256ELi256ELi2ELi4ELi2ELb1ELb1ELb1EEEvNS_10GemmLaunchE"
    assert bench.kernel_label(mangled) == "gemm<bf16,UPDATE,256x256,8w,rowQ,buf,stream>"
    mixed = "_ZN4muon11gemm_kernelIDF16bLi10ELi128ELi128ELi2ELi2ELi2ELb1ELb0ELb1EEEvNS_10GemmLaunchE"
    assert bench.kernel_label(mixed) == "gemm<bf16,FINAL_W_MIX,128x128,4w,rowQ,dma,stream>"
    assert bench.kernel_label(name)  # demangled names get a label too


def test_tile_table_marks_the_faster_tile(tmp_path, capsys):
    # three --tile-sweep outputs of one set: the table shows both tiles'
    # launch times and marks the kinds where the chosen tile is the faster
    def line(env, step, kinds, tiles):
        return json.dumps({"set": "4x2048x2048", "count": 4, "rows": 2048, "cols": 2048,
                           "tile_env": env, "tiles": tiles, "step_ms": step, "kinds": kinds})
    chosen = {"gram": 256, "poly": 256, "update": 128}
    paths = []
    for env, step, kinds in (
            ("128", 1.05, {"gram": 0.054, "poly": 0.057, "update": 0.076, "final": 0.101}),
            ("256", 0.97, {"gram": 0.049, "poly": 0.051, "update": 0.075, "final": 0.093}),
            ("", 0.99, {"gram": 0.049, "poly": 0.051, "update": 0.076, "final": 0.101})):
        p = tmp_path / f"ts_{env or 'auto'}.jsonl"
        p.write_text(line(env, step, kinds, chosen) + "\n")
        paths.append(str(p))
    bench.tile_table(paths)
    rows = [r for r in capsys.readouterr().out.splitlines() if r.startswith("| 4x2048")]
    assert len(rows) == 1
    cells = [c.strip() for c in rows[0].strip("|").split("|")]
    assert cells[1] == "144 / 256"   # tiles at 256 over the 4 matrices: triangle / full
    assert cells[2] == "1.050 / 0.970 / 0.990"
    assert cells[3] == "256 / 256 / 128"
    assert cells[4].endswith("✓") and cells[5].endswith("✓")   # 256 was faster
    assert not cells[6].endswith("✓")                  # update: 256 faster, 128 chosen
    assert not cells[7].endswith("✓")


def test_counter_summaries_only_for_the_current_kernels(tmp_path):
    # a summary keyed to other kernel sources is not used (null in the line)
    good = {"kernel_source_sha256": bench.kernel_source_digest(),
            "kernels": {"update_3072x12288": {"traffic_bytes": 1.0, "mfma_busy_frac": 0.5}}}
    stale = dict(good, kernel_source_sha256="0" * 64)
    for data, expect in ((good, 0.5), (stale, None)):
        p = tmp_path / "summary.json"
        p.write_text(json.dumps(data))
        e = bench.profile_entry(str(p), "update_3072x12288")
        assert (e["mfma_busy_frac"] if e else None) == expect
    assert bench.profile_entry(str(tmp_path / "missing.json"), "update_3072x12288") is None


def test_launch_sequence_groups_match_the_library():
    # bench.py's model of the launch order groups matrices as the library's
    # planner does: oriented shapes in order of first appearance, chunks of
    # at most 64 (one prep launch each)
    import dataclasses
    import random
    import muon_newton_schulz_step_amd as mn
    rng = random.Random(11)
    sides = (1, 64, 130, 300, 768, 1024, 2049)
    for _ in range(40):
        shapes = tuple((rng.choice(sides), rng.choice(sides)) for _ in range(rng.randint(1, 150)))
        w = dataclasses.replace(wl.GPT_D768, shapes=shapes)
        _, groups = mn.plan_groups(shapes)
        seq = bench.launch_sequence(w)
        order, preps = [], {}
        for kind, m, n in seq:
            if (m, n) not in preps:
                order.append((m, n))
                preps[(m, n)] = 0
            preps[(m, n)] += kind == "prep"
        assert order == [(m, n) for m, n, _ in groups]
        assert [preps[(m, n)] for m, n, _ in groups] == [-(-c // 64) for _, _, c in groups]

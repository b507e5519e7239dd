"""Host-side pieces of bench.py (no GPU): the one-GPU guard and the code hash
that keys the stored HBM traffic summary to the kernel source."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_code_hash_ignores_comments_and_whitespace(tmp_path):
    src = 'int f(int x) {\n    // twice\n    return 2 * x; /* no carry */\n}\nconst char *s = "a // b";\n'
    a = tmp_path / "a.hip"
    a.write_text(src)
    h = bench._code_sha256(str(a))
    a.write_text(src.replace("// twice", "// two times x").replace("    return", "\n\treturn"))
    assert bench._code_sha256(str(a)) == h
    a.write_text(src.replace("2 * x", "3 * x"))                 # code
    assert bench._code_sha256(str(a)) != h
    a.write_text(src.replace('"a // b"', '"a // c"'))           # a string literal is code
    assert bench._code_sha256(str(a)) != h


def _fake_pmc(tmp_path, workload):
    """One rocprofv3-style counter CSV for one step of `workload`: the pack
    copy kernel reads and writes the set once (FETCH_SIZE reads half of it, as
    the copy kernel's calibration found), a B X launch 3 GB and 1 GB."""
    import csv
    ms = bench.build_workload(workload)
    copy_kib = sum(bench._numel(s) for s in ms.shapes) * 2 / 1024.0
    d = tmp_path / "pmc"
    d.mkdir()
    bx = "_ZN3nsq12_GLOBAL__N_117ns_product_kernelIDF16bNS0_7TileCfgILi256ELi2ELi4ELi128ELi2EEELi2ELb0EDF16bEEv"
    rows = [(1, "_ZN3nsq12_GLOBAL__N_117route_copy_kernelILb1EEEvPKNS_8RouteSegE", "FETCH_SIZE", copy_kib / 2),
            (1, "_ZN3nsq12_GLOBAL__N_117route_copy_kernelILb1EEEvPKNS_8RouteSegE", "WRITE_SIZE", copy_kib),
            (2, bx, "FETCH_SIZE", 3e9 / 1024 / 2), (2, bx, "WRITE_SIZE", 1e9 / 1024),
            (2, bx, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 4 * 256 * 1e6), (2, bx, "GRBM_GUI_ACTIVE", 8e6),
            (2, bx, "SQ_INSTS_VALU_MFMA_MOPS_BF16", bench.alg_phase_flops(ms)["bx"] / 512)]
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)
    return d


def test_counter_summary_and_stored_traffic(tmp_path, monkeypatch):
    d = _fake_pmc(tmp_path, "routed-square")
    summary = bench.summarize_counters([str(d)], "routed-square")
    bx = summary["phases"]["bx"]
    assert abs(summary["factor_fetch"] - 2.0) < 1e-12 and abs(summary["factor_write"] - 1.0) < 1e-12
    assert abs(bx["traffic_bytes_per_launch"] - 4e9) < 1.0
    assert bx["mfma_busy"] == 0.5
    assert bx["mfma_over_alg"] == 1.0
    # bench reads the committed summary only while the kernel code it was taken on is unchanged
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    with open(bench.counters_file("routed-square"), "w") as f:
        import json
        json.dump(summary, f)
    assert abs(bench.stored_traffic("routed-square", "bx") - 4e9) < 1.0
    summary["source_code_sha256"]["ns_kernels.hip"] = "0" * 64
    with open(bench.counters_file("routed-square"), "w") as f:
        json.dump(summary, f)
    assert bench.stored_traffic("routed-square", "bx") is None
    assert bench.stored_traffic("many-small", "bx") is None


def test_trace_summary_table(tmp_path):
    import csv
    d = tmp_path / "trace"
    d.mkdir()
    bx = "_ZN3nsq12_GLOBAL__N_117ns_product_kernelIDF16bNS0_7TileCfgILi256ELi2ELi4ELi128ELi2EEELi2ELb0EDF16bEEv"
    sx = bx.replace("ELi2ELb0E", "ELi0ELb0E")
    with open(d / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        w.writerow([bx, 4, 4 * 40000, 40000, 80, 39000, 41000, 1])
        w.writerow([sx, 5, 5 * 8000, 8000, 20, 7000, 9000, 1])
    table = bench.summarize_trace(str(d), "routed-square", 1)
    lines = table.splitlines()
    assert "X' = B' X" in lines[2] and "| 4 | 40.00 |" in lines[2] and "80.0 %" in lines[2]
    # 16 x 2 x 1024^3 flops in 40 us
    assert f"{16 * 2 * 1024 ** 3 / 40e-6 / 1e12:.1f}" in lines[2]


def test_cpu_baseline_sample_is_bounded_and_extrapolated():
    from workloads import dense_transformer
    ms = dense_transformer(layers=2, hidden=64, ffn=96)
    ms.split_rows = [[s[0] // 2, s[0] - s[0] // 2] for s in ms.shapes]
    ms.num_shards = 2
    r = bench.cpu_baseline(ms, 0.05)
    assert r["kind"] == "oracle" and r["unit"] == "matrices/s" and r["cores"] >= 1
    assert r["extrapolated"] and r["value"] > 0
    assert r["sample"].startswith("4 matrices (4 frequent shapes")


def test_tiling_traffic_model_hand_values():
    """The once-per-group panel model on the 16 x 1024^2 set: per matrix one
    4 x 4 group reads 4 + 4 panels of 256 rows x 1024 (bf16) and writes 16
    tiles of 256^2 (no X'^T at m = 1024); the last launch writes the output."""
    import bench
    from workloads import routed_square_batch, many_small
    ms = routed_square_batch(True)
    per_reads = 8 * 256 * 1024 * 2
    assert bench.tiling_traffic(ms, "bx") == 16 * (per_reads + 16 * 256 * 256 * 2)
    assert bench.tiling_traffic(ms, "bx_final") == 16 * (per_reads + 1024 * 1024 * 2)
    assert bench.tiling_traffic(ms, "syrk_x") is None
    assert bench.tiling_traffic(many_small(), "bx") is None      # small size class present

"""bench.py --summarize: rocprofv3 CSV outputs (here synthetic, in the layout rocprofv3
writes) become a profile summary and a traffic record with the copy calibration
applied (FETCH_SIZE scaled by what the 512 MiB copy reads, WRITE_SIZE likewise)."""
import csv
import json
import os

import bench

NAME = "void arrms::(anonymous namespace)::row_kernel<4, 1>(arrms::RowArgs<4>)"
COPY = "__amd_rocclr_copyBuffer"


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_summary_from_synthetic_rocprof_outputs(tmp_path):
    run, out = tmp_path / "run", tmp_path / "out"
    run.mkdir()
    out.mkdir()
    T, H, W = 4096, 2048, 4
    alg = bench.algorithmic_bytes(W, T, H)
    plan = {"grid": 4096, "block": 256}
    json.dump({"config": {"plan": plan}, "roofline": {"kernel_mean_us": 20.9, "achieved": alg / 20.9e-6 / 1e9}},
              open(run / "bench.json", "w"))
    trace = [[NAME, 4096 * 256, 256, 0, 20000 + i] for i in range(5)] + [[COPY, 131072, 512, 0, 200000]] * 3
    _write_csv(str(run / "prof_bench" / "bench_kernel_trace.csv"),
               ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"], trace)
    copy_kib = 512 * 1024
    fetch = [[NAME, 4096 * 256, (2 * T * H * (W + 1) + 2 * H) / 2 / 1024]] * 4 + [[COPY, 131072, copy_kib / 2]]
    write = [[NAME, 4096 * 256, 2 * T * H * 2 / 1024]] * 4 + [[COPY, 131072, copy_kib]]
    _write_csv(str(run / "pmc_fetch" / "fetch_counter_collection.csv"), ["Kernel_Name", "Grid_Size", "Counter_Value"],
               fetch)
    _write_csv(str(run / "pmc_write" / "write_counter_collection.csv"), ["Kernel_Name", "Grid_Size", "Counter_Value"],
               write)
    bench.summarize_profiles(str(run), "prefill", out_dir=str(out))
    rec = json.load(open(out / "traffic_prefill_w4_h2048_t4096.json"))
    assert rec["kernel"] == "row_kernel<4, 1>"
    assert abs(rec["copy_calibration"]["fetch_scale"] - 2.0) < 1e-9 and abs(rec["copy_calibration"]["write_scale"] - 1) < 1e-9
    assert abs(rec["traffic_over_algorithmic"] - 1.0) < 1e-9
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_hash()
    md = open(out / "row_kernel_prefill_w4_h2048_t4096.md").read()
    assert "| row_kernel<4, 1> | 1048576 | 256 | 5 | 20.00 |" in md and "Total traffic / algorithmic bytes = 1.0000" in md

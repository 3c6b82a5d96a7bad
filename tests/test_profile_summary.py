"""bench.py --summarize: rocprofv3 CSV outputs (here synthetic, in the layout rocprofv3
writes) become a profile summary and a traffic record.  DRAM bytes come from the gfx950
counters that count DRAM reads and writes in 32-byte units, with no calibration factor;
request-size counters, the raw terms of the derived FETCH_SIZE and the stall counters
are carried alongside."""
import csv
import json
import os

import pytest

import bench

NAME = "void arrms::(anonymous namespace)::row_kernel<4, 1>(arrms::RowArgs<4>)"
FLAT = ("void arrms::(anonymous namespace)::row_kernel_flat<4, 1, false>(int, int, unsigned int, float, void const*, "
        "void const*, void const*, void const*, void const*, void const*, void const*, void const*, void const*, "
        "void const*, void*, void*)")
COPY = "__amd_rocclr_copyBuffer"


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _counters(run, name, values, dispatches=4, grid=4096 * 256, kernel=NAME):
    rows = [[kernel, grid, c, v] for _ in range(dispatches) for c, v in values.items()]
    rows += [[COPY, 131072, c, 1.0] for c in values]   # another kernel: ignored
    _write_csv(str(run / ("pmc_" + name) / (name + "_counter_collection.csv")),
               ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"], rows)


# the headline kernel taking one argument block, and its twin with preloaded arguments
@pytest.mark.parametrize("full,short", [(NAME, "row_kernel<4, 1>"), (FLAT, "row_kernel_flat<4, 1, false>")])
def test_summary_from_synthetic_rocprof_outputs(tmp_path, full, short):
    run, out = tmp_path / "run", tmp_path / "out"
    run.mkdir()
    out.mkdir()
    T, H, W = 4096, 2048, 4
    alg = bench.algorithmic_bytes(W, T, H)
    rd, wr = 2 * T * H * (W + 1) + 2 * H, 2 * T * H * 2
    plan = {"grid": 4096, "block": 256}
    json.dump({"config": {"plan": plan}, "roofline": {"kernel_mean_us": 20.9, "achieved": alg / 20.9e-6 / 1e9}},
              open(run / "bench.json", "w"))
    trace = [[full, 4096 * 256, 256, 0, 20000 + i] for i in range(5)] + [[COPY, 131072, 512, 0, 200000]] * 3
    _write_csv(str(run / "prof_bench" / "bench_kernel_trace.csv"),
               ["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"], trace)
    n128 = rd / 128
    _counters(run, "dram", {"TCC_EA0_RDREQ_DRAM_32B_sum": rd / 32, "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum": wr / 32,
                            "TCC_EA0_RDREQ_sum": n128, "TCC_BUBBLE_sum": 0.0}, kernel=full)
    _counters(run, "size", {"TCC_EA0_RDREQ_32B_sum": 0.0, "TCC_EA0_RDREQ_64B_sum": 0.0, "TCC_EA0_RDREQ_128B_sum": n128,
                            "TCC_EA0_WRREQ_64B_sum": wr / 64}, kernel=full)
    _counters(run, "stall", {"TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum": 500.0, "TCC_EA0_WRREQ_DRAM_CREDIT_STALL_sum": 100.0,
                             "TCC_BUSY_sum": 10000.0, "TCC_EA0_RDREQ_LEVEL_sum": n128 * 800}, kernel=full)
    _counters(run, "fetch", {"FETCH_SIZE": n128 * 64 / 1024}, kernel=full)
    _counters(run, "write", {"WRITE_SIZE": wr / 1024}, kernel=full)
    bench.summarize_profiles(str(run), "prefill", out_dir=str(out))
    rec = json.load(open(out / "traffic_prefill_w4_h2048_t4096.json"))
    assert rec["kernel"] == short and rec["plan"] == plan
    assert rec["read_bytes_per_launch"] == rd and rec["write_bytes_per_launch"] == wr
    assert abs(rec["traffic_over_algorithmic"] - 1.0) < 1e-12
    assert rec["read_bytes_by_request_size"] == rd
    # with no 128-byte requests counted by TCC_BUBBLE, the derived formula sees half the reads
    assert rec["fetch_size_formula_bytes"] == rd / 2
    assert abs(rec["stalls"]["read_dram_credit_stall_pct_of_busy"] - 5.0) < 1e-12
    assert abs(rec["stalls"]["mean_read_latency_cycles"] - 800.0) < 1e-9
    assert rec["dispatches"]["TCC_BUSY_sum"] == 4
    assert rec["kernel_source_sha256_16"] == bench.kernel_source_hash()
    assert any("--pmc TCC_EA0_RDREQ_DRAM_32B_sum" in c for c in rec["commands"])
    md = open(out / ("%s_prefill_w4_h2048_t4096.md" % short.split("<")[0])).read()
    assert "| %s | 1048576 | 256 | 5 | 20.00 |" % short in md
    assert "| total / algorithmic | 1.0000 | 1 |" in md and "credits" in md

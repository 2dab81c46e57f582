"""The bench's FLOP/byte accounting against the figures the pages print.

The first TileLang page works the 4096-cube fp16 product through (about 137
billion flops, 32 MB per matrix, 96 MB ideal traffic, about 275 GB for a naive
one-output-at-a-time kernel); the second prices the example tile (16 KB of
shared memory per stage, 48 KB for 3 stages, a 64 KB accumulator = 128
registers per thread at 128 threads).  The same functions must also show that
this build's own tile fits CDNA4's 160 KB LDS and 256 accumulator registers.
"""
import json
import os

import bench

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_example.json")


def golden():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_worked_example_flops_and_bytes():
    g = golden()["gemm_4096_fp16"]
    M, N, K, b = g["M"], g["N"], g["K"], g["bytes_per_element"]
    flops = bench.gemm_flops(M, N, K)
    assert flops == 2 * 4096 ** 3
    assert abs(flops - g["flops_approx"]) <= g["flops_rel_tol"] * g["flops_approx"]
    assert M * K * b == g["matrix_bytes_approx_MiB"] * 2 ** 20
    assert bench.gemm_alg_bytes(M, N, K, elt=b) == g["ideal_traffic_approx_MiB"] * 2 ** 20
    naive = bench.naive_input_bytes(M, N, K, elt=b)
    assert abs(naive - g["naive_input_traffic_approx_GB"] * 1e9) <= g["naive_rel_tol"] * naive


def test_tile_cost_of_the_pages_example():
    g = golden()["tile_cost_128x128x32"]
    bm, bn, bk, st, thr, b = (g[k] for k in ("block_M", "block_N", "block_K", "num_stages", "threads",
                                             "bytes_per_element"))
    assert bench.staged_tile_bytes(bm, bn, bk, 1, b) == g["stage_KiB"] * 1024
    assert bench.staged_tile_bytes(bm, bn, bk, st, b) == g["total_KiB"] * 1024
    assert bm * bn * 4 == g["accumulator_KiB"] * 1024
    assert bench.accumulator_regs_per_thread(bm, bn, thr) == g["accumulator_regs_per_thread"]


def test_this_builds_tiles_fit_cdna4():
    # vector kernel: 4 stages of 256 x 256 x 32; generic kernel: 2 stages of 256 x 256 x 64
    assert bench.staged_tile_bytes(256, 256, 32, 4) == 128 * 1024 <= 160 * 1024
    assert bench.staged_tile_bytes(256, 256, 64, 2) == 128 * 1024 <= 160 * 1024
    # 256 x 256 fp32 accumulators over 256 threads: 256 registers each, the AGPR file of one wave
    assert bench.accumulator_regs_per_thread(256, 256, 256) == 256


def test_workload_accounting_matches_the_stated_figures():
    assert bench.gemm_flops(8192, 8192, 8192) == 1_099_511_627_776
    assert bench.gemm_alg_bytes(8192, 8192, 8192, bias=True) == 402_669_568
    assert bench.gemm_alg_bytes(16, 11008, 4096) == 90_660_864


def test_counter_hash_covers_every_kernel_source():
    # The measured HBM traffic, MFMA utilisation and clock in
    # profiles/counters.json are reported only while the hash of the kernel
    # sources matches; every file the library is built from must be part of
    # that hash, or a change to it would leave stale figures in the bench line.
    csrc = os.path.join(os.path.dirname(bench.__file__), "tiled_dense_gemm_tg_amd", "csrc")
    sources = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h", ".inc")))
    assert sorted(bench.KERNEL_SOURCES) == sources


def test_stale_counters_are_not_reported(tmp_path, monkeypatch):
    # A counter record taken on other kernel sources gives None, a current
    # one its figures.
    path = tmp_path / "counters.json"
    rec = {"lines": {"w": {"kernel_hash": bench.kernel_source_hash(), "bytes_per_launch": 123, "mfma_util": 0.5},
                     "old": {"kernel_hash": "0" * 16, "bytes_per_launch": 456}}}
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(path))
    assert bench.measured_traffic("w") == 123
    assert bench.measured("w")["mfma_util"] == 0.5
    assert bench.measured_traffic("old") is None
    assert bench.measured_traffic("missing") is None


def test_dispatch_log_labels_the_unfused_passes(tmp_path):
    # The summariser pairs the library's dispatches of a rocprofv3 run with
    # the bench's dispatch log, position by position, and names the three
    # launches of an unfused call after their roles.
    run = tmp_path / "run"
    run.mkdir()
    log = bench.DispatchLog()
    log.note("main", 2)
    log.note("main unfused_gelu unfused", 6)
    log.note("main")
    (run / "dispatch_log.json").write_text(json.dumps({"entries": log.entries}))
    hdr = "Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp\n"
    rows = [f"{i + 1},tg::k{i},{1000 * i},{1000 * i + 500}" for i in range(9)]
    rows.insert(3, "99,torch_kernel,0,1")   # not a library kernel: skipped
    (run / "run_kernel_trace.csv").write_text(hdr + "\n".join(rows) + "\n")
    got = bench._dispatches(str(run), "*kernel_trace.csv", False)
    labels = [lab for lab, _ in got]
    assert labels == ["main", "main",
                      "main unfused_gelu unfused product", "main unfused_gelu unfused bias pass",
                      "main unfused_gelu unfused GELU pass"] * 1 + [
                      "main unfused_gelu unfused product", "main unfused_gelu unfused bias pass",
                      "main unfused_gelu unfused GELU pass", "main"]
    assert all(rec["dur_us"] == 0.5 for _, rec in got)


def test_counter_means_per_bench_line(tmp_path):
    # --counter-means averages every counter of a --pmc run over the
    # dispatches of each bench line (rows of one dispatch and counter are
    # summed first, as rocprofv3 splits some counters over dimensions).
    run = tmp_path / "run"
    run.mkdir()
    log = bench.DispatchLog()
    log.note("a", 2)
    log.note("b", 1)
    (run / "dispatch_log.json").write_text(json.dumps({"entries": log.entries}))
    hdr = "Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp,Counter_Name,Counter_Value\n"
    rows = ["1,tg::k,0,2000,X,10", "1,tg::k,0,2000,X,5", "1,tg::k,0,2000,Y,1",
            "2,tg::k,0,4000,X,30", "2,tg::k,0,4000,Y,3",
            "7,other_kernel,0,1,X,1000",
            "3,tg::k,0,1000,X,7", "3,tg::k,0,1000,Y,0"]
    (run / "run_counter_collection.csv").write_text(hdr + "\n".join(rows) + "\n")
    got = bench.counter_means(str(run))
    assert got == {"a": {"dispatches": 2, "dur_us": 3.0, "X": 22.5, "Y": 2.0},
                   "b": {"dispatches": 1, "dur_us": 1.0, "X": 7.0, "Y": 0.0}}

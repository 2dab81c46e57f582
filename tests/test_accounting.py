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


def test_traffic_hash_covers_every_kernel_source():
    # The measured HBM traffic in profiles/traffic.json is reported only while
    # the hash of the kernel sources matches; every file the library is built
    # from must be part of that hash, or a change to it would leave stale
    # figures in the bench line.
    csrc = os.path.join(os.path.dirname(bench.__file__), "tiled_dense_gemm_tg_amd", "csrc")
    sources = sorted(f for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    assert sorted(bench.KERNEL_SOURCES) == sources


def test_committed_traffic_matches_the_kernel_sources():
    # Every workload in the committed traffic file was measured on the
    # current sources (re-profile after any kernel change).
    with open(bench.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    h = bench.kernel_source_hash()
    stale = [k for k, v in rec.items() if isinstance(v, dict) and v.get("kernel_hash") != h]
    assert not stale, stale

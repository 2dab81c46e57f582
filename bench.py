#!/usr/bin/env python3
"""Throughput of the tiled half-precision GEMM on one MI355X; prints ONE JSON line.

A step is one call of tg_gemm over the 8192-cube fp16 workload with the fused
bias + GELU(tanh) epilogue (inputs resident in HBM), which runs every stage of
the tiled path: tile raster, global->LDS staging, swizzled LDS, the
double-buffered k-loop, MFMA accumulation, the fused epilogue and the store.
The 4096-cube (MFMA-bound, no epilogue) and the M=16 decode shape (HBM-bound,
the skinny kernel), the weight-only 4-bit product at that decode shape and the
attention forward at the FlashAttention benchmark shape are timed as secondary
lines in the same JSON object.

Timing: W warm-up launches, then further untimed launches until a quarter of
a second has passed (the clock takes a few tens of milliseconds to settle
after a change of load), then K launches back to back on torch's current
stream (the stream tg_gemm is given), bracketed by torch.cuda.synchronize()
and HIP events recorded on that stream; the per-launch time is the events'
elapsed time / K.  Every secondary line settles the same way before it is
timed.  The fused and unfused forms of an epilogue workload (and the product
without epilogue) are timed in alternating blocks and compared by their
medians.  The skinny shape rotates over 8 independent operand sets (720 MB,
more than the 256 MB Infinity Cache) so every launch streams B from HBM.

Roofline: FLOPs = 2*M*N*K (padded-tile work and the epilogue's few flops per
output are not counted); algorithmic bytes = every operand once + C once (+
bias).  Peaks are MI355X's published dense fp16/bf16 MFMA rate (2.5 PFLOP/s)
and HBM3E bandwidth (8 TB/s).  HBM traffic, MFMA utilisation and the shader
clock come from rocprofv3 counter runs of this same script, summarised into
profiles/counters.json by `bench.py --summarise` (reported only while the
kernel sources are the ones profiled).  The CPU baseline is the oracle (test
infrastructure, untuned) timed on a bounded sample of rows of the same
workload on the host cores.

Profiling: `--dispatch-log FILE` records, in launch order, a label for every
kernel this script launches through the library; `--profile-run` drops the
settling and shortens every line (for counter runs, which serialise
dispatches).  `--summarise DIR` reads the rocprofv3 CSV output of the runs
that PROFILE_COMMANDS lists, together with their dispatch logs, and writes
the summaries under profiles/.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_MFMA_F16_TFLOPS = 2500.0   # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
MFMA_FLOP_PER_CLK_SIMD = 1024   # dense fp16/bf16 MFMA: 2.5 PFLOP/s = 1024 SIMDs x 1024 x 2.4 GHz
METRIC = "GEMM TFLOP/s and % MFMA peak at 4096³/8192³ fp16; HBM GB/s at M=16"
MAIN = "gemm_f16_8192x8192x8192_bias_gelu_tanh"
SQUARE = "gemm_f16_4096x4096x4096"
SKINNY = "gemm_f16_skinny_16x11008x4096"
RAGGED = "gemm_bf16_4000x4093x4111_bias_gelu_tanh"
KERNEL_SOURCES = ["gemm_tiled.hip", "gemm_tiled_generic.hip", "gemm_skinny.hip", "gemm_w4.hip", "attention_fwd.hip",
                  "elementwise.hip", "tg_device.h", "tg_tile.h", "tg_launch.h", "tg_split.h", "tg_direct.h",
                  "tg_gemm_host.hip", "tg_tile_model.inc"]
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters.json")
SETTLE_S = 0.25   # untimed launches before every timed line, in seconds of wall time
FUSION_ROUNDS = 4  # alternating blocks of fused / unfused / no-epilogue launches


# ---------------------------------------------------------------- accounting

# Elementwise passes the unfused form adds after the product, each reading
# and writing M x N 16-bit values (4 bytes per element).
EPILOGUE_PASSES = {0: 0, 1: 1, 2: 2}


def gemm_flops(M: int, N: int, K: int) -> int:
    """Multiply-adds counted as two flops: 2*M*N*K."""
    return 2 * M * N * K


def gemm_alg_bytes(M: int, N: int, K: int, elt: int = 2, bias: bool = False) -> int:
    """Each operand read once, C written once (the ideal of perfect on-chip reuse)."""
    return elt * (M * K + K * N + M * N + (N if bias else 0))


def naive_input_bytes(M: int, N: int, K: int, elt: int = 2) -> int:
    """Inputs read by a one-output-at-a-time kernel: K values of A and K of B per output."""
    return M * N * 2 * K * elt


def staged_tile_bytes(bm: int, bn: int, bk: int, stages: int, elt: int = 2) -> int:
    """On-chip staging of one A tile and one B tile per pipeline stage."""
    return stages * (bm * bk + bk * bn) * elt


def accumulator_regs_per_thread(bm: int, bn: int, threads: int, acc_bytes: int = 4) -> int:
    """32-bit registers per thread holding a bm x bn accumulator."""
    return bm * bn * acc_bytes // 4 // threads


def attention_flops(B: int, H: int, D: int, Sq: int, Sk: int, causal: bool) -> int:
    """Two products of 2*D flops per visible (query, key) pair: 4*B*H*D*pairs;
    with the causal mask (Sq == Sk) a query i sees keys 0..i."""
    pairs = Sq * (Sq + 1) // 2 if causal else Sq * Sk
    return 4 * B * H * D * pairs


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and runs of white space
    removed: a change of comments alone leaves the compiled kernels, and so
    the counters taken on them, as they were."""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tiled_dense_gemm_tg_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured(label: str):
    """The committed counter record of one bench line (HBM traffic, MFMA
    utilisation, shader clock), if it was taken on the current kernel
    sources; else None."""
    try:
        with open(COUNTERS_FILE) as fh:
            rec = json.load(fh).get("lines", {}).get(label)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_hash") != kernel_source_hash():
        return None
    return rec


def measured_traffic(label: str):
    """HBM bytes per launch (fetched + written past L2) of one bench line."""
    rec = measured(label)
    return rec.get("bytes_per_launch") if rec else None


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class DispatchLog:
    """A label for every kernel the bench launches through the library, in
    launch order, run-length encoded as [label, kernels]; written with
    --dispatch-log so that the profile summariser can tell which dispatch of
    a rocprofv3 run belongs to which bench line."""

    def __init__(self):
        self.entries = []

    def note(self, label: str, kernels: int = 1) -> None:
        if self.entries and self.entries[-1][0] == label:
            self.entries[-1][1] += kernels
        else:
            self.entries.append([label, kernels])

    def expand(self):
        return [lab for lab, n in self.entries for _ in range(n)]


LOG = DispatchLog()
UNFUSED_PARTS = {1: ["product", "bias pass"], 2: ["product", "bias pass", "GELU pass"]}


# ---------------------------------------------------------------- timing

class Timing:
    """How lines are timed: settle seconds before each timed line, and a
    divisor for the step counts (profile runs shorten everything)."""
    settle_s = SETTLE_S
    short = False


def steps_for(n: int) -> int:
    return max(2, n // 10) if Timing.short else n


def time_calls(torch, launch, steps, warmup, with_wall=False, settle_s=None):
    """Per-launch time (ms) of launch(i) for i = 0 .. steps-1 on the current
    stream: HIP events recorded on that stream around the timed launches,
    after `warmup` untimed ones, then further untimed ones until `settle_s`
    seconds have passed (the clock takes a few tens of milliseconds to settle
    after a change of load: the first ~15 ms of a 150-us kernel ran 10 %
    slower), and a synchronisation; with `with_wall`, also the host's wall
    time (s) from before the first timed launch to after the closing
    synchronisation."""
    if settle_s is None:
        settle_s = Timing.settle_s
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    if settle_s > 0:
        t_end = time.perf_counter() + settle_s
        i = warmup
        while time.perf_counter() < t_end:
            for _ in range(20):
                launch(i)
                i += 1
            torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        launch(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / steps
    return (ms, wall) if with_wall else ms


def gemm_launcher(torch, tg, w, sets, label, mode="fused", ws=None, splits=0):
    """launch(i) for tg_gemm over `sets` rotating operand sets; mode
    "unfused" runs tg_gemm_unfused (product, then one pass per epilogue
    step), "none" the product without epilogue, "split" tg_gemm_split with
    `splits` and the workspace `ws` (allocated and zeroed before the timed
    region, as a caller holds one per stream)."""
    handle = torch.cuda.current_stream().cuda_stream
    calls = [(A.data_ptr(), B.data_ptr(), bias.data_ptr() if bias is not None else None, C.data_ptr())
             for A, B, bias, C in sets]
    nk = 1 + (EPILOGUE_PASSES[w.epilogue] if mode == "unfused" else 0)
    wsp, wsn = (ws.data_ptr(), ws.numel()) if ws is not None else (None, 0)

    def launch(i):
        a, b, bi, c = calls[i % len(calls)]
        LOG.note(label, nk)
        if mode == "split":
            st = tg.tg_gemm_split(splits, w.M, w.N, w.K, w.dtype, a, b, bi, w.epilogue, c, wsp, wsn, handle)
        elif mode == "unfused":
            st = tg.tg_gemm_unfused(w.M, w.N, w.K, w.dtype, a, b, bi, w.epilogue, c, handle)
        elif mode == "none":
            st = tg.tg_gemm(w.M, w.N, w.K, w.dtype, a, b, None, 0, c, handle)
        else:
            st = tg.tg_gemm(w.M, w.N, w.K, w.dtype, a, b, bi, w.epilogue, c, handle)
        if st != tg.TG_OK:
            raise RuntimeError(f"tg_gemm failed: {tg.tg_status_string(st)}")

    return launch


def time_gemm(torch, tg, w, sets, steps, warmup, label=None, mode="fused", settle_s=None, ws=None, splits=0):
    """Per-launch time (ms) and wall time (s) of one gemm line."""
    launch = gemm_launcher(torch, tg, w, sets, label or w.name, mode, ws, splits)
    return time_calls(torch, launch, steps, warmup, with_wall=True, settle_s=settle_s)


def fusion_comparison(torch, tg, w, sets, steps, warmup):
    """The fused epilogue against the unfused form (product, then a pass per
    epilogue step) and against the product alone, timed in alternating
    blocks under the same conditions: one settle before the first block,
    then FUSION_ROUNDS rounds of one block of each form, the order reversed
    every round; each form's time is the median over its blocks."""
    modes = ["fused", "unfused", "none"]
    labels = {"fused": w.name, "unfused": f"{w.name} unfused", "none": f"{w.name} no epilogue"}
    launch = {m: gemm_launcher(torch, tg, w, sets, labels[m], m) for m in modes}
    time_calls(torch, launch["fused"], 1, warmup)   # settle
    times = {m: [] for m in modes}
    for r in range(FUSION_ROUNDS):
        for m in (modes if r % 2 == 0 else modes[::-1]):
            times[m].append(time_calls(torch, launch[m], steps, 2, settle_s=0.0))
    med = {m: sorted(v)[len(v) // 2] for m, v in times.items()}
    return {"fused_us": round(med["fused"] * 1e3, 2), "unfused_us": round(med["unfused"] * 1e3, 2),
            "no_epilogue_us": round(med["none"] * 1e3, 2),
            "fusion_speedup": round(med["unfused"] / med["fused"], 3),
            "epilogue_cost": round(med["fused"] / med["none"] - 1.0, 4),
            "blocks": FUSION_ROUNDS, "launches_per_block": steps,
            "unfused_extra_bytes": EPILOGUE_PASSES[w.epilogue] * 4 * w.M * w.N}


def bench_w4(torch, tg, I, steps, warmup, copies=16):
    """The weight-only 4-bit product at the decode shape, with `copies`
    rotating weight sets (more bytes than the 256 MB MALL) so the packed
    weights stream from HBM, and with one set (cache-resident)."""
    wq = I.W4_WORKLOAD
    M, N, K, G, dt = wq["M"], wq["N"], wq["K"], wq["group"], wq["dtype"]
    tdt = torch.float16 if dt == I.F16 else torch.bfloat16
    sa, sq, ss = wq["seeds"]

    def dev(bits, shape):
        return torch.from_numpy(bits.view(np.int16).reshape(shape).copy()).view(tdt).cuda()

    A = dev(I.random_bits((M, K), wq["a_dist"], dt, sa), (M, K))
    sets = []
    for c in range(copies):
        q = torch.from_numpy(I.w4_weights(K, N, sq + 10 * c)).cuda()
        LOG.note("w4 weight packing")
        packed = tg.w4_pack(q)
        del q
        S = dev(I.random_bits((K // G, N), wq["scale_dist"], dt, ss + 10 * c), (K // G, N))
        C = torch.empty((M, N), dtype=tdt, device="cuda")
        sets.append((packed, S, C))
    handle = torch.cuda.current_stream().cuda_stream

    def launch(i, pool=sets, label=wq["name"]):
        packed, S, C = pool[i % len(pool)]
        LOG.note(label)
        st = tg.tg_gemm_w4(M, N, K, dt, A.data_ptr(), packed.data_ptr(), S.data_ptr(), G, None, I.EPI_NONE,
                           C.data_ptr(), handle)
        if st != tg.TG_OK:
            raise RuntimeError(f"tg_gemm_w4 failed: {tg.tg_status_string(st)}")

    ms = time_calls(torch, launch, steps, warmup)
    hot = time_calls(torch, lambda i: launch(i, sets[:1], f"{wq['name']} hot"), steps, warmup)
    nbytes = tg.tg_w4_packed_bytes(K, N) + 2 * (K // G) * N + 2 * M * K + 2 * M * N
    return wq["name"], ms, hot, nbytes


def tile_configs(tg):
    """Every tile configuration of the tiled family: name -> tg_tiles value."""
    return {tg.TILES_NAMES[c]: c for c in sorted(tg.TILES_AXES)}


def time_alternating(torch, launches, steps, rounds=3, settle_s=None):
    """Median per-launch time (ms) of each launch(i) in `launches` (name ->
    fn), timed in `rounds` rounds of one block each, the order reversed every
    round, after one settle: so that forms compared with each other see the
    same clock."""
    names = list(launches)
    time_calls(torch, launches[names[0]], 1, 2, settle_s=settle_s)
    times = {n: [] for n in names}
    for r in range(rounds):
        for n in (names if r % 2 == 0 else names[::-1]):
            times[n].append(time_calls(torch, launches[n], steps, 1, settle_s=0.0))
    return {n: sorted(v)[len(v) // 2] for n, v in times.items()}


def tiled_launcher(torch, tg, M, N, K, dtype, epi, A, B, bias, C, cfg, label, group_m=0):
    """launch(i) of tg_gemm_tiled_grouped with configuration cfg (0: the
    library's choice, through tg_gemm)."""
    handle = torch.cuda.current_stream().cuda_stream
    a, b, bi, c = A.data_ptr(), B.data_ptr(), bias.data_ptr() if bias is not None else None, C.data_ptr()

    def launch(i):
        LOG.note(label)
        st = (tg.tg_gemm_tiled_grouped(cfg, group_m, M, N, K, dtype, a, b, bi, epi, c, handle) if cfg or group_m
              else tg.tg_gemm(M, N, K, dtype, a, b, bi, epi, c, handle))
        if st != tg.TG_OK:
            raise RuntimeError(f"tg_gemm_tiled_grouped failed: {tg.tg_status_string(st)}")

    return launch


def axes_of(tg, cfg):
    """The tuning axes of a tile configuration, with the raster group the
    library uses unless a call picks another (tg_gemm_tiled_grouped)."""
    if cfg not in tg.TILES_AXES:
        return None
    bm, bn, bk, stages, waves = tg.TILES_AXES[cfg]
    return {"BM": bm, "BN": bn, "BK": bk, "stages": stages, "waves": waves, "group_m": 4}


def bench_tile_choice(torch, tg, I, steps, warmup):
    """Every tile configuration, and the library's own choice, on the shape
    classes the choice is for, timed in alternating blocks."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    configs = tile_configs(tg)
    out = {}
    for name, w in I.TILE_WORKLOADS.items():
        _, sets = device_operands(torch, I, w)
        A, B, bias, C = sets[0]
        flops = gemm_flops(w.M, w.N, w.K)
        launches = {cname: tiled_launcher(torch, tg, w.M, w.N, w.K, w.dtype, w.epilogue, A, B, bias, C, cfg,
                                          f"{name} {cname}") for cname, cfg in configs.items()}
        launches["auto"] = tiled_launcher(torch, tg, w.M, w.N, w.K, w.dtype, w.epilogue, A, B, bias, C, 0,
                                          f"{name} auto")
        per = time_alternating(torch, launches, steps)
        ms_auto = per.pop("auto")
        st, auto = tg.tg_gemm_tiles_plan(w.M, w.N, w.K, cus)
        best = min(per, key=per.get)
        out[name] = {"auto": tg.TILES_NAMES.get(auto, "?"), "auto_axes": axes_of(tg, auto),
                     "auto_us": round(ms_auto * 1e3, 2),
                     "auto_TFLOP/s": round(flops / (ms_auto * 1e-3) / 1e12, 1),
                     "per_config_us": {k: round(v * 1e3, 2) for k, v in per.items()},
                     "fastest": best, "fastest_axes": axes_of(tg, configs[best]),
                     "auto_vs_fastest": round(per[best] / ms_auto, 3),
                     "speedup_vs_256x256": round(per["256x256"] / ms_auto, 3),
                     "traffic": measured_traffic(f"{name} auto")}
        log(f"{name}: auto {tg.TILES_NAMES.get(auto)} {ms_auto * 1e3:.1f} us, fastest {best} "
            f"{per[best] * 1e3:.1f} us, 256x256 {per['256x256'] * 1e3:.1f} us")
        del sets, A, B, bias, C, launches
        torch.cuda.empty_cache()
    return out


def fit_tile_model(meas, cus):
    """The tile-choice cost model's parameters from the sweep's timings (us):
    per configuration, a1 + b1 K for a round of one tile per CU on every CU
    (two points in K), a2 + b2 K for a round of two per CU (two workgroups per
    CU only), kappa (a round on a fraction u of the CUs takes 1 - kappa (1 - u)
    of the full-load time: less contention; measured at u = 1/4, and u below
    that is priced as 1/4), phi (rounds after the first:
    the 8192-cube's time over its rounds' prediction) and rho (misaligned
    shapes, K and N not multiples of 8: time over the aligned time)."""
    out = {}
    for name, m in meas.items():
        k1, k2 = m["k"]
        b1 = (m["solo"][1] - m["solo"][0]) / (k2 - k1)
        a1 = m["solo"][0] - b1 * k1
        rec = {"a1": a1, "b1": b1}
        if "pair" in m:
            b2 = (m["pair"][1] - m["pair"][0]) / (k2 - k1)
            rec.update(a2=m["pair"][0] - b2 * k1, b2=b2)
        rec["kappa"] = max(0.0, min(0.9, (1.0 - m["quarter"] / (a1 + b1 * k2)) / 0.75))
        pred = predict_tile_time(dict(rec, phi=1.0, rho=1.0, bm=m["bm"], bn=m["bn"], occ=m["occ"]),
                                 *m["full_shape"], cus, True)
        rec["phi"] = m["full"] / pred
        rec["rho"] = m["ragged"] / m["solo"][1]
        out[name] = {k: round(v, 6) for k, v in rec.items()}
    return out


def predict_tile_time(p, M, N, K, cus, aligned):
    """The cost model (mirrors the library's auto_tiles): the sum over the
    rounds of the persistent grid of each round's time."""
    tiles = -(-M // p["bm"]) * -(-N // p["bn"])
    per_round = cus * p["occ"]
    t, left, rounds = 0.0, tiles, 0
    while left > 0:
        busy = min(left, per_round)
        if busy > cus:    # some CUs hold two workgroups
            t += p["a2"] + p["b2"] * K
        else:
            t += (p["a1"] + p["b1"] * K) * (1.0 - p["kappa"] * (1.0 - max(busy / cus, 0.25)))
        left -= busy
        rounds += 1
    if rounds > 1:
        t *= p["phi"]
    return t if aligned else t * p["rho"]


TILE_MODEL_INC = os.path.join(ROOT, "tiled_dense_gemm_tg_amd", "csrc", "tg_tile_model.inc")


# The rows of the model table in the library's order (the default first).
TILE_ENUM = {"256x256": "TG_TILES_256x256", "256x128": "TG_TILES_256x128", "128x256": "TG_TILES_128x256",
             "128x128": "TG_TILES_128x128", "256x256_k64": "TG_TILES_256x256_K64",
             "256x128_k64": "TG_TILES_256x128_K64", "128x256_k64": "TG_TILES_128x256_K64",
             "128x128_k64": "TG_TILES_128x128_K64", "256x256_w8": "TG_TILES_256x256_W8"}
TILE_SWEEP_MD = os.path.join(ROOT, "profiles", "tile_sweep.md")


def _tile_row(name, p):
    bm, bn = (int(v) for v in name.split("_")[0].split("x"))
    occ = 2 if (bm, bn) == (128, 128) else 1
    return dict(p, bm=bm, bn=bn, occ=occ, a2=p.get("a2", 0.0), b2=p.get("b2", 0.0))


def model_choice(model, M, N, K, cus, aligned=True):
    """The configuration the library's auto_tiles picks with these model
    parameters: rows in table order, a row taking over only when its
    prediction is below 0.98 of the best so far."""
    pick, best = None, None
    for name in TILE_ENUM:
        t = predict_tile_time(_tile_row(name, model[name]), M, N, K, cus, aligned)
        if best is None or t < best * 0.98:
            pick, best = name, t
    return pick


def write_tile_model(sweep: dict, path: str = TILE_MODEL_INC) -> None:
    """Writes the cost model's parameter table (the rows of kTileChoices in
    tg_gemm_host.hip) from a --sweep result; the default configuration comes
    first (ties go to earlier rows)."""
    model = sweep["tile_sweep"]["model"] if "tile_sweep" in sweep else sweep["model"]
    lines = ["// tg_tile_model.inc -- parameters of the tile-choice cost model (see auto_tiles in",
             "// tg_gemm_host.hip), written by bench.py from `python3 bench.py --sweep` on one MI355X:",
             "// {tiles, BM, BN, workgroups per CU, a1, b1, a2, b2, kappa, phi, rho}, times in us."]
    for name in TILE_ENUM:
        p = _tile_row(name, model[name])
        lines.append(f"    {{{TILE_ENUM[name]}, {p['bm']}, {p['bn']}, {p['occ']}, {p['a1']:.6g}, {p['b1']:.6g}, "
                     f"{p['a2']:.6g}, {p['b2']:.6g}, {p['kappa']:.6g}, {p['phi']:.6g}, {p['rho']:.6g}}},")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def write_sweep_summary(sweep: dict, path: str = TILE_SWEEP_MD) -> None:
    """profiles/tile_sweep.md from a --sweep result: the measured times, the
    fitted parameters, the raster-group sweep and, per shape class, the
    configuration the model fitted from this sweep picks (model_choice)
    against the fastest measured."""
    d = sweep["tile_sweep"] if "tile_sweep" in sweep else sweep
    meas, model, cus = d["measured_us"], d["model"], d["cus"]

    def f(v):
        return v if isinstance(v, str) else f"{v:.1f}"
    L = ["# Tile-configuration sweep (tiled family)", "",
         "Commands (one MI355X, committed files only; the second writes `tiled_dense_gemm_tg_amd/csrc/tg_tile_model.inc`",
         "and this file):", "",
         "```", "python3 bench.py --sweep > sweep.json", "python3 bench.py --write-tile-model sweep.json", "```", "",
         f"CUs: {cus}. fp16 operands normal(0, 0.1), no epilogue. Times in us, one block of launches each after a settle.", "",
         "| configuration (BM x BN, BK, stages, waves) | one tile per CU, K=2048 | K=8192 | two per CU, K=2048 | K=8192 "
         "| a quarter of the CUs, K=8192 | 8192-cube | ragged (K, N not multiples of 8), K=8187 |",
         "|---|---|---|---|---|---|---|---|"]
    for name, m in meas.items():
        bm, bn = (int(v) for v in name.split("_")[0].split("x"))
        bk = 64 if "k64" in name else 32
        stages = {"256x256_k64": 2, "128x128_k64": 2}.get(name, 3 if "k64" in name else 4)
        waves = 8 if name.endswith("_w8") else 4
        pair = m.get("pair", ["-", "-"])
        L.append(f"| {name} ({bm}x{bn}, {bk}, {stages}, {waves}) | {f(m['solo'][0])} | {f(m['solo'][1])} | "
                 f"{f(pair[0])} | {f(pair[1])} | {f(m['quarter'])} | {f(m['full'])} | {f(m['ragged'])} |")
    L += ["", "Fitted model parameters (`fit_tile_model` in bench.py; the table the library compiles in). A round on a "
          "fraction u of", "the CUs is priced at (1 - kappa (1 - max(u, 1/4))) of a full round: the sweep measures "
          "u = 1/4 and nothing below it.", "",
          "| configuration | a1 | b1 | a2 | b2 | kappa | phi | rho |", "|---|---|---|---|---|---|---|---|"]
    for name, p in model.items():
        L.append(f"| {name} | {p['a1']:.3f} | {p['b1']:.6f} | {p.get('a2', 0):.3f} | {p.get('b2', 0):.6f} | "
                 f"{p['kappa']:.3f} | {p['phi']:.3f} | {p['rho']:.3f} |")
    L += ["", "Raster group size (tile rows per group, `tg_gemm_tiled_grouped`), configuration the library picks:", "",
          "| shape | group_m=1 | group_m=2 | group_m=4 | group_m=8 | group_m=16 |", "|---|---|---|---|---|---|"]
    for shape, g in d["raster_groups"].items():
        L.append(f"| {shape} | " + " | ".join(f"{g[f'group_m={k}']:.1f}" for k in (1, 2, 4, 8, 16)) + " |")
    L += ["", "Shape classes, every configuration in alternating blocks (the same function as the bench line "
          "`tile_choice`); `auto` is", "the configuration the model fitted from this sweep picks (`model_choice`, "
          "the library's `auto_tiles` rule), priced at this sweep's time:", "",
          "| shape | auto | auto us | fastest | fastest us | auto / fastest |", "|---|---|---|---|---|---|"]
    for shape, c in d["shape_classes"].items():
        M, N, K = (int(x) for x in re.search(r"(\d+)x(\d+)x(\d+)", shape).groups())
        auto = model_choice(model, M, N, K, cus)
        pc = c["per_config_us"]
        fastest = min(pc, key=pc.get)
        L.append(f"| {shape} | {auto} | {pc[auto]} | {fastest} | {pc[fastest]} | {pc[auto] / pc[fastest]:.3f} |")
    with open(path, "w") as fh:
        fh.write("\n".join(L) + "\n")


def tile_sweep(torch, tg, I, steps, warmup):
    """Measures what the library's tile-choice cost model needs for every
    configuration (fit_tile_model), the raster group sizes on the large
    shapes, and the shape classes.  Operands are normal(0, 0.1) fp16 drawn on
    the device (timing only)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20001)

    def operands(M, N, K):
        A = (torch.randn((M, K), generator=gen, device="cuda") * 0.1).half()
        B = (torch.randn((K, N), generator=gen, device="cuda") * 0.1).half()
        return A, B, torch.empty((M, N), dtype=torch.float16, device="cuda")

    def one(cfg, M, N, K, label, group_m=0):
        A, B, C = operands(M, N, K)
        t = time_alternating(torch, {"x": tiled_launcher(torch, tg, M, N, K, 0, 0, A, B, None, C, cfg, label,
                                                         group_m)}, steps, rounds=1)["x"] * 1e3
        del A, B, C
        return t

    meas = {}
    ks = (2048, 8192)
    side = int(round(cus ** 0.5))
    for cname, cfg in tile_configs(tg).items():
        bm, bn, bk, stages, waves = tg.TILES_AXES[cfg]
        occ = 2 if (bm, bn) == (128, 128) else 1
        m = {"bm": bm, "bn": bn, "occ": occ, "k": ks}
        tm, tn = side, cus // side
        m["solo"] = [one(cfg, tm * bm, tn * bn, k, f"sweep {cname} solo") for k in ks]
        if occ == 2:
            m["pair"] = [one(cfg, tm * bm, 2 * tn * bn, k, f"sweep {cname} pair") for k in ks]
        m["quarter"] = one(cfg, (tm // 2) * bm, (tn // 2) * bn, ks[1], f"sweep {cname} quarter")
        m["full_shape"] = (8192, 8192, 8192)
        m["full"] = one(cfg, 8192, 8192, 8192, f"sweep {cname} full")
        m["ragged"] = one(cfg, tm * bm - 3, tn * bn - 3, ks[1] - 5, f"sweep {cname} ragged")
        meas[cname] = m
        log(f"sweep {cname}: {m}")
    res = {"cus": cus, "measured_us": meas, "model": fit_tile_model(meas, cus)}
    groups = {}
    for M, N, K in ((8192, 8192, 8192), (4096, 4096, 4096), (512, 11008, 4096)):
        st, auto = tg.tg_gemm_tiles_plan(M, N, K, cus)
        A, B, C = operands(M, N, K)
        launches = {f"group_m={gm}": tiled_launcher(torch, tg, M, N, K, 0, 0, A, B, None, C, auto,
                                                    f"sweep group {gm}", gm) for gm in (1, 2, 4, 8, 16)}
        groups[f"{M}x{N}x{K} {tg.TILES_NAMES[auto]}"] = {k: round(v * 1e3, 2)
                                                         for k, v in time_alternating(torch, launches, steps).items()}
        log(f"sweep raster groups {M}x{N}x{K}: {groups[f'{M}x{N}x{K} {tg.TILES_NAMES[auto]}']}")
        del A, B, C, launches
    res["raster_groups"] = groups
    res["shape_classes"] = bench_tile_choice(torch, tg, I, steps, warmup)
    torch.cuda.empty_cache()
    return res


def bench_attention(torch, tg, I, steps, warmup):
    """The attention forward at the benchmark shape, without and with the
    causal mask: per-launch time and TFLOP/s."""
    wa = I.ATTN_WORKLOAD
    Bn, H, S, D, dt = wa["batch"], wa["heads"], wa["seq"], wa["head_dim"], wa["dtype"]
    tdt = torch.float16 if dt == I.F16 else torch.bfloat16

    def dev(seed):
        bits = I.random_bits((Bn, S, H, D), wa["dist"], dt, seed)
        return torch.from_numpy(bits.view(np.int16).reshape(Bn, S, H, D).copy()).view(tdt).cuda()

    Q, K, V = (dev(s) for s in wa["seeds"])
    O = torch.empty_like(Q)
    handle = torch.cuda.current_stream().cuda_stream
    out = {}
    for causal in (False, True):
        key = "causal" if causal else "non_causal"
        label = f"{wa['name']} {key.replace('_', '-')}"

        def launch(i, c=int(causal), label=label):
            LOG.note(label)
            st = tg.tg_attention_fwd(Bn, S, S, H, D, dt, Q.data_ptr(), K.data_ptr(), V.data_ptr(), c, 0.0,
                                     O.data_ptr(), handle)
            if st != tg.TG_OK:
                raise RuntimeError(f"tg_attention_fwd failed: {tg.tg_status_string(st)}")

        ms = time_calls(torch, launch, steps, warmup)
        tf = attention_flops(Bn, H, D, S, S, causal) / (ms * 1e-3) / 1e12
        out[key] = {"us_per_launch": round(ms * 1e3, 2), "TFLOP/s": round(tf, 2),
                    "frac_mfma_peak": round(tf / PEAK_MFMA_F16_TFLOPS, 4),
                    "traffic": measured_traffic(label)}
        log(f"{wa['name']} causal={causal}: {ms * 1e3:.1f} us, {tf:.1f} TFLOP/s")
    return wa["name"], out


def path_of(tg, w, operand_set):
    """Name of the kernel family tg_gemm picks for these operands."""
    A, B, bias, C = operand_set
    st, path = tg.tg_gemm_plan(w.M, w.N, w.K, w.dtype, A.data_ptr(), B.data_ptr(),
                               bias.data_ptr() if bias is not None else None, w.epilogue, C.data_ptr())
    return tg.PATH_NAMES.get(path, "?") if st == tg.TG_OK else "error"


def bench_rows(torch, tg, I, steps, warmup, copies=8):
    """17 <= M <= 64 at the decode width (N = 11008, K = 4096, fp16, no
    epilogue): the skinny kernel with two, three and four 16-row blocks per
    workgroup (the library's choice there), and the tiled family on the same
    operands for comparison, over `copies` rotating weight sets so that B
    streams from HBM."""
    N, K = 11008, 4096
    handle = torch.cuda.current_stream().cuda_stream

    def dev(bits, shape):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).reshape(shape).to("cuda")

    Bs = [dev(I.random_bits((K, N), ("normal", 0.0, 0.02), I.F16, 4100 + c), (K, N)) for c in range(copies)]
    res = {}
    for M in (32, 48, 64):
        A = dev(I.random_bits((M, K), ("normal", 0.0, 1.0), I.F16, 4200 + M), (M, K))
        C = torch.empty((M, N), dtype=torch.float16, device="cuda")
        st, path = tg.tg_gemm_plan(M, N, K, I.F16, A.data_ptr(), Bs[0].data_ptr(), None, I.EPI_NONE, C.data_ptr())
        assert st == tg.TG_OK, st
        name = f"gemm_f16_rows_{M}x{N}x{K}"
        times = {}
        for p in (tg.TG_PATH_AUTO, tg.TG_PATH_TILED):
            label = name if p == tg.TG_PATH_AUTO else f"{name} tiled"

            def launch(i, p=p, label=label):
                LOG.note(label)
                st = tg.tg_gemm_path(p, M, N, K, I.F16, A.data_ptr(), Bs[i % copies].data_ptr(), None, I.EPI_NONE,
                                     C.data_ptr(), handle)
                if st != tg.TG_OK:
                    raise RuntimeError(f"tg_gemm_path: {tg.tg_status_string(st)}")
            times[p] = time_calls(torch, launch, steps, warmup)
        nbytes = gemm_alg_bytes(M, N, K)
        ms = times[tg.TG_PATH_AUTO]
        res[name] = {
            "us_per_launch": round(ms * 1e3, 3), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
            "path": tg.PATH_NAMES[path], "tiled_us": round(times[tg.TG_PATH_TILED] * 1e3, 3),
            "speedup_vs_tiled": round(times[tg.TG_PATH_TILED] / ms, 3),
            "traffic": measured_traffic(name)}
        log(f"rows M={M}: {ms * 1e3:.2f} us ({tg.PATH_NAMES[path]}), tiled {times[tg.TG_PATH_TILED] * 1e3:.2f} us")
    return res


def device_operands(torch, I, w, copies=1):
    ops = I.make_operands(w)
    tdt = torch.float16 if w.dtype == I.F16 else torch.bfloat16

    def dev(bits, shape):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(tdt).reshape(shape).to("cuda")

    A = dev(ops.A, (w.M, w.K))
    B = dev(ops.B, (w.K, w.N))
    bias = dev(ops.bias, (w.N,)) if ops.bias is not None else None
    sets = []
    for c in range(copies):
        sets.append((A if c == 0 else A.clone(), B if c == 0 else B.clone(),
                     None if bias is None else (bias if c == 0 else bias.clone()),
                     torch.empty((w.M, w.N), dtype=tdt, device="cuda")))
    return ops, sets


def workload_named(I, name: str):
    """A workload by name: the fixed ones, or a decode shape
    gemm_f16_skinny_MxNxK with the decode workload's distributions and
    seeds (for profiling other widths)."""
    import dataclasses
    import re
    if name in I.WORKLOADS:
        return I.WORKLOADS[name]
    m = re.fullmatch(r"gemm_f16_skinny_(\d+)x(\d+)x(\d+)", name)
    if not m:
        raise SystemExit(f"unknown workload {name}")
    M, N, K = (int(v) for v in m.groups())
    return dataclasses.replace(I.WORKLOADS[SKINNY], name=name, M=M, N=N, K=K)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(I, w, ops, budget_s):
    """The oracle on a bounded sample of rows of workload w (test infrastructure)."""
    import oracle
    probes = []
    for k in (2, 34):
        t0 = time.perf_counter()
        oracle.gemm(w.M, w.N, w.K, w.dtype, ops.A, ops.B, ops.bias, w.epilogue, ops.rows[:k])
        probes.append(time.perf_counter() - t0)
    per_row = max((probes[1] - probes[0]) / 32, 1e-6)
    fixed = max(probes[0] - 2 * per_row, 0.0)
    n = int(max(4, min(w.M, (budget_s - fixed) / per_row)))
    rng = np.random.Generator(np.random.PCG64(w.seeds["rows"] + 17))
    rows = np.sort(rng.choice(w.M, size=n, replace=False)).astype(np.int64)
    t0 = time.perf_counter()
    oracle.gemm(w.M, w.N, w.K, w.dtype, ops.A, ops.B, ops.bias, w.epilogue, rows)
    dt = time.perf_counter() - t0
    return {
        "value": round(gemm_flops(n, w.N, w.K) / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.max_threads(),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"{n} of {w.M} rows of {w.name} (all {w.N} columns, K={w.K}), fp64 accumulate, "
                  f"{dt:.2f} s wall incl. decoding B",
    }


# ---------------------------------------------------------------- profile summaries

def _csv_rows(run_dir: str, pattern: str):
    import csv
    import glob
    files = sorted(glob.glob(os.path.join(run_dir, pattern), recursive=True))
    if not files:
        raise FileNotFoundError(f"no {pattern} under {run_dir}")
    out = []
    for f in files:
        with open(f) as fh:
            out += list(csv.DictReader(fh))
    return out


def _dispatches(run_dir: str, csv_pattern: str, counters: bool):
    """The library's dispatches of one rocprofv3 run (kernel names in namespace
    tg::) in dispatch order, each paired with the label its run's dispatch
    log gives the same position: [(label, {"name", "dur_us", counters...})]."""
    recs = {}
    for r in _csv_rows(run_dir, csv_pattern):
        name = r["Kernel_Name"]
        if "tg::" not in name:
            continue
        d = recs.setdefault(int(r["Dispatch_Id"]), {"name": name})
        d["dur_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if counters:
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    with open(os.path.join(run_dir, "dispatch_log.json")) as fh:
        labels = DispatchLog()
        labels.entries = json.load(fh)["entries"]
    lab = labels.expand()
    ids = sorted(recs)
    if len(ids) != len(lab):
        raise ValueError(f"{run_dir}: {len(ids)} library dispatches in the trace, {len(lab)} in the dispatch log")
    out = []
    run_start = 0
    for i, did in enumerate(ids):
        label = lab[i]
        if i == 0 or lab[i - 1] != label:
            run_start = i
        if label.endswith(" unfused"):   # the product, then one elementwise pass per epilogue step
            parts = ["product", "bias pass", "GELU pass"][:3 if "gelu" in label else 2]
            label = f"{label} {parts[(i - run_start) % len(parts)]}"
        out.append((label, recs[did]))
    return out


def _group(disp):
    g = {}
    for lab, rec in disp:
        g.setdefault(lab, []).append(rec)
    return g


def _mean(v):
    return sum(v) / len(v) if v else float("nan")


def counter_means(run_dir: str) -> dict:
    """Per bench line of one rocprofv3 --pmc run under run_dir (its CSV and
    the dispatch log bench.py wrote beside it): the number of the library's
    dispatches, their mean duration and the mean of every counter over them
    (each counter summed over its dimensions, as rocprofv3 reports it)."""
    out = {}
    for label, recs in _group(_dispatches(run_dir, "**/*counter_collection.csv", True)).items():
        keys = sorted({k for r in recs for k in r if k not in ("name", "dur_us")})
        out[label] = {"dispatches": len(recs), "dur_us": _mean([r["dur_us"] for r in recs]),
                      **{k: _mean([r.get(k, 0.0) for r in recs]) for k in keys}}
    return out


def _bench_json(path: str):
    with open(path) as fh:
        lines = [ln for ln in fh.read().splitlines() if ln.startswith("{")]
    return json.loads(lines[-1]) if lines else {}


def _alg(label: str, I, tg):
    """(flops, algorithmic bytes) of one bench line's launch, or (None, None)."""
    base = label.split(" ")[0]
    if base.startswith("attention"):
        wa = I.ATTN_WORKLOAD
        B, H, S, D = wa["batch"], wa["heads"], wa["seq"], wa["head_dim"]
        return attention_flops(B, H, D, S, S, "non-causal" not in label), 4 * B * H * S * D * 2
    if base == I.W4_WORKLOAD["name"]:
        wq = I.W4_WORKLOAD
        M, N, K, G = wq["M"], wq["N"], wq["K"], wq["group"]
        return gemm_flops(M, N, K), tg.tg_w4_packed_bytes(K, N) + 2 * (K // G) * N + 2 * M * K + 2 * M * N
    if base.startswith("gemm_f16_rows_"):
        M, N, K = (int(v) for v in base[len("gemm_f16_rows_"):].split("x"))
        return gemm_flops(M, N, K), gemm_alg_bytes(M, N, K)
    w = I.WORKLOADS.get(base) or I.TILE_WORKLOADS.get(base)
    if w is None:
        return None, None
    if label.endswith(("bias pass", "GELU pass")):
        return None, 4 * w.M * w.N
    epi = w.epilogue != I.EPI_NONE and "no epilogue" not in label and "product" not in label
    return gemm_flops(w.M, w.N, w.K), gemm_alg_bytes(w.M, w.N, w.K, bias=epi)


MFMA_COUNTERS = ["SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES",
                 "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
# LDS occupancy and MFMA / VALU overlap: a pass of its own (at most 8 SQ
# counters per pass)
LDS_COUNTERS = ["SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_VALU_MFMA_BUSY_CYCLES",
                "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_VALU_TRANS_F32", "GRBM_GUI_ACTIVE"]
PROFILE_COMMANDS = {
    "bench": "python3 bench.py > <out>/bench.json",
    "trace": "rocprofv3 --kernel-trace --stats --output-format csv -d <out>/trace -o run -- "
             "python3 bench.py --no-cpu-baseline --dispatch-log <out>/trace/dispatch_log.json "
             "> <out>/trace/bench.json",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/fetch -o run -- "
             "python3 bench.py --profile-run --dispatch-log <out>/fetch/dispatch_log.json",
    "write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/write -o run -- "
             "python3 bench.py --profile-run --dispatch-log <out>/write/dispatch_log.json",
    "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/copy_fetch -o run -- "
                  "python3 bench.py --copy-calibration 1024",
    "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/copy_write -o run -- "
                  "python3 bench.py --copy-calibration 1024",
    "mfma": "rocprofv3 --pmc " + " ".join(MFMA_COUNTERS) + " --output-format csv -d <out>/mfma -o run -- "
            "python3 bench.py --profile-run --dispatch-log <out>/mfma/dispatch_log.json",
    "lds": "rocprofv3 --pmc " + " ".join(LDS_COUNTERS) + " --output-format csv -d <out>/lds -o run -- "
           "python3 bench.py --profile-run --dispatch-log <out>/lds/dispatch_log.json",
    "summarise": "python3 bench.py --summarise <out>",
}


def summarise_profiles(run_dir: str, out_dir: str) -> None:
    """Writes profiles/{kernel_trace,hbm_traffic,counters_mfma_lds}.md and
    profiles/counters.json from the rocprofv3 runs under run_dir (the
    commands in PROFILE_COMMANDS, each in the subdirectory of its name).

    HBM traffic: FETCH_SIZE and WRITE_SIZE (KiB per dispatch, each from a
    run of its own) are scaled by what the same counter reads for a 1 GiB
    device copy.  Shader clock: GRBM_GUI_ACTIVE counts busy cycles of each of
    the 8 XCDs' graphics engines and rocprofv3 sums the 8, so the clock is
    GRBM_GUI_ACTIVE / 8 / the dispatch's duration.  MFMA utilisation:
    SQ_VALU_MFMA_BUSY_CYCLES (summed over the 1024 SIMDs) / (1024 x
    GRBM_GUI_ACTIVE / 8), the fraction of SIMD cycles at that clock in which
    the matrix core was busy; SQ_INSTS_VALU_MFMA_MOPS_* x 512 cross-checks
    the flops.  Counter runs serialise dispatches, so their clock is that of
    the counter run, not of the timed bench; and GRBM_GUI_ACTIVE spans the
    counter window, a little longer than the dispatch, which matters only for
    short dispatches (about 10 % at 100 us)."""
    import statistics
    import tiled_dense_gemm_tg_amd as tg
    from tiled_dense_gemm_tg_amd import inputs as I
    os.makedirs(out_dir, exist_ok=True)
    khash = kernel_source_hash()
    cmd_lines = ["```", "cd /tmp && export TMPDIR=/tmp   # rocprofv3 writes temporary files there",
                 "cd /root/repo"] + [PROFILE_COMMANDS[k].replace("<out>", "$OUT") for k in PROFILE_COMMANDS] + ["```"]

    # kernel trace
    trace = _group(_dispatches(os.path.join(run_dir, "trace"), "**/*kernel_trace.csv", False))
    tres = _bench_json(os.path.join(run_dir, "trace", "bench.json")) if os.path.exists(
        os.path.join(run_dir, "trace", "bench.json")) else {}
    bres = _bench_json(os.path.join(run_dir, "bench.json")) if os.path.exists(os.path.join(run_dir, "bench.json")) else {}
    lines = ["# Kernel trace of the default bench (rocprofv3 --kernel-trace --stats)", "",
             "Commands (one MI355X; `$OUT` a scratch directory; committed files only):", ""] + cmd_lines + [
             "", f"Kernel sources: `bench.kernel_source_hash()` = `{khash}`.", "",
             "Per-dispatch durations from the trace, grouped by the bench line each dispatch belongs to (the "
             "dispatch log that `--dispatch-log` writes labels every library launch; warm-up and settling "
             "dispatches included):", "",
             "| bench line | kernel | calls | average us | median us | min us | max us |", "|---|---|---|---|---|---|---|"]
    for lab, recs in trace.items():
        ds = [r["dur_us"] for r in recs]
        lines.append(f"| {lab} | `{recs[0]['name']}` | {len(ds)} | {_mean(ds):.2f} | {statistics.median(ds):.2f} | "
                     f"{min(ds):.2f} | {max(ds):.2f} |")
    if tres:
        lines += ["", f"The traced run's own line: {tres.get('value')} {tres.get('unit')}, "
                      f"{tres.get('ms_per_step', 0) * 1e3:.1f} us per launch (HIP events, back to back)."]
    if bres:
        lines += ["", f"The unprofiled run: {bres.get('value')} {bres.get('unit')}, "
                      f"{bres.get('ms_per_step', 0) * 1e3:.1f} us per launch."]
    with open(os.path.join(out_dir, "kernel_trace_bench_default.md"), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    # HBM traffic
    def copy_value(sub, cname):
        rs = _csv_rows(os.path.join(run_dir, sub), "**/*counter_collection.csv")
        return max(float(r["Counter_Value"]) for r in rs if r["Counter_Name"] == cname)

    fscale = 1024 * 1024 / copy_value("copy_fetch", "FETCH_SIZE")
    wscale = 1024 * 1024 / copy_value("copy_write", "WRITE_SIZE")
    fetch = _group(_dispatches(os.path.join(run_dir, "fetch"), "**/*counter_collection.csv", True))
    write = _group(_dispatches(os.path.join(run_dir, "write"), "**/*counter_collection.csv", True))
    mfma = _group(_dispatches(os.path.join(run_dir, "mfma"), "**/*counter_collection.csv", True))
    record = {"_about": summarise_profiles.__doc__.split("\n\n", 1)[1].strip(), "kernel_hash": khash,
              "fetch_scale": round(fscale, 5), "write_scale": round(wscale, 5), "lines": {}}
    h = ["# HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
         "Commands:", ""] + cmd_lines + [
         "", f"Calibration: a 1 GiB device copy reads FETCH_SIZE x {fscale:.4f} and WRITE_SIZE x {wscale:.4f} "
             "KiB per GiB moved, so fetched bytes = FETCH_SIZE x 1024 x that factor (written likewise).", "",
         "| bench line | fetched MB | written MB | total MB | algorithmic MB | total / algorithmic |",
         "|---|---|---|---|---|---|"]
    m = ["# MFMA utilisation, shader clock and LDS counters (rocprofv3 --pmc)", "",
         "Commands:", ""] + cmd_lines + [
         "", "Derivations (per dispatch, then the mean over the bench line's dispatches):",
         "* clock = GRBM_GUI_ACTIVE / 8 XCDs / dispatch duration (rocprofv3 sums the 8 XCDs' counters);",
         "* MFMA utilisation = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8);",
         "* MFMA flops = (SQ_INSTS_VALU_MFMA_MOPS_F16 + _BF16) x 512, against 2MNK.",
         "Counter runs serialise the dispatches, so the clock is the counter run's, not the timed bench's.",
         "GRBM_GUI_ACTIVE covers the counter sampling window, a little longer than the dispatch: for dispatches",
         "near 1 ms the clock agrees within about 1 % with the clock measured inside the kernel (s_memtime against",
         "the 100 MHz s_memrealtime), for 100-us dispatches it reads about 10 % high and the utilisation as much",
         "low, and for dispatches of a few tens of us both are meaningless (clocks above the 2.4 GHz maximum).", "",
         "| bench line | duration us | clock GHz | MFMA util | MFMA flops / 2MNK | LDS instr | LDS bank conflicts |",
         "|---|---|---|---|---|---|---|"]
    for lab in fetch:
        if lab.startswith(("w4 weight packing", "sweep")):
            continue
        fb = _mean([r["FETCH_SIZE"] for r in fetch[lab]]) * 1024 * fscale
        wb = _mean([r["WRITE_SIZE"] for r in write.get(lab, [])]) * 1024 * wscale if lab in write else float("nan")
        flops, ab = _alg(lab, I, tg)
        rec = {"kernel": fetch[lab][0]["name"], "kernel_hash": khash, "bytes_per_launch": int(fb + wb),
               "fetched_bytes": int(fb), "written_bytes": int(wb), "algorithmic_bytes": ab}
        h.append(f"| {lab} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {(fb + wb) / 1e6:.1f} | "
                 f"{ab / 1e6 if ab else float('nan'):.1f} | {(fb + wb) / ab if ab else float('nan'):.2f} |")
        if lab in mfma:
            rs = mfma[lab]
            clk = [r["GRBM_GUI_ACTIVE"] / 8 / (r["dur_us"] * 1e3) for r in rs]
            util = [r["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * r["GRBM_GUI_ACTIVE"] / 8) for r in rs]
            mops = _mean([r["SQ_INSTS_VALU_MFMA_MOPS_F16"] + r["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for r in rs]) * 512
            rec.update({"sclk_ghz": round(_mean(clk), 3), "mfma_util": round(_mean(util), 4),
                        "counter_run_us": round(_mean([r["dur_us"] for r in rs]), 2),
                        "mfma_flops": mops, "lds_instructions": _mean([r["SQ_INSTS_LDS"] for r in rs]),
                        "lds_bank_conflicts": _mean([r["SQ_LDS_BANK_CONFLICT"] for r in rs])})
            m.append(f"| {lab} | {rec['counter_run_us']:.1f} | {rec['sclk_ghz']:.3f} | {rec['mfma_util']:.3f} | "
                     f"{mops / flops if flops else float('nan'):.3f} | {rec['lds_instructions']:.0f} | "
                     f"{rec['lds_bank_conflicts']:.0f} |")
        record["lines"][lab] = rec
    lds_dir = os.path.join(run_dir, "lds")
    if os.path.isdir(lds_dir):
        lds = _group(_dispatches(lds_dir, "**/*counter_collection.csv", True))
        m += ["", "LDS occupancy and MFMA / VALU overlap (the `lds` pass), per dispatch, then the mean:",
              "* LDS busy = SQ_LDS_IDX_ACTIVE / (256 CUs x GRBM_GUI_ACTIVE / 8): the fraction of CU cycles in "
              "which the LDS serves indexed (ds_*) accesses; the direct-to-LDS buffer loads are not indexed "
              "accesses;",
              "* MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8), as above;",
              "* co-issue = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES: the share of the matrix "
              "core's busy cycles in which the same SIMD's VALU also issued;",
              "* VALU active = SQ_ACTIVE_INST_VALU x 4 (quad-cycles) / (1024 x GRBM_GUI_ACTIVE / 8);",
              "* exp2/rcp per SIMD cycle = SQ_INSTS_VALU_TRANS_F32 / (1024 x GRBM_GUI_ACTIVE / 8).", "",
              "| bench line | duration us | LDS busy | MFMA busy | co-issue | VALU active | trans instr / SIMD cycle |",
              "|---|---|---|---|---|---|---|"]
        for lab, rs in lds.items():
            if lab.startswith(("w4 weight packing", "sweep")):
                continue
            simd = [1024 * r["GRBM_GUI_ACTIVE"] / 8 for r in rs]
            busy = _mean([r["SQ_LDS_IDX_ACTIVE"] / (256 * r["GRBM_GUI_ACTIVE"] / 8) for r in rs])
            mb = _mean([r["SQ_VALU_MFMA_BUSY_CYCLES"] / c for r, c in zip(rs, simd)])
            co = _mean([r["SQ_VALU_MFMA_COEXEC_CYCLES"] / max(r["SQ_VALU_MFMA_BUSY_CYCLES"], 1) for r in rs])
            va = _mean([4 * r["SQ_ACTIVE_INST_VALU"] / c for r, c in zip(rs, simd)])
            tr = _mean([r["SQ_INSTS_VALU_TRANS_F32"] / c for r, c in zip(rs, simd)])
            m.append(f"| {lab} | {_mean([r['dur_us'] for r in rs]):.1f} | {busy:.3f} | {mb:.3f} | {co:.3f} | "
                     f"{va:.3f} | {tr:.4f} |")
            if lab in record["lines"]:
                record["lines"][lab].update({"lds_busy": round(busy, 4), "mfma_valu_coissue": round(co, 4)})
    with open(os.path.join(out_dir, "hbm_traffic.md"), "w") as fh:
        fh.write("\n".join(h) + "\n")
    with open(os.path.join(out_dir, "counters_mfma_lds.md"), "w") as fh:
        fh.write("\n".join(m) + "\n")
    with open(os.path.join(out_dir, "counters.json"), "w") as fh:
        json.dump(record, fh, indent=1)
        fh.write("\n")


# ---------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--workload", default=MAIN, help="workload timed as the main line (for profiling runs)")
    ap.add_argument("--sweep", action="store_true",
                    help="only time every tile configuration of the tiled family (prints its own JSON line)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run torch's device copy of MIB MiB, 10 times (to scale HBM byte counters)")
    ap.add_argument("--dispatch-log", default=None, metavar="FILE",
                    help="write the label of every library kernel launch, in order, to FILE (JSON)")
    ap.add_argument("--profile-run", action="store_true",
                    help="no settling, short lines: for rocprofv3 counter runs")
    ap.add_argument("--summarise", default=None, metavar="DIR",
                    help="only summarise the rocprofv3 runs under DIR into profiles/")
    ap.add_argument("--counter-means", default=None, metavar="DIR",
                    help="only print, per bench line, the mean of every counter of the rocprofv3 --pmc run under DIR")
    ap.add_argument("--write-tile-model", default=None, metavar="SWEEP_JSON",
                    help="only write the tile-choice model table and profiles/tile_sweep.md from a --sweep output line")
    args = ap.parse_args()
    if args.summarise:
        summarise_profiles(args.summarise, os.path.join(ROOT, "profiles"))
        return 0
    if args.counter_means:
        print(json.dumps(counter_means(args.counter_means), indent=1))
        return 0
    if args.write_tile_model:
        with open(args.write_tile_model) as fh:
            sweep = json.loads([ln for ln in fh.read().splitlines() if ln.startswith("{")][-1])
        write_tile_model(sweep)
        write_sweep_summary(sweep)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this GEMM runs on a single "
              "MI355X and has no multi-GPU path.", file=sys.stderr)
        return 2
    if args.profile_run:
        Timing.settle_s = 0.0
        Timing.short = True
        args.steps, args.warmup = 3, 1
        args.no_cpu_baseline = True

    import torch
    import tiled_dense_gemm_tg_amd as tg
    from tiled_dense_gemm_tg_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.copy_calibration} MiB 10 times")
        return 0
    tg.load_library()
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")
    if args.sweep:
        print(json.dumps({"tile_sweep": tile_sweep(torch, tg, I, max(args.steps // 2, 20), args.warmup)}),
              flush=True)
        return 0

    w = workload_named(I, args.workload)
    log(f"main workload {w.name}: generating inputs")
    ops, sets = device_operands(torch, I, w)
    ms, wall = time_gemm(torch, tg, w, sets, args.steps, args.warmup)
    flops = gemm_flops(w.M, w.N, w.K)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{w.name}: {ms * 1e3:.1f} us/launch, {tflops:.1f} TFLOP/s")
    path_name = {I.EPI_NONE: "none", I.EPI_BIAS: "bias", I.EPI_BIAS_GELU_TANH: "bias + GELU(tanh)"}[w.epilogue]
    st, path = tg.tg_gemm_plan(w.M, w.N, w.K, w.dtype, *[sets[0][i].data_ptr() if sets[0][i] is not None else None
                                                        for i in (0, 1, 2)], w.epilogue, sets[0][3].data_ptr())
    cnt = measured(w.name) or {}
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": I.DTYPE_NAMES[w.dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "inputs": I.DTYPE_NAMES[w.dtype],
                   "accumulate": "fp32", "output": I.DTYPE_NAMES[w.dtype], "epilogue": path_name,
                   "path": tg.PATH_NAMES.get(path, "?"), "parallelism": "none"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": PEAK_MFMA_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_MFMA_F16_TFLOPS, 4),
            "traffic": cnt.get("bytes_per_launch"),
            "mfma_util": cnt.get("mfma_util"),
            "sclk_ghz": cnt.get("sclk_ghz"),
            "counters": ("profiles/counters.json: rocprofv3 --pmc runs of this script on the current kernel "
                         "sources; clock = GRBM_GUI_ACTIVE / 8 XCDs / dispatch time, MFMA util = "
                         "SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x that cycle count), both in the counter run")
            if cnt else None,
            "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": gemm_alg_bytes(w.M, w.N, w.K, bias=w.epilogue != I.EPI_NONE),
            "timed_region_wall_s": round(wall, 4),
        },
    }
    fusion = {}
    if not args.no_secondary and w.epilogue != I.EPI_NONE:
        log(f"{w.name}: fused, unfused (product, bias pass, GELU pass) and no epilogue, alternating")
        fusion[w.name] = fusion_comparison(torch, tg, w, sets, steps_for(10), args.warmup)
        log(f"{w.name}: {fusion[w.name]}")
    del sets
    torch.cuda.empty_cache()

    if not args.no_secondary:
        sec = {}
        w2 = I.WORKLOADS[SQUARE]
        log(f"secondary {w2.name}")
        _, sets2 = device_operands(torch, I, w2)
        ms2, _ = time_gemm(torch, tg, w2, sets2, steps_for(max(args.steps, 50)), args.warmup)
        t2 = gemm_flops(w2.M, w2.N, w2.K) / (ms2 * 1e-3) / 1e12
        c2 = measured(w2.name) or {}
        sec[w2.name] = {"us_per_launch": round(ms2 * 1e3, 2), "TFLOP/s": round(t2, 2),
                        "frac_mfma_peak": round(t2 / PEAK_MFMA_F16_TFLOPS, 4), "path": path_of(tg, w2, sets2[0]),
                        "traffic": c2.get("bytes_per_launch"), "mfma_util": c2.get("mfma_util"),
                        "sclk_ghz": c2.get("sclk_ghz")}
        del sets2
        torch.cuda.empty_cache()
        w4 = I.WORKLOADS[SKINNY]
        log(f"secondary {w4.name} (8 rotating operand sets)")
        _, sets4 = device_operands(torch, I, w4, copies=8)
        steps4 = steps_for(max(args.steps, 400))
        ms4, _ = time_gemm(torch, tg, w4, sets4, steps4, args.warmup)
        hot, _ = time_gemm(torch, tg, w4, sets4[:1], steps4, args.warmup, label=f"{w4.name} hot")
        # stream-K over every CU, the opt-in split mode (not the library's
        # choice at this shape): its time, for the record
        ws4 = torch.zeros(tg.tg_gemm_split_workspace_bytes(w4.N, tg.TG_SPLIT_STREAM_K), dtype=torch.uint8,
                          device="cuda")
        msk, _ = time_gemm(torch, tg, w4, sets4, steps4, args.warmup, label=f"{w4.name} stream-K", mode="split",
                           ws=ws4, splits=tg.TG_SPLIT_STREAM_K)
        del ws4
        nbytes = gemm_alg_bytes(w4.M, w4.N, w4.K)
        gbps = nbytes / (ms4 * 1e-3) / 1e9
        sec[w4.name] = {"us_per_launch": round(ms4 * 1e3, 3), "GB/s": round(gbps, 1),
                        "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                        "hot_cache_GB/s_not_the_metric": round(nbytes / (hot * 1e-3) / 1e9, 1),
                        "stream_k_us": round(msk * 1e3, 3),
                        "TFLOP/s": round(gemm_flops(w4.M, w4.N, w4.K) / (ms4 * 1e-3) / 1e12, 2),
                        "path": path_of(tg, w4, sets4[0]), "traffic": measured_traffic(w4.name)}
        log(f"{w4.name}: {ms4 * 1e3:.2f} us, {gbps:.0f} GB/s; stream-K {msk * 1e3:.2f} us")
        del sets4
        torch.cuda.empty_cache()
        log("secondary: 32, 48 and 64 rows at the decode width (8 rotating weight sets)")
        sec.update(bench_rows(torch, tg, I, steps_for(max(args.steps, 400)), args.warmup))
        torch.cuda.empty_cache()
        log("secondary: weight-only 4-bit product at the same shape (16 rotating weight sets)")
        wname, msq, hotq, qbytes = bench_w4(torch, tg, I, steps_for(max(args.steps, 400)), args.warmup)
        qgbps = qbytes / (msq * 1e-3) / 1e9
        sec[wname] = {"us_per_launch": round(msq * 1e3, 3), "GB/s": round(qgbps, 1),
                      "frac_hbm_peak": round(qgbps / PEAK_HBM_GBPS, 4),
                      "hot_cache_us_not_the_metric": round(hotq * 1e3, 3),
                      "algorithmic_bytes": qbytes, "speedup_vs_16bit_weights": round(ms4 / msq, 3),
                      "path": "w4", "traffic": measured_traffic(wname)}
        log(f"{wname}: {msq * 1e3:.2f} us, {qgbps:.0f} GB/s, {ms4 / msq:.2f}x the 16-bit weights")
        torch.cuda.empty_cache()
        w3 = I.WORKLOADS[RAGGED]
        log(f"secondary {w3.name}")
        _, sets3 = device_operands(torch, I, w3)
        ms3, _ = time_gemm(torch, tg, w3, sets3, steps_for(max(args.steps, 50)), args.warmup)
        t3 = gemm_flops(w3.M, w3.N, w3.K) / (ms3 * 1e-3) / 1e12
        c3 = measured(w3.name) or {}
        sec[w3.name] = {"us_per_launch": round(ms3 * 1e3, 2), "TFLOP/s": round(t3, 2),
                        "frac_mfma_peak": round(t3 / PEAK_MFMA_F16_TFLOPS, 4), "path": path_of(tg, w3, sets3[0]),
                        "traffic": c3.get("bytes_per_launch"), "mfma_util": c3.get("mfma_util"),
                        "sclk_ghz": c3.get("sclk_ghz")}
        log(f"{w3.name}: {ms3 * 1e3:.1f} us; fused, unfused and no epilogue, alternating")
        fusion[w3.name] = fusion_comparison(torch, tg, w3, sets3, steps_for(50), args.warmup)
        del sets3
        torch.cuda.empty_cache()
        log("secondary: tile configurations on the mid-size shape classes")
        sec["tile_choice"] = bench_tile_choice(torch, tg, I, steps_for(max(args.steps // 2, 20)), args.warmup)
        log("secondary: attention forward (FlashAttention benchmark shape)")
        aname, ares = bench_attention(torch, tg, I, steps_for(max(args.steps // 2, 20)), args.warmup)
        sec[aname] = ares
        sec["epilogue_fusion"] = fusion
        result["secondary"] = sec

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(I, w, ops, args.cpu_budget)

    if args.dispatch_log:
        os.makedirs(os.path.dirname(os.path.abspath(args.dispatch_log)), exist_ok=True)
        with open(args.dispatch_log, "w") as fh:
            json.dump({"argv": sys.argv[1:], "entries": LOG.entries}, fh)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

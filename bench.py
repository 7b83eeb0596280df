#!/usr/bin/env python3
"""Benchmark of the Stream-K GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload sgemm-sweep|hgemm-8192]

A step is one pass of the whole hot path over one batch of synthetic inputs:
  sgemm-sweep (default): the fp32 square sweep m = n = k in {1024, 2048, 3072,
      4096, 5120, 6144}, row-major A and B, entries U[-1, 1], C pre-filled
      U[-1, 1], alpha = 1, beta = 1 -- six GEMM calls;
  hgemm-8192: one 8192^3 fp16 GEMM, A row-major and B column-major, entries
      N(0, 1)/sqrt(k), fp32 accumulation, alpha = 1, beta = 0.
Inputs are generated on the host from the seeded counter-based generator and
are resident in HBM before the timed region.  W untimed steps, then K timed
steps between synchronisations; one JSON line is printed.

The line carries
  roofline: the GEMM kernel's achieved rate (algorithmic flops per launch over
      its mean launch time, from HIP events on the launch stream) against
      MI355X's dense peak for the data type;
  cpu_baseline: the CPU oracle timed on a bounded sample of the workload;
  hgemm / sgemm: the other workload's throughput, measured in the same run.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}
PEAK_HBM_GBS = 8000.0
METRIC = "GEMM TFLOPS + % of MI355X MFMA peak (fp32, fp16) over shape sweep"
SWEEP = [1024, 2048, 3072, 4096, 5120, 6144]
# HBM bytes per dispatch measured with rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE, scaled by the copy-kernel calibration); None when not measured
# for the current kernel.
# HBM traffic per launch of the dominant kernel (bytes), from rocprofv3 --pmc
# FETCH_SIZE and WRITE_SIZE runs of this script scaled by the copy-kernel
# calibration (read and written bytes per counter KiB).  Valid only for the
# kernel sources whose hash is recorded: after any kernel change the field
# reports null until the counters are taken again.
KERNEL_SOURCES = ("work_centric_decomposition_amd/csrc/sk_kernels.hip",
                  "work_centric_decomposition_amd/csrc/sk_internal.h")
TRAFFIC = {"kernel_hash": "8feefbd6b145e4fd",
           # mean over the six launches of one step (1024^3 ... 6144^3)
           "sgemm-sweep": 1170550910,
           # fp16 8192^3 launch
           "hgemm-8192": 1775136510,
           # bf16 8192^3 launch (same counter runs)
           "hgemm-8192-bf16": 1764242395}


def kernel_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(wl):
    return TRAFFIC[wl] if TRAFFIC["kernel_hash"] == kernel_hash() else None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="sgemm-sweep", choices=["sgemm-sweep", "hgemm-8192"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true", help="skip the other workload")
    p.add_argument("--sweep", type=int, default=0, metavar="COUNT",
                   help="only the Stream-K shape sweep on COUNT shapes (2000: all) and print its summary")
    p.add_argument("--sweep-out", default="", help="CSV file for the per-shape sweep results")
    p.add_argument("--sweep-legs", default="auto,dp",
                   help="schedules timed per sweep shape: auto, dp, page, large, small, basic, hybrid2, "
                        "hybrid2_w2, hybrid1, xcd_w2")
    p.add_argument("--sweep-count", type=int, default=300,
                   help="shapes of the sweep leg in the default run (0: no sweep leg)")
    p.add_argument("--skinny", action="store_true",
                   help="time eight memory-bound skinny fp16 shapes of the sweep (AUTO and DP), "
                        "--steps launches each")
    p.add_argument("--peaks", action="store_true",
                   help="measure the sustained MFMA rates and the HBM read rate only")
    p.add_argument("--gemv", action="store_true",
                   help="time the matrix-vector products only (m == 1 or n == 1 shapes)")
    p.add_argument("--abft", action="store_true",
                   help="time the fp32 4096^3 GEMM with and without ABFT only")
    p.add_argument("--compare-schedules", action="store_true",
                   help="time AUTO, the page's schedules and data-parallel on a few fp16 shapes "
                        "(one launch each with --steps 1, e.g. under rocprofv3 --pmc)")
    p.add_argument("--library-gemm", action="store_true",
                   help="time only the vendor GEMM behind torch.mm on the 8192^3 fp16 and bf16 "
                        "inputs of the hgemm workload (context for the kernel's counters; not "
                        "this library's path)")
    p.add_argument("--calibrate-model", type=int, default=0, metavar="SHAPES",
                   help="measure the runtime model's constants a, b, c, d (single-tile and split-tile "
                        "timings) for fp16 and fp32, then compare basic Stream-K at the model's grid "
                        "(default and measured constants) with the best grid of an exhaustive search "
                        "on SHAPES seeded fp16 sweep shapes below one wave")
    p.add_argument("--layouts", action="store_true",
                   help="time only 8192^3 fp16 GEMMs with B read in place (beta 0 and 1), B repacked and "
                        "both operands repacked (--steps calls each after 3 warm-ups)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device-to-device copy 5 times (calibrates the "
                        "FETCH_SIZE / WRITE_SIZE counters against a kernel of known traffic)")
    return p.parse_args()


COMPARE_SHAPES = [(9392, 2976, 14144), (4352, 4096, 4096), (3808, 4624, 720), (2048, 2048, 8192)]


def compare_schedules(torch, sk, S, steps):
    """Each shape of COMPARE_SHAPES (fp16, A row-major, B column-major) on the
    256x256 tile under the data-parallel schedule, the page's two-tile hybrid
    (basic Stream-K below one wave) and the XCD-aware split, then AUTO with
    its own tile choice, in that order; `steps` timed launches each after one
    warm-up (with steps == 1 the launches are easy to pick out of a counter
    trace: dispatches come in pairs per leg)."""
    out = []
    g = torch.Generator(device="cuda")
    g.manual_seed(S.SEED_SWEEP)
    for m, n, k in COMPARE_SHAPES:
        A = (torch.randn(m * k, generator=g, device="cuda") / math.sqrt(k)).to(torch.float16)
        B = torch.randn(k * n, generator=g, device="cuda").to(torch.float16)
        C = torch.empty(m * n, device="cuda", dtype=torch.float16)
        d = sk.make_desc(m, n, k, 1.0, A, k, B, k, 0.0, C, n, sk.F16, sk.A_ROW_B_COL)
        large = sk.TILE_LARGE
        pl = sk.plan_query(d, sk.make_options(tile=large))
        page = sk.SCHED_SK_HYBRID2 if pl.tiles >= pl.slots else sk.SCHED_SK_BASIC
        for name, opts in (("dp", sk.make_options(schedule=sk.SCHED_DP, tile=large)),
                           ("page", sk.make_options(schedule=page, tile=large)),
                           ("auto", sk.make_options(tile=large)), ("auto_tile", sk.make_options())):
            sk.gemm_ex(d, opts)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                sk.gemm_ex(d, opts)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            p = sk.plan_query(d, opts)
            out.append({"shape": [m, n, k], "schedule": name, "resolved": p.schedule, "tile": p.tile_m, "grid": p.grid,
                        "sk_tiles": p.sk_tiles, "phase_div": p.phase_div, "us": round(us, 1),
                        "tflops": round(2.0 * m * n * k / us / 1e6, 1)})
        del A, B, C
    return out


def layouts_leg(torch, sk, S, steps):
    """8192^3 fp16 (the hgemm workload's N(0,1)/sqrt(k) operands, alpha = 1)
    in every storage order, all read in place (k-contiguous operands as
    they are, m-contiguous A and n-contiguous B through transposing LDS
    reads), beta 0 and, for A row-major and B column-major, 1; and B
    row-major with a leading dimension of n + 4 (not a multiple of 8
    elements), which is repacked: `steps` calls per case between one event
    pair after 3 warm-ups, and 30 warm-up calls before the first case."""
    h = make_hgemm_inputs(torch, sk, S, sk.F16)
    n, A, B, C = h["n"], h["A"], h["B"], h["C"]
    Bp = torch.empty(n * (n + 4), dtype=B.dtype, device=B.device)
    Bp.view(n, n + 4)[:, :n].copy_(B.view(n, n))
    cases = [("A row, B col: k-contiguous", sk.A_ROW_B_COL, 0.0, B, n),
             ("A row, B col: k-contiguous, beta 1", sk.A_ROW_B_COL, 1.0, B, n),
             ("A row, B row: B n-contiguous", sk.A_ROW_B_ROW, 0.0, B, n),
             ("A col, B col: A m-contiguous", sk.A_COL_B_COL, 0.0, B, n),
             ("A col, B row: both mn-contiguous", sk.A_COL_B_ROW, 0.0, B, n),
             ("A row, B row, ldb = n + 4: B repacked", sk.A_ROW_B_ROW, 0.0, Bp, n + 4)]
    d0 = sk.make_desc(n, n, n, 1.0, A, n, B, n, 0.0, C, n, sk.F16, sk.A_ROW_B_COL)
    for _ in range(30):
        sk.gemm_ex(d0, None)
    torch.cuda.synchronize()
    out = []
    for name, layout, beta, Bx, ldb in cases:
        d = sk.make_desc(n, n, n, 1.0, A, n, Bx, ldb, beta, C, n, sk.F16, layout)
        for _ in range(3):
            sk.gemm_ex(d, None)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            sk.gemm_ex(d, None)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / steps * 1e3
        out.append({"case": name, "beta": beta, "packs": sk.plan_query(d).packs, "us_per_call": round(us, 1),
                    "tflops": round(2.0 * n ** 3 / us * 1e-6, 1)})
    return out


def library_gemm(torch, sk, S, steps, warmup):
    """The vendor GEMM (torch.mm) on the hgemm workload's inputs: A row-major,
    B column-major (a transposed view of its k-contiguous storage)."""
    out = []
    for dt, name in ((sk.F16, "f16"), (sk.BF16, "bf16")):
        h = make_hgemm_inputs(torch, sk, S, dt)
        n = h["n"]
        a = h["A"].view(n, n)
        b = h["B"].view(n, n).t()
        for _ in range(warmup):
            torch.mm(a, b)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            torch.mm(a, b)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out.append({"library_gemm": "torch.mm", "dtype": name, "shape": [n, n, n], "ms": round(ms, 4),
                    "tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)})
        del h, a, b
    return out


# (m, n, k, dtype, layout): k-contiguous matrix operand (dot-product form),
# the matrix contiguous along the output (axpy form), eight vectors (multi
# form)
GEMV_SHAPES = [(1, 16384, 16384, "f16", 1), (16384, 1, 16384, "f16", 1), (1, 16384, 16384, "f32", 1),
               (1, 1, 1 << 24, "f32", 1), (1, 16384, 16384, "f16", 0), (16384, 1, 16384, "f16", 3),
               (1, 16384, 16384, "f32", 0), (8, 16384, 16384, "f16", 1), (8, 16384, 16384, "f32", 1),
               (8, 16384, 16384, "f16", 0)]


def gemv_leg(torch, sk, S, reps=20):
    """Matrix-vector products through the even split of dot products (AUTO
    picks it for m == 1 or n == 1), and a few vectors at once (the multi form
    when both operands are k-contiguous, else the tiled kernels, form
    "tiled"): per-launch time queued behind a spin kernel, bytes = the
    matrix, the vectors and the output once each, against the 8 TB/s HBM
    peak; torch.matmul on the same operands for context."""
    import statistics
    dts = {"f16": (sk.F16, torch.float16, 2), "f32": (sk.F32, torch.float32, 4)}
    spin = _spin_cycles(torch, 300e-6)
    out = []
    for (m, n, k, name, layout) in GEMV_SHAPES:
        dt, tdt, es = dts[name]
        g = torch.Generator(device="cuda").manual_seed(m + n + k)
        A = (torch.rand(m * k, device="cuda", generator=g) * 2 - 1).to(tdt)
        B = (torch.rand(k * n, device="cuda", generator=g) * 2 - 1).to(tdt)
        C = torch.zeros(m * n, device="cuda", dtype=tdt)
        a_row, b_row = layout in (0, 1), layout in (0, 2)
        d = sk.make_desc(m, n, k, 1.0, A, k if a_row else m, B, n if b_row else k, 0.0, C, n, dt, layout)
        p = sk.plan_query(d)
        opts = sk.make_options()
        us = min(_gpu_time_us(torch, sk, d, opts, spin, reps) for _ in range(3))
        # the same operands as torch tensors (row-major views or transposed ones)
        Am = A.view(m, k) if a_row else A.view(k, m).t()
        Bm = B.view(k, n) if b_row else B.view(n, k).t()
        torch.matmul(Am, Bm)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda._sleep(spin)
        for e0, e1 in ev:
            e0.record()
            torch.matmul(Am, Bm)
            e1.record()
        torch.cuda.synchronize()
        lib_us = statistics.median(e0.elapsed_time(e1) for e0, e1 in ev) * 1e3
        by = es * (m * k + k * n + m * n)
        out.append({"shape": [m, n, k], "dtype": name, "layout": ["A row, B row", "A row, B col", "A col, B row",
                                                                  "A col, B col"][layout],
                    "form": ("tiled" if p.schedule != sk.SCHED_GEMV_SPLIT else
                             "multi" if p.tile_m > 0 else ("axpy" if p.tile_n > 0 else "dot")),
                    "schedule": int(p.schedule),
                    "chunks": int(p.sk_blocks), "grid": int(p.grid), "us": round(us, 2),
                    "GB_s": round(by / us / 1e3, 1), "frac_hbm": round(by / us / 1e3 / PEAK_HBM_GBS, 4),
                    "torch_matmul_us": round(lib_us, 2)})
        del A, B, C
    return out


def skinny_shapes(S, count=8, min_tmin_us=20.0):
    """The first `count` skinny shapes of the fp16 Stream-K sweep (m in
    [128, 256], k in [8192, 16384]) whose roofline time is at least
    `min_tmin_us`, so that the launch's fixed cost does not decide them."""
    out = []
    for kind, m, n, k in S.sweep_shapes(2000, S.SEED_SWEEP):
        if kind != "skinny":
            continue
        tmin = max(2.0 * m * n * k / (PEAK_TFLOPS["f16"] * 1e6), 2.0 * (m * k + k * n + m * n) / (PEAK_HBM_GBS * 1e3))
        if tmin >= min_tmin_us:
            out.append((m, n, k))
        if len(out) == count:
            break
    return out


def skinny_leg(torch, sk, S, min_ms=20.0):
    """Skinny fp16 GEMMs (A row-major, B column-major, alpha=1, beta=0) under
    AUTO, on the narrow-m tile (Stream-K, XCD-aware split) and data-parallel
    on the 256x256 tile, on each tile instance forced (AUTO's schedule), and
    under AUTO and each forced instance with the same B buffer taken as
    row-major (n-contiguous: `x @ W` with W stored k x n), each timed as R
    launches back to back between one event pair (at least `min_ms` per
    measurement, host enqueue hidden behind a spin kernel).  Bytes =
    2(mk + kn + mn), read and written once each."""
    out = []
    g = torch.Generator(device="cuda")
    g.manual_seed(S.SEED_SWEEP)
    for m, n, k in skinny_shapes(S):
        A = (torch.randn(m * k, generator=g, device="cuda") / math.sqrt(k)).to(torch.float16)
        B = torch.randn(k * n, generator=g, device="cuda").to(torch.float16)
        C = torch.empty(m * n, device="cuda", dtype=torch.float16)
        d = sk.make_desc(m, n, k, 1.0, A, k, B, k, 0.0, C, n, sk.F16, sk.A_ROW_B_COL)
        d_brow = sk.make_desc(m, n, k, 1.0, A, k, B, n, 0.0, C, n, sk.F16, sk.A_ROW_B_ROW)
        by = 2.0 * (m * k + k * n + m * n)
        fl = 2.0 * m * n * k
        tmin = max(fl / (PEAK_TFLOPS["f16"] * 1e6), by / (PEAK_HBM_GBS * 1e3))
        row = {"shape": [m, n, k], "bytes": int(by), "tmin_us": round(tmin, 2)}
        for name, dd, opts in (("auto", d, sk.make_options()),
                               ("narrow", d, sk.make_options(tile=sk.TILE_NARROW)),
                               ("dp", d, sk.make_options(schedule=sk.SCHED_DP, tile=sk.TILE_LARGE)),
                               ("large", d, sk.make_options(tile=sk.TILE_LARGE)),
                               ("small", d, sk.make_options(tile=sk.TILE_SMALL)),
                               ("auto_b_row", d_brow, sk.make_options()),
                               ("large_b_row", d_brow, sk.make_options(tile=sk.TILE_LARGE)),
                               ("small_b_row", d_brow, sk.make_options(tile=sk.TILE_SMALL))):
            us, R, _ = back_to_back_us(torch, lambda: sk.gemm_ex(dd, opts), min_ms=min_ms)
            p = sk.plan_query(dd, opts)
            row[name] = {"us": round(us, 2), "GB_s": round(by / us / 1e3, 1), "tflops": round(fl / us / 1e6, 1),
                         "util": round(tmin / us, 4), "tile": [int(p.tile_m), int(p.tile_n)], "grid": int(p.grid),
                         "schedule": int(p.schedule), "packs": int(p.packs), "launches": R}
        out.append(row)
        del A, B, C
    return out


def measured_peaks(torch, sk, reps=5):
    """The machine's own sustained rates (libskmb.so, include/sk_microbench.h):
    MFMA issue rate per type with two waves on every SIMD (8 independent MFMAs
    per round, 20000 rounds per launch), the HBM read rate of a 4 GiB buffer
    and the LDS read rate with eight waves per CU (16-byte and transposing
    8-byte reads); each the best of `reps` launches after two warm-up
    launches, HIP events on the launch stream."""
    import ctypes
    mb = ctypes.CDLL(os.path.join(os.path.dirname(sk.LIB_PATH), "libskmb.so"))
    mb.skmb_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    mb.skmb_mfma.restype = ctypes.c_int
    mb.skmb_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    mb.skmb_read.restype = ctypes.c_int
    mb.skmb_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    mb.skmb_lds.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def best_ms(launch):
        for _ in range(2):
            assert launch() == 0
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            assert launch() == 0
            e1.record(stream)
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return min(out)

    res = {}
    grid, rounds = 2 * cus, 20000
    sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    for dt, name, fl in ((0, "f32", 2048), (1, "f16", 32768), (2, "bf16", 32768)):
        ms = best_ms(lambda: mb.skmb_mfma(dt, rounds, grid, ctypes.c_void_p(sink.data_ptr()), sp))
        res[f"mfma_{name}_tflops"] = round(grid * 4 * rounds * 8 * fl / (ms * 1e-3) / 1e12, 1)
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    rgrid = 16 * cus
    rsink = torch.empty(rgrid * 256, dtype=torch.int32, device="cuda")
    ms = best_ms(lambda: mb.skmb_read(ctypes.c_void_p(buf.data_ptr()), nbytes, rgrid,
                                      ctypes.c_void_p(rsink.data_ptr()), sp))
    res["hbm_read_GB_s"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    # LDS read rate, eight waves per CU: 16-byte reads and 8-byte transposing
    # reads; per CU in bytes per nanosecond (bytes per clock = that / GHz)
    # (and per clock, at the core clock sampled while the same launches repeat)
    lrounds = 20000
    for mode, name, per in ((0, "lds_read", 1024), (1, "lds_tr_read", 512)):
        launch = lambda: mb.skmb_lds(mode, lrounds, grid, ctypes.c_void_p(rsink.data_ptr()), sp)  # noqa: E731
        ms = best_ms(launch)
        tot = grid * 4 * lrounds * 8 * per
        res[f"{name}_TB_s"] = round(tot / (ms * 1e-3) / 1e12, 1)
        res[f"{name}_B_per_ns_per_cu"] = round(tot / (ms * 1e-3) / 1e9 / cus, 1)
        clk = sample_clock(torch, lambda _: launch())
        if clk:
            res[f"{name}_clock_mhz"] = clk["median"]
            res[f"{name}_B_per_clk_per_cu"] = round(tot / (ms * 1e-3) / cus / (clk["median"] * 1e6), 1)
    del buf
    torch.cuda.empty_cache()
    return res


def _gpu_time_us(torch, sk, d, opts, spin, reps=7):
    """Median of `reps` launches, each between its own HIP events, queued
    behind a spin kernel (so the host's launch cost is not timed)."""
    import statistics
    sk.gemm_ex(d, opts)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda._sleep(spin)
    for e0, e1 in ev:
        e0.record()
        sk.gemm_ex(d, opts)
        e1.record()
    torch.cuda.synchronize()
    return statistics.median(e0.elapsed_time(e1) for e0, e1 in ev) * 1e3


def calibrate_model(torch, sk, S, n_shapes):
    """The runtime model T(g) = a + b [split] + c ipc(g) + d (peers) of the
    page's grid-size section, measured on this GPU.  Per element type, one
    tile on one workgroup: T(ipt) = a + c ipt (least squares over ipt = 1 ..
    256) gives a and c; one tile of 32 iterations split over g = 2 .. 32
    workgroups by basic Stream-K (the owner adds g - 1 partials in a row)
    gives b (one partial stored) and d (one partial added).  Constants are
    reported in microseconds and in units of c.  Then, on fp16 sweep shapes
    with fewer tiles than slots, basic Stream-K at the model's grid (library
    defaults, and the measured constants) against the best of an exhaustive
    set of grids."""
    import numpy as np
    spin = _spin_cycles(torch, 400e-6)
    out = {"calibration": "runtime model"}
    consts = {}
    for dt, tile, name in ((sk.F16, sk.TILE_LARGE, "f16"), (sk.F16, sk.TILE_SMALL, "f16_small"),
                           (sk.F32, sk.TILE_AUTO, "f32")):
        topt = sk.make_options(tile=tile)
        probe = sk.plan_query(sk.make_desc(256, 256, 256, 1.0, 0, 256, 0, 256, 0.0, 0, 256, dt, sk.A_ROW_B_COL),
                              topt)
        bm, bk = probe.tile_m, probe.tile_k
        tdt = torch.float16 if dt == sk.F16 else torch.float32
        kmax = 256 * bk
        A = torch.randn(bm * kmax, device="cuda").to(tdt)
        B = torch.randn(bm * kmax, device="cuda").to(tdt)
        C = torch.zeros(bm * bm, device="cuda", dtype=tdt)
        ipts = [1, 2, 4, 8, 16, 32, 64, 128, 256]
        ts = []
        for ipt in ipts:
            d = sk.make_desc(bm, bm, ipt * bk, 1.0, A, ipt * bk, B, ipt * bk, 0.0, C, bm, dt, sk.A_ROW_B_COL)
            ts.append(_gpu_time_us(torch, sk, d, sk.make_options(schedule=sk.SCHED_DP, tile=tile), spin))
        c_us, a_us = np.polyfit(np.array(ipts, float), np.array(ts), 1)
        gs = [2, 3, 4, 8, 16, 32]
        d = sk.make_desc(bm, bm, 32 * bk, 1.0, A, 32 * bk, B, 32 * bk, 0.0, C, bm, dt, sk.A_ROW_B_COL)
        rows, rhs = [], []
        split_t = {}
        for g in gs:
            t = _gpu_time_us(torch, sk, d, sk.make_options(schedule=sk.SCHED_SK_BASIC, forced_grid=g, tile=tile),
                             spin)
            split_t[g] = round(t, 2)
            rows.append([1.0, g - 1.0])
            rhs.append(t - a_us - c_us * -(-32 // g))
        (b_us, d_us), *_ = np.linalg.lstsq(np.array(rows), np.array(rhs), rcond=None)
        consts[name] = (a_us / c_us, b_us / c_us, 1.0, d_us / c_us)
        out[name] = {"tile": bm, "bk": bk, "single_tile_us": dict(zip(ipts, [round(x, 2) for x in ts])),
                     "split_32_iterations_us": split_t,
                     "us": {"a": round(a_us, 2), "b": round(b_us, 2), "c": round(c_us, 3), "d": round(d_us, 2)},
                     "units_of_c": {k: round(v, 2) for k, v in zip("abcd", consts[name])}}
        del A, B, C
    # exhaustive grid search on fp16 shapes below one wave
    probe = sk.plan_query(sk.make_desc(256, 256, 256, 1.0, 0, 256, 0, 256, 0.0, 0, 256, sk.F16, sk.A_ROW_B_COL))
    shapes = [sh for sh in S.sweep_shapes(2000, S.SEED_SWEEP, probe.tile_m, probe.tile_n, probe.slots)
              if sh[0] == "random"]
    chosen = []
    for kind, m, n, k in shapes:
        t = -(-m // probe.tile_m) * -(-n // probe.tile_n)
        if t < probe.slots and -(-k // 64) >= 16 and 2 * m * n * k >= 2e10:
            chosen.append((m, n, k))
        if len(chosen) == n_shapes:
            break
    mx = max(max(m * k, k * n, m * n) for m, n, k in chosen)
    A = torch.randn(mx, device="cuda").to(torch.float16)
    B = torch.randn(mx, device="cuda").to(torch.float16)
    C = torch.zeros(mx, device="cuda", dtype=torch.float16)
    regrets = {"default": [], "measured": [], "auto": []}
    per_shape = []
    for m, n, k in chosen:
        d = sk.make_desc(m, n, k, 1.0, A, k, B, k, 0.0, C, n, sk.F16, sk.A_ROW_B_COL)
        p = sk.plan_query(d, sk.make_options(tile=sk.TILE_LARGE))
        t, slots = p.tiles, p.slots
        large = sk.TILE_LARGE
        grid_default = sk.plan_query(d, sk.make_options(schedule=sk.SCHED_SK_BASIC, tile=large)).grid
        grid_measured = sk.plan_query(d, sk.make_options(schedule=sk.SCHED_SK_BASIC, tile=large,
                                                         model=consts["f16"])).grid
        cands = sorted({g for g in [t * s for s in range(1, 9)] + [slots, grid_default, grid_measured]
                        if t <= g <= slots})
        times = {g: _gpu_time_us(torch, sk, d, sk.make_options(schedule=sk.SCHED_SK_BASIC, forced_grid=g,
                                                                 tile=large), spin)
                 for g in cands}
        best = min(times.values())
        t_auto = _gpu_time_us(torch, sk, d, sk.make_options(tile=large), spin)
        regrets["default"].append(times[grid_default] / best)
        regrets["measured"].append(times[grid_measured] / best)
        regrets["auto"].append(t_auto / best)
        per_shape.append({"shape": [m, n, k], "tiles": t, "best_g": min(times, key=times.get),
                          "best_us": round(best, 1), "g_default": grid_default, "g_measured": grid_measured,
                          "auto_us": round(t_auto, 1)})
    out["grid_search"] = {
        "shapes": len(chosen),
        "basic_sk_time_over_best": {k: {"geomean": round(float(np.exp(np.mean(np.log(v)))), 4),
                                        "max": round(float(max(v)), 3)} for k, v in regrets.items() if v},
        "per_shape": per_shape}
    return out


def calibrate_copy(torch):
    n = (1 << 30) // 4  # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_dispatch": 1 << 30,
                      "bytes_written_per_dispatch": 1 << 30, "dispatches": 5}), flush=True)


def make_sweep_inputs(torch, sk, S):
    cases = []
    for n in SWEEP:
        A = S.matrix(S.SEED_SGEMM_SQUARE, S.STREAM_A, n, n, S.F32)
        B = S.matrix(S.SEED_SGEMM_SQUARE, S.STREAM_B, n, n, S.F32)
        C = S.matrix(S.SEED_SGEMM_SQUARE, S.STREAM_C, n, n, S.F32)
        cases.append(dict(n=n, host=(A, B, C), A=torch.from_numpy(A).cuda(),
                          B=torch.from_numpy(B).cuda(), C=torch.from_numpy(C).cuda()))
    return cases


def make_hgemm_inputs(torch, sk, S, dtype):
    import numpy as np
    n = 8192
    tdt = torch.float16 if dtype == sk.F16 else torch.bfloat16
    A = S.matrix(S.SEED_HGEMM_LARGE, S.STREAM_A, n, n, dtype, "normal", "row", None, 1 / math.sqrt(n))
    B = S.matrix(S.SEED_HGEMM_LARGE, S.STREAM_B, n, n, dtype, "normal", "col", None, 1 / math.sqrt(n))
    dA = torch.from_numpy(A.view(np.int16)).view(tdt).cuda()
    dB = torch.from_numpy(B.view(np.int16)).view(tdt).cuda()
    dC = torch.zeros(n * n, dtype=tdt, device="cuda")
    return dict(n=n, dtype=dtype, A=dA, B=dB, C=dC)


def sweep_step(sk, cases, events=None):
    for i, c in enumerate(cases):
        n = c["n"]
        if events is not None:
            events[i][0].record()
        sk.gemm(n, n, n, 1.0, c["A"], n, c["B"], n, 1.0, c["C"], n, sk.F32, sk.A_ROW_B_ROW)
        if events is not None:
            events[i][1].record()


def hgemm_step(sk, h, events=None):
    n = h["n"]
    if events is not None:
        events[0][0].record()
    sk.gemm(n, n, n, 1.0, h["A"], n, h["B"], n, 0.0, h["C"], n, h["dtype"], sk.A_ROW_B_COL)
    if events is not None:
        events[0][1].record()


def timed(torch, step, n_launch, steps, warmup):
    """Runs warmup + timed steps; returns (ms per step, mean ms per launch
    for each launch index of the step)."""
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_launch)] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for s in range(steps):
        step(ev[s])
    t1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - wall0) * 1e3
    total_ms = t0.elapsed_time(t1)
    per_launch = [sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)) / steps
                  for i in range(n_launch)]
    return max(total_ms, 0.0) / steps, per_launch, wall / steps


def abft_overhead(torch, sk, S, steps=10):
    """4096^3 fp32 GEMM (row-major, U[-1,1], alpha=1, beta=0) with and without
    ABFT (no faults), each timed over `steps` launches, best of three rounds."""
    import ctypes
    n = 4096
    A = torch.from_numpy(S.matrix(S.SEED_ABFT, S.STREAM_A, n, n, S.F32)).cuda()
    B = torch.from_numpy(S.matrix(S.SEED_ABFT, S.STREAM_B, n, n, S.F32)).cuda()
    C = torch.zeros(n * n, dtype=torch.float32, device="cuda")
    rep = torch.zeros(ctypes.sizeof(sk.AbftReport), dtype=torch.uint8, device="cuda")
    d = sk.make_desc(n, n, n, 1.0, A, n, B, n, 0.0, C, n, sk.F32, sk.A_ROW_B_ROW)
    out = {}
    best = {}
    # three rounds, the two legs alternating, three warm-up launches before
    # each timed run; the best run of each leg (a leg timed first after other
    # work otherwise runs at a lower clock and flatters the ratio)
    for _ in range(3):
        for name, opts in (("plain", sk.make_options()), ("abft", sk.make_options(abft=True))):
            def one():
                sk.gemm_ex(d, opts, rep if name == "abft" else None)
            for _ in range(3):
                one()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                one()
            e1.record()
            torch.cuda.synchronize()
            best[name] = min(best.get(name, 1e30), e0.elapsed_time(e1) / steps)
    for name, ms in best.items():
        out[name] = {"ms": round(ms, 4), "tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 2)}
    r = sk.read_report(rep)
    out["overhead"] = round(out["abft"]["ms"] / out["plain"]["ms"] - 1.0, 4)
    out["false_positives"] = int(r.detected)
    out["config"] = "fp32 4096^3 row-major U[-1,1], alpha=1 beta=0, no faults injected"
    return out


def _spin_cycles(torch, seconds):
    """Argument of torch.cuda._sleep that keeps the GPU busy for about
    `seconds` (calibrated on a 1e6-cycle spin)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1000)
    e0.record()
    torch.cuda._sleep(1000000)
    e1.record()
    torch.cuda.synchronize()
    per_cycle = e0.elapsed_time(e1) * 1e-3 / 1e6
    return max(1000, int(seconds / per_cycle))


def _spin_for(torch, seconds, _cache={}):
    """Queues a spin kernel that keeps the GPU busy for about `seconds`."""
    if "per_cycle" not in _cache:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record()
        torch.cuda._sleep(1000000)
        e1.record()
        torch.cuda.synchronize()
        _cache["per_cycle"] = e0.elapsed_time(e1) * 1e-3 / 1e6
    torch.cuda._sleep(max(1000, int(seconds / _cache["per_cycle"])))


def back_to_back_us(torch, launch, min_ms=20.0, max_launches=4096):
    """Mean time of one launch, from R launches timed back to back between
    one pair of HIP events, R chosen so that the measurement spans at least
    `min_ms` (at least 5 launches).  A spin kernel queued ahead keeps the GPU
    busy while the host enqueues the R launches, so they run back to back on
    the GPU and the host's cost of a call (planning, argument marshalling)
    is not charged to the kernel.  Returns (microseconds, R, host
    microseconds per call)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    host = []
    for _ in range(3):  # warm-up (plan cache, clocks), and the host's cost of a call
        h0 = time.perf_counter()
        launch()
        host.append(time.perf_counter() - h0)
    torch.cuda.synchronize()
    h = min(host)
    _spin_for(torch, 4 * h + 2e-4)
    e0.record()
    launch()
    e1.record()
    torch.cuda.synchronize()
    t1 = max(e0.elapsed_time(e1), 1e-4)  # ms
    R = int(min(max_launches, max(5, math.ceil(min_ms / t1))))
    spin_s = 1.3 * R * h + 5e-4
    _spin_for(torch, spin_s)
    e0.record()
    h0 = time.perf_counter()
    for _ in range(R):
        launch()
    enq = time.perf_counter() - h0
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / R
    # the launches ran back to back on the GPU only if the host had queued
    # them all before the spin ended (a full queue would block the host)
    back_to_back_us.last = {"enqueue_ms": enq * 1e3, "spin_ms": spin_s * 1e3, "host_bound": enq > spin_s}
    return us, R, h * 1e6


def sweep_subset(S, count, tile_m=256, tile_n=256, slots=256):
    """`count` shapes of the seeded 2000-shape Stream-K sweep in its
    proportions (3/4 random, 1/8 skinny, 1/8 tile-count adversarial): every
    (2000/count)-th shape of the list, which holds the kinds in that order."""
    shapes = S.sweep_shapes(2000, S.SEED_SWEEP, tile_m, tile_n, slots)
    if count >= len(shapes):
        return shapes
    return [shapes[int(i * len(shapes) / count)] for i in range(count)]


def sweep_legs(sk, names, page_sched):
    """Options of each named leg (the schedule of the same kernels)."""
    L = sk.TILE_LARGE
    table = {
        "auto": sk.make_options(),
        "dp": sk.make_options(schedule=sk.SCHED_DP, tile=L),
        "page": sk.make_options(schedule=page_sched, tile=L),
        "large": sk.make_options(tile=L),
        "small": sk.make_options(tile=sk.TILE_SMALL),
        "basic": sk.make_options(schedule=sk.SCHED_SK_BASIC, tile=L),
        "hybrid2": sk.make_options(schedule=sk.SCHED_SK_HYBRID2, tile=L),
        "hybrid2_w2": sk.make_options(schedule=sk.SCHED_SK_HYBRID2, tile=L, hybrid_min_waves=2),
        "hybrid1": sk.make_options(schedule=sk.SCHED_SK_HYBRID1, tile=L),
        "xcd_w2": sk.make_options(schedule=sk.SCHED_XCD_ALIGNED, tile=L, hybrid_min_waves=2),
    }
    return [(n, table[n]) for n in names]


def shape_sweep(torch, sk, S, count, out_path="", legs=("auto", "dp"), min_ms=20.0):
    """Stream-K shape sweep: fp16 GEMMs (A row-major, B column-major, both
    contiguous along k; alpha=1, beta=0) on `count` shapes of the seeded
    sweep list (sweep_subset), each run under the named schedules of the
    same kernels ("dp": data-parallel on the large tile, the baseline).

    Per shape and leg: back_to_back_us (R launches back to back, at least
    20 ms per measurement).  Roofline time T_min = max(2mnk / P_fp16,
    2(mk + kn + mn) / BW_HBM); utilisation = T_min / T.  Inputs:
    N(0,1)-scaled normal values drawn on the GPU from a generator seeded with
    the sweep seed (timing only; parity of sweep shapes is in the tests)."""
    import statistics
    probe = sk.make_desc(256, 256, 256, 1.0, 0, 256, 0, 256, 0.0, 0, 256, sk.F16, sk.A_ROW_B_COL)
    tile = sk.plan_query(probe, sk.make_options(tile=sk.TILE_LARGE))
    shapes = sweep_subset(S, count, tile.tile_m, tile.tile_n, tile.slots)
    mx = max(max(m * k, k * n, m * n) for _, m, n, k in shapes)
    g = torch.Generator(device="cuda")
    g.manual_seed(S.SEED_SWEEP)
    A = torch.randn(mx, generator=g, device="cuda", dtype=torch.float32).to(torch.float16)
    B = torch.randn(mx, generator=g, device="cuda", dtype=torch.float32).to(torch.float16)
    C = torch.empty(mx, device="cuda", dtype=torch.float16)
    peak, bw = PEAK_TFLOPS["f16"] * 1e12, PEAK_HBM_GBS * 1e9
    rows = []
    for idx, (kind, m, n, k) in enumerate(shapes):
        d = sk.make_desc(m, n, k, 1.0, A, k, B, k, 0.0, C, n, sk.F16, sk.A_ROW_B_COL)
        pl = sk.plan_query(d, sk.make_options(tile=sk.TILE_LARGE))
        t, slots = pl.tiles, pl.slots
        w, r = divmod(t, slots)
        page = sk.SCHED_DP if r == 0 else sk.SCHED_SK_HYBRID2 if w >= 1 else sk.SCHED_SK_BASIC
        lg = sweep_legs(sk, legs, page)
        # rotate the order per shape so that clock ramps do not favour one leg
        lg = lg[idx % len(lg):] + lg[:idx % len(lg)]
        fl = 2.0 * m * n * k
        by = 2.0 * (m * k + k * n + m * n)
        tmin = max(fl / peak, by / bw)
        row = dict(kind=kind, m=m, n=n, k=k, tiles=t, waves=w, tail=r, tmin_us=tmin * 1e6,
                   mem_bound=int(by / bw > fl / peak), dp_quant_eff=t / (slots * -(-t // slots)))
        for name, opts in lg:
            us, R, host_us = back_to_back_us(torch, lambda: sk.gemm_ex(d, opts), min_ms)
            row[f"err_{name}"] = _sampled_check(torch, A, B, C, m, n, k, idx)
            pq = sk.plan_query(d, opts)
            row[f"t_{name}_us"] = us
            row[f"launches_{name}"] = R
            row[f"host_{name}_us"] = host_us
            row[f"util_{name}"] = tmin * 1e6 / us
            row[f"tflops_{name}"] = fl / (us * 1e-6) / 1e12
            row[f"schedule_{name}"] = pq.schedule
            row[f"tile_{name}"] = pq.tile_m
            row[f"enqueue_ms_{name}"] = back_to_back_us.last["enqueue_ms"]
            row[f"spin_ms_{name}"] = back_to_back_us.last["spin_ms"]
            row[f"host_bound_{name}"] = int(back_to_back_us.last["host_bound"])
        rows.append(row)
        if idx % 50 == 0:
            print(f"sweep {idx}/{len(shapes)}", file=sys.stderr, flush=True)
    if out_path:
        with open(out_path, "w") as f:
            keys = list(rows[0].keys())
            f.write(",".join(keys) + "\n")
            for r in rows:
                f.write(",".join(f"{r[k]:.6g}" if isinstance(r[k], float) else str(r[k]) for k in keys) + "\n")
    return sweep_summary(rows, legs)


def _sampled_check(torch, A, B, C, m, n, k, seed, count=64):
    """The timed launches' result on `count` seeded entries against fp32
    dot products of the same fp16 inputs on the GPU (torch, not this
    library): max |C_ij - ref_ij| / sum_l |a_il||b_lj|."""
    g = torch.Generator(device="cuda")
    g.manual_seed(1000003 + seed)
    ii = torch.randint(0, m, (count,), generator=g, device="cuda")
    jj = torch.randint(0, n, (count,), generator=g, device="cuda")
    a = A[: m * k].view(m, k)[ii].float()
    b = B[: n * k].view(n, k)[jj].float()
    ref = (a * b).sum(1)
    bound = (a.abs() * b.abs()).sum(1).clamp_min(1e-30)
    got = C[: m * n].view(m, n)[ii, jj].float()
    return float(((got - ref).abs() / bound).max())


def sweep_summary(rows, legs):
    import statistics

    def cv(xs):
        mu = statistics.fmean(xs)
        return statistics.pstdev(xs) / mu if mu > 0 else float("nan")

    def summary(sel):
        if not sel:
            return None
        out = {"shapes": len(sel)}
        for name in legs:
            if name == "dp" or "dp" not in legs:
                continue
            sp = [r["t_dp_us"] / r[f"t_{name}_us"] for r in sel]
            out[f"{name}_over_dp"] = {
                "geomean": round(math.exp(statistics.fmean(math.log(x) for x in sp)), 4),
                "median": round(statistics.median(sp), 4), "min": round(min(sp), 3),
                "max": round(max(sp), 3), "frac_not_slower": round(sum(x >= 0.98 for x in sp) / len(sp), 4)}
        for name in legs:
            u = [r[f"util_{name}"] for r in sel]
            us = sorted(u)
            out[f"util_{name}"] = {"mean": round(statistics.fmean(u), 4), "cv": round(cv(u), 4),
                                   "p5_p95": [round(us[int(0.05 * (len(us) - 1))], 4),
                                              round(us[int(0.95 * (len(us) - 1))], 4)]}
        if "auto" in legs:
            out["host_call_us_median"] = round(statistics.median(r["host_auto_us"] for r in sel), 2)
        out["host_bound_measurements"] = sum(r[f"host_bound_{name}"] for r in sel for name in legs)
        return out

    classes = {
        "all": rows,
        "compute_bound": [r for r in rows if not r["mem_bound"]],
        "memory_bound": [r for r in rows if r["mem_bound"]],
        "random": [r for r in rows if r["kind"] == "random"],
        "skinny": [r for r in rows if r["kind"] == "skinny"],
        "adversarial": [r for r in rows if r["kind"] == "adversarial"],
        # by the roofline time: below 10 us the fixed cost of a launch dominates
        "tmin_lt_10us": [r for r in rows if r["tmin_us"] < 10.0],
        "tmin_10_100us": [r for r in rows if 10.0 <= r["tmin_us"] < 100.0],
        "tmin_ge_100us": [r for r in rows if r["tmin_us"] >= 100.0],
        "compute_bound_tmin_ge_100us": [r for r in rows if not r["mem_bound"] and r["tmin_us"] >= 100.0],
        # full waves of large tiles: the page's hybrids differ only from one wave on
        "waves_0": [r for r in rows if r["waves"] == 0],
        "waves_1_tail": [r for r in rows if r["waves"] == 1 and r["tail"] > 0],
        "waves_2plus_tail": [r for r in rows if r["waves"] >= 2 and r["tail"] > 0],
    }
    return {"workload": "Stream-K shape sweep, fp16, A row-major / B column-major, alpha=1 beta=0; "
                        f"{len(rows)} shapes of the seeded 2000-shape list in its proportions",
            "timing": "R launches back to back between one event pair, >= 20 ms per measurement",
            "legs": list(legs),
            "roofline": {"peak_tflops": PEAK_TFLOPS["f16"], "hbm_tb_s": PEAK_HBM_GBS / 1000,
                         "t_min": "max(2mnk/peak, 2(mk+kn+mn)/bw)"},
            # every timed leg's result, 64 seeded entries per shape against
            # fp32 dot products of the same inputs (torch), error / bound
            "result_check": {"entries": 64 * len(rows) * len(legs),
                             "max_err": max(r[f"err_{name}"] for r in rows for name in legs),
                             "gate": 5e-3,
                             "failed": sum(r[f"err_{name}"] > 5e-3 for r in rows for name in legs)},
            "classes": {name: summary(sel) for name, sel in classes.items()}}


def _sclk_path():
    """The driver's core-clock file of the GPU (the clock rocm-smi
    --showclocks reports), or None."""
    import glob
    for path in sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")):
        try:
            with open(path) as f:
                if "*" in f.read():
                    return path
        except OSError:
            continue
    return None


def _read_sclk(path):
    try:
        with open(path) as f:
            for line in f:
                if "*" in line:
                    return float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0])
    except (OSError, ValueError, IndexError):
        return None
    return None


def sample_clock(torch, step, seconds=0.3, interval=0.004):
    """Core clock while the workload runs: `step` repeated for about
    `seconds` after the timed region (so the sampling thread cannot perturb
    the timing), the clock read every `interval` seconds from the driver."""
    import statistics
    import threading
    path = _sclk_path()
    if path is None:
        return None
    samples, stop = [], threading.Event()

    def run():
        while not stop.is_set():
            v = _read_sclk(path)
            if v:
                samples.append(v)
            time.sleep(interval)

    step(None)
    torch.cuda.synchronize()
    th = threading.Thread(target=run, daemon=True)
    th.start()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        step(None)
        torch.cuda.synchronize()
    stop.set()
    th.join()
    if not samples:
        return None
    return {"min": min(samples), "median": statistics.median(samples), "max": max(samples),
            "samples": len(samples), "source": "pp_dpm_sclk (as rocm-smi --showclocks), repeated steps"}


def cpu_baseline(S, budget_s=25.0):
    """The oracle (six-loop fp64 GEMM, full output) on the fp32 sweep's
    shapes, smallest first, on the host's cores, stopping once about
    `budget_s` seconds of CPU work have been spent."""
    import oracle
    flops, secs = 0.0, 0.0
    sample = []
    prev, last_t = None, 0.0
    for n in SWEEP:
        if prev is not None and secs + last_t * (n / prev) ** 3 > budget_s:
            break
        A = S.matrix(S.SEED_SGEMM_SQUARE, S.STREAM_A, n, n, S.F32)
        B = S.matrix(S.SEED_SGEMM_SQUARE, S.STREAM_B, n, n, S.F32)
        C = S.matrix(S.SEED_SGEMM_SQUARE, S.STREAM_C, n, n, S.F32)
        t0 = time.perf_counter()
        oracle.gemm(n, n, n, 1.0, A, n, B, n, 1.0, C, n, oracle.F32, oracle.A_ROW_B_ROW)
        last_t = time.perf_counter() - t0
        secs += last_t
        prev = n
        flops += 2.0 * n ** 3
        sample.append(f"{n}^3")
    return {"value": round(flops / secs / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "full oracle (fp64 six-loop, alpha=1 beta=1) on the " + ", ".join(sample) +
                      " shapes of the fp32 square sweep; " + f"{secs:.1f} s of CPU work"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this path has no "
              "multi-GPU mode: run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import sk_synth as S
    import work_centric_decomposition_amd as sk
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(3)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(torch)
        return
    if args.sweep:
        print(json.dumps(shape_sweep(torch, sk, S, args.sweep, args.sweep_out,
                                     legs=tuple(args.sweep_legs.split(",")))), flush=True)
        return
    if args.calibrate_model:
        print(json.dumps(calibrate_model(torch, sk, S, args.calibrate_model)), flush=True)
        return
    if args.library_gemm:
        for r in library_gemm(torch, sk, S, args.steps, args.warmup):
            print(json.dumps(r), flush=True)
        return
    if args.gemv:
        print(json.dumps(gemv_leg(torch, sk, S)), flush=True)
        return
    if args.layouts:
        for r in layouts_leg(torch, sk, S, args.steps):
            print(json.dumps(r), flush=True)
        return
    if args.peaks:
        print(json.dumps(measured_peaks(torch, sk)), flush=True)
        return
    if args.abft:
        print(json.dumps(abft_overhead(torch, sk, S, steps=args.steps)), flush=True)
        return
    if args.skinny:
        # (--steps below 5: five launches per leg, for counter runs)
        for r in skinny_leg(torch, sk, S, min_ms=20.0 if args.steps >= 5 else 0.0):
            print(json.dumps(r), flush=True)
        return
    if args.compare_schedules:
        for r in compare_schedules(torch, sk, S, args.steps):
            print(json.dumps(r), flush=True)
        return

    results = {}
    order = [args.workload] + ([] if args.no_extra else
                               [w for w in ("sgemm-sweep", "hgemm-8192") if w != args.workload])
    for wl in order:
        main_wl = wl == args.workload
        # the clock needs tens of ms of load to settle: extra legs get 30 warm-up steps
        steps = args.steps if main_wl else max(10, args.steps // 2)
        warmup = args.warmup if main_wl else 30
        if wl == "sgemm-sweep":
            cases = make_sweep_inputs(torch, sk, S)
            ms, per_launch, wall = timed(torch, lambda ev: sweep_step(sk, cases, ev), len(cases),
                                         steps, warmup)
            flops = [2.0 * c["n"] ** 3 for c in cases]
            # algorithmic flops: 2mnk MACs plus the alpha/beta epilogue (3mn)
            step_flops = sum(2.0 * c["n"] ** 3 + 3.0 * c["n"] ** 2 for c in cases)
            kern_ms = sum(per_launch)
            achieved = sum(flops) / (kern_ms * 1e-3) / 1e12
            clock = sample_clock(torch, lambda ev: sweep_step(sk, cases, ev))
            tiles = {}
            for c in cases:  # the tile instance AUTO runs each shape on
                n = c["n"]
                d = sk.make_desc(n, n, n, 1.0, c["A"], n, c["B"], n, 1.0, c["C"], n, sk.F32, sk.A_ROW_B_ROW)
                p = sk.plan_query(d)
                tiles[str(n)] = f"{p.tile_m}x{p.tile_n}"
            results[wl] = dict(
                value=step_flops / (ms * 1e-3) / 1e12, ms=ms, wall_ms=wall, dtype="f32", clock=clock,
                per_shape={str(c["n"]): round(f / (t * 1e-3) / 1e12, 2)
                           for c, f, t in zip(cases, flops, per_launch)},
                roofline={"bound": "mfma", "achieved": round(achieved, 2),
                          "peak": PEAK_TFLOPS["f32"], "unit": "TFLOP/s",
                          "frac": round(achieved / PEAK_TFLOPS["f32"], 4),
                          "traffic": traffic_for(wl),
                          "kernel": "sgemm_kernel<k-major A, n-major B>",
                          "tile_per_shape": tiles,
                          "launch_ms": round(kern_ms / len(cases), 4)},
                config={"workload": "SGEMM fp32 square sweep m=n=k in {1024,2048,3072,4096,5120,6144},"
                                    " row-major A and B, U[-1,1] inputs, C pre-filled U[-1,1],"
                                    " alpha=1 beta=1", "shapes": SWEEP, "schedule": "AUTO"})
            del cases
        else:
            out = {}
            for dt, name in ((sk.F16, "f16"), (sk.BF16, "bf16")):
                h = make_hgemm_inputs(torch, sk, S, dt)
                ms, per_launch, wall = timed(torch, lambda ev: hgemm_step(sk, h, ev), 1, steps, warmup)
                clock = sample_clock(torch, lambda ev: hgemm_step(sk, h, ev))
                fl = 2.0 * 8192 ** 3
                achieved = fl / (per_launch[0] * 1e-3) / 1e12
                out[name] = dict(value=fl / (ms * 1e-3) / 1e12, ms=ms, wall_ms=wall, dtype=name, clock=clock,
                                 roofline={"bound": "mfma", "achieved": round(achieved, 2),
                                           "peak": PEAK_TFLOPS[name], "unit": "TFLOP/s",
                                           "frac": round(achieved / PEAK_TFLOPS[name], 4),
                                           # counters were taken on the fp16 launch only
                                           "traffic": traffic_for(wl if name == "f16" else wl + "-bf16"),
                                           "kernel": f"hgemm_kernel<{name}>",
                                           "launch_ms": round(per_launch[0], 4)})
                del h
                torch.cuda.empty_cache()
            r = out["f16"]
            r["bf16"] = {k: out["bf16"][k] for k in ("value", "ms", "roofline", "clock")} if "bf16" in out else None
            r["config"] = {"workload": "HGEMM 8192^3, fp16 in/out (bf16 also timed), fp32 accumulate,"
                                       " A row-major, B column-major, N(0,1)/sqrt(k), alpha=1 beta=0",
                           "schedule": "AUTO"}
            results[wl] = r
        torch.cuda.empty_cache()

    m = results[args.workload]
    line = {"metric": METRIC, "value": round(m["value"], 3), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(m["ms"], 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": m["dtype"], "data": "synthetic", "config": m["config"],
            "roofline": m["roofline"], "clock_mhz": m.get("clock")}
    if "per_shape" in m:
        line["per_shape_tflops"] = m["per_shape"]
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(S)
    if not args.no_extra and args.sweep_count > 0:
        line["sweep"] = shape_sweep(torch, sk, S, args.sweep_count)
    if not args.no_extra:
        line["abft"] = abft_overhead(torch, sk, S)
        line["gemv"] = gemv_leg(torch, sk, S)
        line["measured_peaks"] = measured_peaks(torch, sk)
    for wl, r in results.items():
        if wl == args.workload:
            continue
        extra = {"value": round(r["value"], 3), "unit": "TFLOP/s", "ms_per_step": round(r["ms"], 4),
                 "dtype": r["dtype"], "roofline": r["roofline"], "clock_mhz": r.get("clock"),
                 "config": r["config"]}
        if r.get("bf16"):
            extra["bf16"] = {"value": round(r["bf16"]["value"], 3), "roofline": r["bf16"]["roofline"],
                             "clock_mhz": r["bf16"].get("clock")}
        if "per_shape" in r:
            extra["per_shape_tflops"] = r["per_shape"]
        line["hgemm" if wl == "hgemm-8192" else "sgemm"] = extra
    if "measured_peaks" in line:
        # the same kernels' rates against what this chip sustains
        peaks = line["measured_peaks"]
        key = {"f32": "mfma_f32_tflops", "f16": "mfma_f16_tflops", "bf16": "mfma_bf16_tflops"}
        for obj in (line, line.get("sgemm"), line.get("hgemm"), (line.get("hgemm") or {}).get("bf16")):
            if obj and "roofline" in obj:
                rf = obj["roofline"]
                dt = "f32" if rf["peak"] == PEAK_TFLOPS["f32"] else ("bf16" if "bf16" in rf["kernel"] else "f16")
                rf["frac_of_measured"] = round(rf["achieved"] / peaks[key[dt]], 4)
        for g in line.get("gemv", []):
            g["frac_of_measured_hbm"] = round(g["GB_s"] / peaks["hbm_read_GB_s"], 4)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the bit-packed weight products on one MI355X.

Headline step: one ternary x int8 decode GEMV (M=1, K=4096, N=14336, group 128)
through bpw_gemv_packed, with its int8 activations (one fp32 scale per row)
already resident in HBM. Weight copies totalling >= 1 GiB are read as a ring
so each call streams its weights from HBM rather than the 256 MB Infinity
Cache. The K timed steps run as one captured HIP graph between HIP events on
the launch stream; the graph is timed 7 times (after an untimed replay, and
each time after a spin kernel that hides the host's submission and half a
ring of untimed calls) next to a one-call graph timed the same way, and the
median of (T(K) - T(1)) / (K - 1) is reported, with the spread: the
difference cancels the fixed cost of a graph replay and its events.
value = logical weight bytes (codes + scales) per call / time per call.

Also reported (same JSON line): the complete decode call from the fp32 row
(the quantiser fused into the GEMV launch, and the quantiser launch + GEMV),
the other decode/prefill workloads (ternary decode at M=16, split-K long K,
per-group activation scales and on the 62 MB prefill weight; 4-bit decode GEMV
with act order; bf16 prefill GEMM at M=2048; 4-bit x int8 prefill GEMM at
M=2048, with row scales and in the affine form (scale and exact sum per row
and weight group); ternary x int8 prefill GEMM with row scales and with
per-group scales; hipBLASLt dense GEMMs at the prefill
shapes as a platform reference), HBM read/copy probes, the roofline of the
dominant kernel (and its fraction of the read probe at the same byte count),
the engine clock sampled through amdsmi during each prefill leg (for the
clock-adjusted MFMA fraction), and the CPU oracle timed on bounded samples of
the headline and the other workloads, with the host's core count and model.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]
                       [--legs LEG,...|all|none] [--repeats R]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
PEAK_CLOCK_GHZ = 2.4        # engine clock of the published peaks
METRIC = "weight GB/s (% HBM peak) at M=1 GEMV; TFLOP/s (% MFMA peak) at M=2048"
# Hardware-counter summary of the dominant kernel (HBM bytes per launch from
# FETCH_SIZE and WRITE_SIZE, scaled by the copy probe), and the sources it was
# taken on: the figure is used only while those sources are unchanged.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_t2_row_ternary_decode_m1_traffic.md")
KERNEL_SOURCES = ("bit_packed_weight_amd/csrc/gemv.hip", "bit_packed_weight_amd/csrc/device.h")


def kernel_digest():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch of the decode GEMV from the committed counter summary, or None."""
    try:
        with open(TRAFFIC_FILE) as f:
            vals = dict(re.findall(r"^- (\w+): (\S+)\s*$", f.read(), re.M))
        if vals.get("source_digest") != kernel_digest():
            return None
        return float(vals["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(a, dtype, torch, np):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def rotated_copies(bpw, planes, min_bytes, max_copies=256):
    base = bpw.upload(planes)
    count = max(1, min(max_copies, math.ceil(min_bytes / base.logical_bytes)))
    copies = [base]
    for _ in range(count - 1):
        copies.append(bpw.PackedWeights(base.fmt, base.scale_dtype, base.n, base.k, base.codes.clone(),
                                         base.scales.clone(), None if base.zeros is None else base.zeros.clone(),
                                         None if base.perm is None else base.perm.clone()))
    return copies


REPEATS = 7
SPIN_CYCLES = 1_000_000     # torch's spin kernel (~0.4 ms): the GPU stays busy while the host submits a graph
LAST_SPREAD = {}


def time_calls(torch, call, ncopies, steps, warmup, repeats=None):
    """Median ms per call of `steps` calls captured in one HIP graph.

    call(c) launches one call that reads weight copy c. The copies form a ring
    read in order, and every timed graph is preceded by a flush graph of half a
    ring (>= 512 MB for a >= 1 GiB ring) that ends on the copy just before the
    timed graph's first one, so the 256 MB Infinity Cache holds none of the
    timed bytes when timing starts. Each timed graph runs after torch's spin
    kernel, so the host's submission of the graph is not timed, between two
    events on its stream.

    The spin kernel runs first, then the flush, then the timed graph, so the
    GPU goes straight from a half ring of the same calls into the timed ones.

    A graph replay bracketed by events costs a fixed ~12 us beyond its calls
    (graph boundary and event packets, measured: 20 calls per graph read
    5.42 us per call, 2070 read 4.79). So each repeat times the `steps`-call
    graph T_K and a one-call graph T_1 the same way, and the figure per call is
    (T_K - T_1) / (K - 1): the cost of the calls beyond the first, with the
    boundary cancelled. The median over `repeats` repeats is returned; the
    spread and the undifferenced T_K / K go to LAST_SPREAD.
    """
    repeats = REPEATS if repeats is None else repeats
    stream = torch.cuda.Stream()
    half = max(ncopies // 2, 1)

    def capture(first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(count):
                call((first + i) % ncopies)
        return g

    k = max(int(steps), 1)
    one_first = half                                  # the one-call graph reads the copy half a ring away
    timed = capture(0, k)
    one = capture(one_first, 1)
    flush_k = capture((0 - half) % ncopies, half)     # ends on the copy before timed's first
    flush_1 = capture((one_first - half) % ncopies, half)
    warm = capture(half // 2, max(warmup, 1))
    torch.cuda.synchronize()
    pairs = []
    with torch.cuda.stream(stream):
        for g in (timed, one, flush_k, flush_1, warm):     # first replay of each graph: untimed
            g.replay()
        for _ in range(repeats):
            evs = []
            for flush, g in ((flush_k, timed), (flush_1, one)):
                torch.cuda._sleep(SPIN_CYCLES)
                flush.replay()
                ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                ev0.record(stream)
                g.replay()
                ev1.record(stream)
                evs.append((ev0, ev1))
            pairs.append(evs)
    torch.cuda.synchronize()
    tk = [a.elapsed_time(b) for (a, b), _ in pairs]
    t1 = [a.elapsed_time(b) for _, (a, b) in pairs]
    if k > 1:
        per = sorted((x - y) / (k - 1) for x, y in zip(tk, t1))
    else:
        per = sorted(t1)
    med = per[len(per) // 2]
    LAST_SPREAD.clear()
    LAST_SPREAD.update({"repeats": repeats, "min_us": per[0] * 1e3, "max_us": per[-1] * 1e3,
                        "graph_us_per_call": sorted(tk)[len(tk) // 2] / k * 1e3,
                        "one_call_graph_us": sorted(t1)[len(t1) // 2] * 1e3})
    del timed, one, flush_k, flush_1, warm
    return med


def spread():
    return {k: round(v, 3) if isinstance(v, float) else v for k, v in LAST_SPREAD.items()}


class ClockSampler:
    """Engine (gfx) clock while a timed region runs, polled through amdsmi on a host
    thread (read-only queries; no GPU work): the SMU metrics' per-XCD current clocks
    (mean over XCDs) and the clock-info reading. None when amdsmi is unavailable."""

    def __init__(self, period_s=0.002):
        self.period, self.samples, self._stop, self._thread, self._h = period_s, [], None, None, None
        try:
            import amdsmi  # noqa: PLC0415
            amdsmi.amdsmi_init()
            self._amdsmi = amdsmi
            self._h = amdsmi.amdsmi_get_processor_handles()[0]
        except Exception:  # noqa: BLE001 (no amdsmi on this host: clock stays unknown)
            self._amdsmi = None

    def _read(self):
        out = {}
        try:
            met = self._amdsmi.amdsmi_get_gpu_metrics_info(self._h)
            clks = [float(c) for c in met.get("current_gfxclks", []) if isinstance(c, (int, float)) and c > 0]
            if clks:
                out["xcd"] = sum(clks) / len(clks)
            avg = met.get("average_gfxclk_frequency")
            if isinstance(avg, (int, float)) and avg > 0:
                out["avg"] = float(avg)
        except Exception:  # noqa: BLE001
            pass
        try:
            info = self._amdsmi.amdsmi_get_clock_info(self._h, self._amdsmi.AmdSmiClkType.GFX)
            out["info"] = float(info["clk"])
        except Exception:  # noqa: BLE001
            pass
        return out

    def __enter__(self):
        import threading  # noqa: PLC0415
        self.samples = []
        if self._amdsmi is None:
            return self
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                r = self._read()
                if not r:
                    return
                self.samples.append(r)
                self._stop.wait(self.period)
        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()

    def mean_ghz(self, key):
        v = [r[key] for r in self.samples if key in r]
        return round(sum(v) / len(v) / 1000.0, 3) if v else None


CLOCK = None


def clocked(fn):
    """Run fn() under the clock sampler; returns (result, {source: mean gfx clock in GHz})."""
    global CLOCK
    if CLOCK is None:
        CLOCK = ClockSampler()
    with CLOCK:
        r = fn()
    return r, {"smu_xcd_current": CLOCK.mean_ghz("xcd"), "smu_average": CLOCK.mean_ghz("avg"),
               "clock_info": CLOCK.mean_ghz("info"), "samples": len(CLOCK.samples)}


def decode_leg(name, m, k, n, nbytes, ms, ncopies, **extra):
    gbs = nbytes / (ms * 1e6)
    return {"workload": name, "M": m, "K": k, "N": n, "weight_bytes": nbytes, "us_per_call": ms * 1e3,
            "GB_s": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS, "copies": ncopies, "spread": spread(), **extra}


def gemm_leg(name, m, k, n, ms, clocks, int8, **extra):
    ops = 2.0 * m * n * k
    rate = ops / (ms * 1e9)
    peak = INT8_PEAK_TOPS if int8 else BF16_PEAK_TFLOPS
    ghz = clocks.get("smu_xcd_current") or clocks.get("smu_average") or clocks.get("clock_info")
    out = {"workload": name, "M": m, "K": k, "N": n, "us_per_call": ms * 1e3,
           ("TOP_s" if int8 else "TFLOP_s"): rate,
           ("frac_int8_mfma_peak" if int8 else "frac_bf16_mfma_peak"): rate / peak,
           "gfx_clock_ghz": clocks,
           # the published peak scaled to the engine clock sampled during the timed region
           "frac_clock_adjusted_peak": None if not ghz else rate / (peak * ghz / PEAK_CLOCK_GHZ),
           "spread": spread(), **extra}
    return out


def bench_ternary_decode(bpw, synth, torch, np, steps, warmup):
    w = synth.ternary_decode(1)
    planes = bpw.prepare_packed_host(bpw.TERNARY2, w.codes, w.scales)
    copies = rotated_copies(bpw, planes, 1 << 30)
    x = to_dev(w.x, "f32", torch, np)
    q, xs = bpw.quantize_rows(x)
    y = torch.empty((1, w.n), dtype=torch.float16, device="cuda")
    nbytes = copies[0].logical_bytes
    nc = len(copies)
    log(f"[bench] ternary decode GEMV M=1 K={w.k} N={w.n}: {nc} weight copies of {nbytes} B")
    ms = time_calls(torch, lambda c: bpw.gemv_packed(copies[c], q, xs, out=y), nc, steps, warmup)
    sp = spread()
    # complete decode call from the fp32 row: one launch (the quantiser fused into
    # the GEMV), and the quantiser launch followed by the GEMV
    ms_full = time_calls(torch, lambda c: bpw.gemv_packed(copies[c], x, out=y), nc, max(steps // 4, 1),
                         max(warmup // 4, 1))
    ms_two = time_calls(torch, lambda c: (bpw.quantize_rows(x, q, xs), bpw.gemv_packed(copies[c], q, xs, out=y)),
                        nc, max(steps // 4, 1), max(warmup // 4, 1))
    return w, nbytes, ms, sp, (ms_full, ms_two), nc


def bench_ternary_decode_large(bpw, synth, torch, np, steps, warmup):
    """The M = 1 decode GEMV on the ternary prefill weight (K=8192, N=28672, 62 MB), first activation row."""
    w = synth.leading_rows(synth.ternary_prefill(), 1)
    planes = bpw.prepare_packed_host(bpw.TERNARY2, w.codes, w.scales)
    w.codes = None
    copies = rotated_copies(bpw, planes, 1 << 30)
    q, xs = bpw.quantize_rows(to_dev(w.x, "f32", torch, np))
    y = torch.empty((1, w.n), dtype=torch.float16, device="cuda")
    ms = time_calls(torch, lambda c: bpw.gemv_packed(copies[c], q, xs, out=y), len(copies), steps, warmup)
    return decode_leg("ternary_decode_gemv_large_weight", 1, w.k, w.n, copies[0].logical_bytes, ms, len(copies))


def bench_probe(bpw, torch, kind, nbytes, steps, warmup):
    """Plain streaming read (or copy) of nbytes per call over rotated buffers (>= 1 GiB).

    The copy leg also calibrates the HBM byte counters: its kernel reads and
    writes exactly nbytes per launch."""
    count = math.ceil((1 << 30) / nbytes)
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(i % 251) for i in range(count)]
    if kind == bpw.PROBE_READ:
        sink = torch.empty(bpw.probe_blocks(nbytes) * 4, dtype=torch.uint8, device="cuda")
        moved, name = nbytes, "hbm_read_probe"
    else:
        sink = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        moved, name = 2 * nbytes, "hbm_copy_probe"
    ms = time_calls(torch, lambda c: bpw.probe(kind, bufs[c], sink), count, steps, warmup)
    del bufs
    return {"workload": name, "bytes": nbytes, "bytes_moved": moved, "us_per_call": ms * 1e3,
            "GB_s": moved / (ms * 1e6), "copies": count, "spread": spread()}


def bench_ternary_decode_m(bpw, synth, torch, np, steps, warmup, m=16):
    """Skinny ternary decode (M rows of int8 activations) through the MFMA GEMV."""
    w = synth.ternary_decode(m)
    planes = bpw.prepare_packed_host(bpw.TERNARY2, w.codes, w.scales)
    copies = rotated_copies(bpw, planes, 1 << 30)
    q, xs = bpw.quantize_rows(to_dev(w.x, "f32", torch, np))
    y = torch.empty((m, w.n), dtype=torch.float16, device="cuda")
    ms = time_calls(torch, lambda c: bpw.gemv_packed(copies[c], q, xs, out=y), len(copies), steps, warmup)
    return decode_leg("ternary_decode_gemv", m, w.k, w.n, copies[0].logical_bytes, ms, len(copies))


def bench_ternary_long_k(bpw, synth, torch, np, steps, warmup, m=16, k=14336, n=4096):
    """Ternary decode with K beyond 32 groups (a down-projection shape): split-K slices
    of 32 groups side by side, then the fixed-order reduce, both inside the call."""
    w = synth.ternary_int8(f"long_k_m{m}", 5, m, k, n, 0.005, 0.05, "f16")
    planes = bpw.prepare_packed_host(bpw.TERNARY2, w.codes, w.scales)
    copies = rotated_copies(bpw, planes, 1 << 30)
    q, xs = bpw.quantize_rows(to_dev(w.x, "f32", torch, np))
    y = torch.empty((m, n), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(bpw.workspace_size(copies[0], m, bpw.I8, bpw.PATH_GEMV), 1), dtype=torch.uint8, device="cuda")
    ms = time_calls(torch, lambda c: bpw.gemv_packed(copies[c], q, xs, out=y, workspace=ws), len(copies), steps,
                    warmup)
    return decode_leg("ternary_decode_gemv_long_k", m, k, n, copies[0].logical_bytes, ms, len(copies))


def bench_ternary_decode_groups(bpw, synth, torch, np, steps, warmup, m=1):
    """Ternary decode with one activation scale per (row, 128-group): the GEMV alone and,
    for the complete call, the GPU group quantiser in front of it."""
    w = synth.ternary_decode(m)
    planes = bpw.prepare_packed_host(bpw.TERNARY2, w.codes, w.scales)
    copies = rotated_copies(bpw, planes, 1 << 30)
    x = to_dev(w.x, "f32", torch, np)
    q, xs = bpw.quantize_groups(x)
    y = torch.empty((m, w.n), dtype=torch.float16, device="cuda")
    nc = len(copies)
    ms = time_calls(torch, lambda c: bpw.gemv_packed(copies[c], q, xs, out=y), nc, steps, warmup)
    sp = spread()
    ms_full = time_calls(torch, lambda c: (bpw.quantize_groups(x, q, xs), bpw.gemv_packed(copies[c], q, xs, out=y)),
                         nc, max(steps // 4, 1), max(warmup // 4, 1))
    leg = decode_leg("ternary_decode_gemv_group_scales", m, w.k, w.n, copies[0].logical_bytes, ms, nc,
                     complete_call_us=ms_full * 1e3)
    leg["spread"] = sp
    return leg


def bench_w4_decode(bpw, synth, torch, np, steps, warmup, m=1):
    w = synth.w4a16_decode(m)
    planes = bpw.prepare_packed_host(bpw.INT4_ZP, w.codes, w.scales, w.zeros, w.g_idx)
    copies = rotated_copies(bpw, planes, 1 << 30)
    x = to_dev(w.x, "f16", torch, np)
    y = torch.empty((m, w.n), dtype=torch.float16, device="cuda")
    ws = torch.empty(bpw.workspace_size(copies[0], m, bpw.F16, bpw.PATH_GEMV), dtype=torch.uint8, device="cuda")
    ms = time_calls(torch, lambda c: bpw.gemv_packed(copies[c], x, out=y, workspace=ws), len(copies), steps, warmup)
    return decode_leg("w4a16_decode_gemv", m, w.k, w.n, copies[0].logical_bytes, ms, len(copies), act_order=True)


def bench_w4_down(bpw, synth, torch, np, steps, warmup, m=1):
    """The down projection of the W4A16 decode layer (K=13824, N=5120): at M = 1 the
    row kernel with K split over two waves, at M = 8 split-K slices and their reduce.
    Act order at this K adds a separate gather launch; the same weight without act
    order times the GEMV alone."""
    out = {}
    for act in (True, False):
        w = synth.w4a16_down(m, act_order=act)
        planes = bpw.prepare_packed_host(bpw.INT4_ZP, w.codes, w.scales, w.zeros, w.g_idx)
        copies = rotated_copies(bpw, planes, 1 << 30)
        x = to_dev(w.x, "f16", torch, np)
        y = torch.empty((m, w.n), dtype=torch.float16, device="cuda")
        ws = torch.empty(max(bpw.workspace_size(copies[0], m, bpw.F16, bpw.PATH_GEMV), 1), dtype=torch.uint8,
                         device="cuda")
        ms = time_calls(torch, lambda c: bpw.gemv_packed(copies[c], x, out=y, workspace=ws), len(copies), steps,
                        warmup)
        out[act] = decode_leg("w4a16_down_gemv", m, w.k, w.n, copies[0].logical_bytes, ms, len(copies),
                              act_order=act)
        del copies
    out[True]["without_act_order"] = out[False]
    return out[True]


def bench_w4_prefill(bpw, synth, torch, np, steps, warmup):
    w = synth.w4a16_prefill()
    planes = bpw.prepare_packed_host(bpw.INT4_SYM, w.codes, w.scales, scale_dtype=bpw.BF16)
    copies = rotated_copies(bpw, planes, 512 << 20, max_copies=18)
    x = to_dev(w.x, "bf16", torch, np)
    y = torch.empty((w.m, w.n), dtype=torch.bfloat16, device="cuda")
    ms, ghz = clocked(lambda: time_calls(torch, lambda c: bpw.gemm_packed(copies[c], x, out=y), len(copies), steps,
                                         warmup))
    return gemm_leg("w4a16_prefill_gemm", w.m, w.k, w.n, ms, ghz, False)


def bench_ternary_prefill(bpw, synth, torch, np, steps, warmup):
    w = synth.ternary_prefill()
    planes = bpw.prepare_packed_host(bpw.TERNARY2, w.codes, w.scales)
    w.codes = None
    copies = rotated_copies(bpw, planes, 512 << 20, max_copies=9)
    q, xs = bpw.quantize_rows(to_dev(w.x, "f32", torch, np))
    y = torch.empty((w.m, w.n), dtype=torch.float16, device="cuda")
    ws = torch.empty(bpw.workspace_size(copies[0], w.m, bpw.I8, bpw.PATH_GEMM), dtype=torch.uint8, device="cuda")
    ms, ghz = clocked(lambda: time_calls(torch, lambda c: bpw.gemm_packed(copies[c], q, xs, out=y, workspace=ws),
                                         len(copies), steps, warmup))
    return gemm_leg("ternary_int8_prefill_gemm", w.m, w.k, w.n, ms, ghz, True)


def bench_w4a8_prefill(bpw, synth, torch, np, steps, warmup):
    """The 4-bit prefill weights against int8 activation rows (the int8 matrix core)."""
    w = synth.w4a16_prefill()
    planes = bpw.prepare_packed_host(bpw.INT4_SYM, w.codes, w.scales, scale_dtype=bpw.BF16)
    copies = rotated_copies(bpw, planes, 512 << 20, max_copies=18)
    q, xs = bpw.quantize_rows(to_dev(w.x, "bf16", torch, np))
    y = torch.empty((w.m, w.n), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(bpw.workspace_size(copies[0], w.m, bpw.I8, bpw.PATH_GEMM), dtype=torch.uint8, device="cuda")
    ms, ghz = clocked(lambda: time_calls(torch, lambda c: bpw.gemm_packed(copies[c], q, xs, out=y, workspace=ws),
                                         len(copies), steps, warmup))
    return gemm_leg("w4a8_prefill_gemm", w.m, w.k, w.n, ms, ghz, True, activations="int8 + fp32 row scale")


def bench_w4a8_affine_prefill(bpw, synth, torch, np, steps, warmup):
    """The 4-bit prefill weights against int8 activations in the affine form of the int8
    prompt GEMM (per row and weight group: scale a and the exact sum of x): the GEMM
    alone, and the complete call with the group quantiser in front of it."""
    w = synth.w4a16_prefill()
    planes = bpw.prepare_packed_host(bpw.INT4_SYM, w.codes, w.scales, scale_dtype=bpw.BF16)
    copies = rotated_copies(bpw, planes, 512 << 20, max_copies=18)
    x = to_dev(w.x, "bf16", torch, np)
    q, xss = bpw.quantize_groups_sums(x)
    y = torch.empty((w.m, w.n), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(bpw.workspace_size(copies[0], w.m, bpw.I8GS, bpw.PATH_GEMM), dtype=torch.uint8, device="cuda")
    nc = len(copies)
    ms, ghz = clocked(lambda: time_calls(torch, lambda c: bpw.gemm_packed(copies[c], q, xss, out=y, workspace=ws),
                                         nc, steps, warmup))
    leg = gemm_leg("w4a8_affine_prefill_gemm", w.m, w.k, w.n, ms, ghz, True,
                   activations="int8 + (scale, exact sum) per row and group")
    ms_full = time_calls(torch, lambda c: (bpw.quantize_groups_sums(x, None, q, xss),
                                           bpw.gemm_packed(copies[c], q, xss, out=y, workspace=ws)),
                         nc, max(steps // 2, 2), max(warmup // 2, 1))
    leg["complete_call_us"] = ms_full * 1e3
    return leg


def bench_ternary_groups_prefill(bpw, synth, torch, np, steps, warmup):
    """The ternary prefill workload with one activation scale per (row, 128-group)."""
    w = synth.ternary_prefill()
    planes = bpw.prepare_packed_host(bpw.TERNARY2, w.codes, w.scales)
    w.codes = None
    copies = rotated_copies(bpw, planes, 512 << 20, max_copies=9)
    q, xs = bpw.quantize_groups(to_dev(w.x, "f32", torch, np))
    y = torch.empty((w.m, w.n), dtype=torch.float16, device="cuda")
    ws = torch.empty(bpw.workspace_size(copies[0], w.m, bpw.I8G, bpw.PATH_GEMM), dtype=torch.uint8, device="cuda")
    ms, ghz = clocked(lambda: time_calls(torch, lambda c: bpw.gemm_packed(copies[c], q, xs, out=y, workspace=ws),
                                         len(copies), steps, warmup))
    return gemm_leg("ternary_int8_group_scales_prefill_gemm", w.m, w.k, w.n, ms, ghz, True,
                    activations="int8 + fp32 scale per row and 128-group")


def bench_dense_reference(torch, steps=20, warmup=5):
    """The platform's dense GEMMs (hipBLASLt through torch) at the two prefill shapes, with
    no quantisation: context for the MFMA fractions, not part of the library. Event-timed
    loops (these calls refuse graph capture here)."""
    def timed(fn, n, w):
        for i in range(w):
            fn(i)
        torch.cuda.synchronize()
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        for i in range(n):
            fn(i)
        en.record()
        torch.cuda.synchronize()
        return st.elapsed_time(en) / n
    out = []
    m, k, n = 2048, 4096, 14336
    a = torch.randn(m, k, device="cuda").to(torch.bfloat16)
    ws = [torch.randn(n, k, device="cuda").to(torch.bfloat16) for _ in range(4)]
    y = torch.empty(m, n, device="cuda", dtype=torch.bfloat16)
    ms = timed(lambda i: torch.matmul(a, ws[i % 4].t(), out=y), steps, warmup)
    out.append({"workload": "reference_dense_bf16_gemm", "M": m, "K": k, "N": n, "us_per_call": ms * 1e3,
                "TFLOP_s": 2.0 * m * n * k / (ms * 1e9), "frac_bf16_mfma_peak": 2.0 * m * n * k / (ms * 1e9) / BF16_PEAK_TFLOPS,
                "kind": "platform reference (hipBLASLt, bf16 weights, no dequant)"})
    del a, ws, y
    m, k, n = 4096, 8192, 28672
    qa = torch.randint(-127, 128, (m, k), device="cuda", dtype=torch.int8)
    qb = [torch.randint(-1, 2, (n, k), device="cuda", dtype=torch.int8).t() for _ in range(2)]   # column-major B
    ms = timed(lambda i: torch._int_mm(qa, qb[i % 2]), max(steps // 3, 2), 2)
    out.append({"workload": "reference_dense_int8_gemm", "M": m, "K": k, "N": n, "us_per_call": ms * 1e3,
                "TOP_s": 2.0 * m * n * k / (ms * 1e9), "frac_int8_mfma_peak": 2.0 * m * n * k / (ms * 1e9) / INT8_PEAK_TOPS,
                "kind": "platform reference (hipBLASLt, int8 weights, int32 out, no fold)"})
    return out


def host_info():
    """BLAS threads the oracle runs on, the host's CPU count and CPU model."""
    try:
        from threadpoolctl import threadpool_info  # noqa: PLC0415
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return threads, os.cpu_count(), model


def _repeat(fn, budget_s):
    """Call fn until budget_s has passed (at least once); returns (calls, seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return reps, el


def cpu_baselines(synth, np, budget_s=12.0):
    """The CPU oracle, unchanged, timed on bounded samples of the workloads: the headline
    decode GEMV (quantise + exact int group partials + fp64 fold), the W4A16 decode GEMV
    (dequantise through g_idx + fp64 product), the W4A16 prefill GEMM (rounded dequant +
    fp64 dgemm) and a leading row slice of the ternary x int8 prefill GEMM (its full
    M x N x G int64 partials would take 60 GB; the oracle's cost is linear in M)."""
    from oracle import quant, reference  # noqa: PLC0415 (test infrastructure, this leg only)
    threads, cpus, model = host_info()
    legs = []
    w = synth.ternary_decode(1)
    nbytes = w.n * w.k // 4 + w.n * (w.k // 128) * 2

    def headline():
        q, xs = quant.quantize_rows(w.x)
        reference.ternary_int8_product(q, xs, w.codes, w.scales)
    reps, el = _repeat(headline, budget_s)
    head = {"value": nbytes * reps / (el * 1e9), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"ternary_decode M=1 K={w.k} N={w.n}: quantise + exact int group partials + fp64 fold, "
                      f"{reps} full calls in {el:.1f} s", "seconds_per_call": el / reps,
            "host_cpus": cpus, "cpu_model": model}

    w3 = synth.w4a16_decode(1)
    b3 = w3.n * w3.k // 2 + w3.n * w3.groups * 2 + w3.n * ((w3.groups + 1) // 2)
    x3 = w3.x_f32()
    reps, el = _repeat(lambda: reference.product(
        x3, reference.weights_int4(w3.codes, w3.scales_f64(), w3.zeros, w3.g_idx)), budget_s / 3)
    legs.append({"workload": "w4a16_decode_gemv", "M": 1, "K": w3.k, "N": w3.n, "GB_s": b3 * reps / (el * 1e9),
                 "seconds_per_call": el / reps, "calls": reps})
    del w3, x3

    w4 = synth.w4a16_prefill()
    x4 = w4.x_f32()
    reps, el = _repeat(lambda: reference.product(
        x4, reference.weights_int4_rounded(w4.codes, w4.scales_f64(), None, None, "bf16")), budget_s / 3)
    legs.append({"workload": "w4a16_prefill_gemm", "M": w4.m, "K": w4.k, "N": w4.n,
                 "TFLOP_s": 2.0 * w4.m * w4.n * w4.k * reps / (el * 1e12), "seconds_per_call": el / reps,
                 "calls": reps})
    del w4, x4

    rows = 16
    w5 = synth.leading_rows(synth.ternary_prefill(), rows)
    q5, xs5 = quant.quantize_rows(w5.x)
    reps, el = _repeat(lambda: reference.ternary_int8_product(q5, xs5, w5.codes, w5.scales), budget_s / 3)
    legs.append({"workload": "ternary_int8_prefill_gemm", "M": rows, "K": w5.k, "N": w5.n,
                 "TOP_s": 2.0 * rows * w5.n * w5.k * reps / (el * 1e12), "seconds_per_call": el / reps,
                 "calls": reps, "sample": f"leading {rows} of 4096 rows (exact int partials + fp64 fold)"})
    head["other_workloads"] = legs
    return head


# Extra legs: name -> (function, steps, warm-up calls, keyword arguments).
LEGS = {
    "t2_m16": (bench_ternary_decode_m, 900, 300, {"m": 16}),
    "t2_long_k": (bench_ternary_long_k, 600, 200, {"m": 16}),
    "t2_large": (bench_ternary_decode_large, 600, 200, {}),
    "t2_groups_m1": (bench_ternary_decode_groups, 900, 300, {"m": 1}),
    "t2_groups_m16": (bench_ternary_decode_groups, 900, 300, {"m": 16}),
    "w4_m1": (bench_w4_decode, 900, 300, {"m": 1}),
    "w4_m8": (bench_w4_decode, 900, 300, {"m": 8}),
    "w4_down_m1": (bench_w4_down, 900, 300, {"m": 1}),
    "w4_down_m8": (bench_w4_down, 900, 300, {"m": 8}),
    "bf16_prefill": (bench_w4_prefill, 30, 6, {}),
    "w4a8_prefill": (bench_w4a8_prefill, 30, 6, {}),
    "t2_prefill": (bench_ternary_prefill, 12, 3, {}),
    "w4a8_affine_prefill": (bench_w4a8_affine_prefill, 30, 6, {}),
    "t2_groups_prefill": (bench_ternary_groups_prefill, 12, 3, {}),
}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2070)
    ap.add_argument("--warmup", type=int, default=690)
    ap.add_argument("--no-extra", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--legs", default="all",
                    help="comma-separated extra legs to run (default all; 'none' = headline and probes): "
                         + ",".join(LEGS))
    ap.add_argument("--repeats", type=int, default=7, help="timed repeats per leg (median reported)")
    args = ap.parse_args()
    global REPEATS
    REPEATS = max(1, args.repeats)
    legs = list(LEGS) if args.legs == "all" else [] if args.legs == "none" else args.legs.split(",")
    unknown = [x for x in legs if x not in LEGS and x != "dense_ref"]
    if unknown:
        ap.error(f"unknown legs {unknown}")
    if args.gpus != 1:
        print("bench.py: the benchmark runs on one GPU only; --gpus must be 1 "
              "(the multi-GPU sharding of the path is described, not implemented)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import bit_packed_weight_amd as bpw
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    w, nbytes, ms, sp, (ms_full, ms_two), ncopies = bench_ternary_decode(bpw, synth, torch, np, args.steps,
                                                                         args.warmup)
    gbs = nbytes / (ms * 1e6)
    log(f"[bench] ternary decode: {ms * 1e3:.3f} us/call (spread {sp}), {gbs:.0f} GB/s; "
        f"complete call {ms_full * 1e3:.2f} us (quantiser launch + GEMV {ms_two * 1e3:.2f} us)")
    extra = []
    read_probe = None
    for kind in (bpw.PROBE_READ, bpw.PROBE_COPY):
        probe = bench_probe(bpw, torch, kind, nbytes, args.steps, args.warmup)
        log(f"[bench] {json.dumps(probe)}")
        extra.append(probe)
        if kind == bpw.PROBE_READ:
            read_probe = probe["GB_s"]
        torch.cuda.empty_cache()
    if not args.no_extra:
        for name in legs:
            if name == "dense_ref":
                continue
            fn, steps, warm, kw = LEGS[name]
            if args.steps < 200:            # short runs (counter passes): fewer calls per leg
                steps, warm = max(2, min(steps, args.steps)), max(1, min(warm, args.warmup))
            r = fn(bpw, synth, torch, np, steps, warm, **kw)
            log(f"[bench] {name}: {json.dumps(r)}")
            extra.append(r)
            torch.cuda.empty_cache()
        if args.legs == "all" or "dense_ref" in legs:
            for r in bench_dense_reference(torch):
                log(f"[bench] {json.dumps(r)}")
                extra.append(r)
            torch.cuda.empty_cache()
    cpu = None if args.no_cpu else cpu_baselines(synth, np)
    if cpu:
        log(f"[bench] cpu oracle: {cpu['value']:.3f} GB/s on {cpu['cores']} threads "
            f"({cpu['host_cpus']} host CPUs, {cpu['cpu_model']}); {json.dumps(cpu['other_workloads'])}")
    out = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": "ternary_decode_gemv", "M": 1, "K": w.k, "N": w.n, "group": 128,
                   "weights": "2-bit ternary codes + fp16 scale per 128", "activations": "int8 + fp32 row scale",
                   "out": "f16", "rotated_weight_copies": ncopies},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic()},
        "frac_of_read_probe": round(gbs / read_probe, 4) if read_probe else None,
        "timing": {"median_of_repeats": sp["repeats"], "per_call_min_us": sp["min_us"],
                   "per_call_max_us": sp["max_us"], "graph_us_per_call": sp["graph_us_per_call"],
                   "one_call_graph_us": sp["one_call_graph_us"],
                   "method": "(T(K calls) - T(1 call)) / (K - 1), each graph after a spin and a half-ring flush"},
        "complete_call_us": round(ms_full * 1e3, 3),
        "complete_call_two_launches_us": round(ms_two * 1e3, 3),
        "cpu_baseline": cpu,
        "other_workloads": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

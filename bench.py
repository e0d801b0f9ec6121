#!/usr/bin/env python
"""Benchmark of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input that
is already resident in HBM:

  1. attn_fwd     causal prefill, B=8, H=32, N=4096, d=128, bf16  (headline)
  2. attn_decode  GQA decode, B=16, H=32, Hkv=8, L_b in [16384, 32768], d=128
  3. attn_hstu_jagged  16 jagged sequences, L_b in [512, 4096], H=4, d=64
  4. attn_bwd     backward of step 1 (dQ, dK, dV for a synthetic dO)
  5. attn_decode_paged  step 2's cache in pages of 16 rows, shuffled
  6. attn_hstu_jagged on step 3's sequences zero-padded to 4096 rows (the dense-padded
     baseline the HSTU page compares jagged tensors against; ``hstu_padded``)
  7. attn_fwd_fp8  step 1's shape with E4M3 Q, K, V and per-head descales

``value`` is the prefill throughput in TFLOP/s with the FLOP convention of the
ledger page (2 n^2 d per (b, h) for causal), from HIP events around every
prefill launch on the stream the kernel runs on; decode GB/s, HSTU TFLOP/s and
backward TFLOP/s (five products, 5 n^2 d per (b, h) causal) are reported
beside it.  After the timed step, ``roofline.clock`` records the shader clock
and socket power (amd-smi) while the prefill runs and the prefill's fraction
of the peak recomputed at that clock.  Prints ONE JSON line.

Other modes (used for profiling, see profiles/):
  --only prefill|decode|hstu|backward|decode_paged|hstu_padded|prefill_fp8   run just that part of the step
  --copy-calib                 run a plain 1 GiB device copy (HBM counter calibration)
  --summarize-trace DIR        summarise a rocprofv3 --kernel-trace --stats run
  --summarize-pmc DIR          summarise a rocprofv3 --pmc run (per-kernel bytes)
  --traffic FETCH WRITE CFETCH CWRITE
                               HBM bytes per prefill launch from FETCH_SIZE / WRITE_SIZE
                               runs, calibrated by the same counters on a 1 GiB copy
  --traffic-kernel NAME        with --traffic: those bytes for the named kernel(s) instead
  --counters DIR... --counter-kernel NAME [--counter-trace DIR]
                               counters of one kernel from --pmc runs, with derived utilisation
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense FP8 MFMA (twice the bf16 rate)
SIMDS = 1024                # 256 CUs x 4 SIMDs
SPEC_CLOCK_HZ = 2.4e9
# Issue cycles of one 64-lane transcendental instruction (v_exp_f32) on one
# SIMD, measured with an in-bounds microbenchmark (v_rcp_f32 taken at the
# same rate): the HSTU weight needs two per score.
TRANS_CYCLES_PER_WAVE_OP = 8.5
# Issue cycles of one 64-lane plain f32 VALU instruction on one SIMD (16 lanes
# per cycle); the SiLU weight adds an add, a multiply and half a bf16 pack per
# score to its two transcendentals.
VALU_CYCLES_PER_WAVE_OP = 4.0
TILE_KERNEL_SOURCES = ["exact_attention_11_amd/csrc/tile_bf16.hip", "exact_attention_11_amd/csrc/common.hpp",
                       "exact_attention_11_amd/csrc/launch.hpp"]
DECODE_KERNEL_SOURCES = ["exact_attention_11_amd/csrc/decode.hip", "exact_attention_11_amd/csrc/common.hpp",
                         "exact_attention_11_amd/csrc/launch.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "tile_bf16_prefill_d128_causal_traffic.txt")


def prefill_flops(B, H, N, d, causal) -> int:
    """Ledger page convention: two products of 2 n^2 d per (b, h), causal
    counted as half (HSTU page, optimisation two)."""
    return B * H * 4 * N * N * d // (2 if causal else 1)


def backward_flops(B, H, N, d, causal) -> int:
    """Five products of 2 n^2 d per (b, h) (S, dP, dV, dQ, dK), causal halved."""
    return B * H * 10 * N * N * d // (2 if causal else 1)


def hstu_flops(lengths, H, d, causal=True) -> int:
    """The prefill convention summed over the jagged sequences."""
    return H * sum(4 * int(L) * int(L) * d for L in lengths) // (2 if causal else 1)


def decode_bytes(seqlens, B, H, Hkv, d) -> int:
    """Algorithmic bytes of one decode call: K and V rows [0, L_b) once per kv
    head, q and O once, LSE and the lengths once (the workspace partials are
    overhead, not algorithmic)."""
    return int(sum(int(L) for L in seqlens)) * Hkv * d * 2 * 2 + 2 * B * H * d * 2 + B * H * 4 + B * 4


def sources_sha(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--only", choices=["prefill", "decode", "hstu", "backward", "decode_paged", "hstu_padded",
                                       "prefill_fp8", "prefill_d64"], default=None,
                    help="run one part (prefill_d64, the B=1 H=32 N=4096 d=64 causal prefill, is a profiling "
                         "mode outside the default step)")
    ap.add_argument("--splits", type=int, default=0, help="decode split count (0 = automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context measurements after the timed step (other prefill shapes, decode "
                         "split sweep)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calib", action="store_true")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-pmc", metavar="DIR")
    ap.add_argument("--counters", nargs="+", metavar="DIR", help="summarise --pmc runs of one kernel (with "
                    "--counter-kernel; optional --counter-trace DIR of a --kernel-trace run)")
    ap.add_argument("--counter-kernel", metavar="NAME")
    ap.add_argument("--counter-trace", metavar="DIR")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH", "WRITE", "CFETCH", "CWRITE"))
    ap.add_argument("--traffic-kernel", action="append", default=None, metavar="NAME",
                    help="with --traffic: report this kernel (substring of its name) instead of the prefill; "
                         "repeatable")
    return ap.parse_args(argv)


# ----------------------------------------------------------------------------- rocprofv3 summaries

def _read_csv(path):
    import csv

    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize_trace(d: str) -> None:
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {d}")
    for path in files:
        rows = _read_csv(path)
        print(f"# {os.path.relpath(path, d)}")
        print(f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_%':>8}  kernel")
        for r in rows:
            name = r.get("Name", r.get("KernelName", "?"))
            print(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                  f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):8.2f}  {name[:110]}")
    # per-dispatch durations: median and the 10th / 90th percentiles
    for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        per = {}
        for r in _read_csv(path):
            name = r.get("Kernel_Name", r.get("Name", "?"))
            try:
                per.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
            except (KeyError, ValueError):
                continue
        if not per:
            continue
        print(f"# {os.path.relpath(path, d)}: per-dispatch duration percentiles")
        print(f"{'calls':>6} {'p10_us':>10} {'median_us':>10} {'p90_us':>10}  kernel")
        for name, ds in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            ds.sort()
            pick = lambda f: ds[min(len(ds) - 1, int(round(f * (len(ds) - 1))))]  # noqa: E731
            print(f"{len(ds):6d} {pick(0.1):10.2f} {pick(0.5):10.2f} {pick(0.9):10.2f}  {name[:110]}")


def summarize_pmc(d: str) -> None:
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    agg = {}
    for path in files:
        for r in _read_csv(path):
            name = r.get("Kernel_Name", "?")
            ctr = r.get("Counter_Name", "?")
            val = float(r.get("Counter_Value", "nan"))
            key = (name, ctr)
            disp = r.get("Dispatch_Id", "")
            agg.setdefault(key, {})
            agg[key][disp] = agg[key].get(disp, 0.0) + val
    print(f"{'dispatches':>10} {'mean_per_dispatch':>18} {'unit':>5}  counter  kernel")
    for (name, ctr), per in sorted(agg.items()):
        vals = list(per.values())
        mean = sum(vals) / len(vals)
        print(f"{len(vals):10d} {mean:18.1f} {'KiB' if ctr.endswith('SIZE') else '':>5}  {ctr}  {name[:100]}")


def _pmc_mean_kib(d: str, kernel_substr: str, counter: str) -> float:
    vals = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in _read_csv(path):
            if kernel_substr in r.get("Kernel_Name", "") and r.get("Counter_Name") == counter:
                k = r.get("Dispatch_Id", "")
                vals[k] = vals.get(k, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit(f"no {counter} for {kernel_substr!r} under {d}")
    return sum(vals.values()) / len(vals)


def counters_report(dirs, kernel_substr: str, trace_dir=None) -> None:
    """Counters of one kernel (mean per dispatch over every --pmc run under
    `dirs`) and what follows from them: MFMA busy fraction, instructions per
    MFMA, the shader clock from the fastest traced dispatch."""
    vals = {}
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            per = {}
            for r in _read_csv(path):
                if kernel_substr in r.get("Kernel_Name", ""):
                    key = (r["Counter_Name"], r.get("Dispatch_Id", ""))
                    per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
            by_ctr = {}
            for (ctr, _), v in per.items():
                by_ctr.setdefault(ctr, []).append(v)
            for ctr, v in by_ctr.items():
                vals[ctr] = sum(v) / len(v)
    if not vals:
        raise SystemExit(f"no counters for {kernel_substr!r}")
    for k in sorted(vals):
        print(f"{k:28s} {vals[k]:.4g}")
    print("# derived (GRBM_GUI_ACTIVE is summed over the 8 XCDs; 1024 SIMDs)")
    gui = vals.get("GRBM_GUI_ACTIVE", float("nan")) / 8
    mfma = vals.get("SQ_INSTS_MFMA", float("nan"))
    if "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
        print(f"mfma_busy_fraction           {vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (gui * 1024):.3f}")
        if mfma > 0:
            print(f"mfma_busy_cycles_per_mfma    {vals['SQ_VALU_MFMA_BUSY_CYCLES'] / mfma:.1f}")
    if mfma > 0:  # instruction mix per matrix product (kernels without products: the counts above)
        for ctr, label in (("SQ_INSTS_VALU", "valu_non_mfma_per_mfma"), ("SQ_INSTS_SALU", "salu_per_mfma"),
                           ("SQ_INSTS_LDS", "lds_per_mfma"), ("SQ_INSTS_VMEM", "vmem_per_mfma"),
                           ("SQ_INSTS_VALU_TRANS_F32", "trans_per_mfma")):
            if ctr in vals:
                v = vals[ctr] - (mfma if ctr == "SQ_INSTS_VALU" else 0)
                print(f"{label:28s} {v / mfma:.2f}")
    if "SQ_BUSY_CYCLES" in vals:
        # SQ_BUSY_CYCLES is summed over the 32 shader engines
        print(f"sq_busy_fraction             {vals['SQ_BUSY_CYCLES'] / 32 / gui:.3f}   (SQ_BUSY_CYCLES / 32 SEs)")
    if "SQ_WAVE_CYCLES" in vals:
        print(f"mean_resident_waves          {vals['SQ_WAVE_CYCLES'] * 4 / gui:.0f}   (SQ_WAVE_CYCLES counts 4-cycle units)")
    if trace_dir:
        for path in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
            ds = sorted(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in _read_csv(path)
                        if kernel_substr in r.get("Kernel_Name", ""))
            if ds:
                print(f"dispatch_us                  {' '.join(f'{x / 1e3:.1f}' for x in ds)}   (kernel-trace run)")
                if ds[0] >= 50_000:
                    print(f"gpu_clock_ghz                {gui / ds[0]:.2f}   (GRBM_GUI_ACTIVE per XCD / fastest dispatch)")
                else:  # the active count also covers the launch's start and drain
                    print("gpu_clock_ghz                n/a   (dispatch under 50 us)")


PREFILL_KERNEL = "tile_kernel<128, true, (fattn::Epilogue)0, false>"


def traffic_summary(fetch_dir, write_dir, cfetch_dir, cwrite_dir, kernels=None) -> None:
    """Print HBM bytes per dispatch: counter KiB scaled so that a 1 GiB device
    copy reads and writes 1 GiB.  Default: the causal d=128 prefill kernel (the
    summary bench.py reads back); with `kernels`, one block per kernel."""
    copy = "copyBuffer"
    gib = float(1 << 30)
    f_cal = gib / (_pmc_mean_kib(cfetch_dir, copy, "FETCH_SIZE") * 1024.0)
    w_cal = gib / (_pmc_mean_kib(cwrite_dir, copy, "WRITE_SIZE") * 1024.0)
    print(f"fetch_calibration: {f_cal:.4f}")
    print(f"write_calibration: {w_cal:.4f}")
    if not kernels:
        fetch = _pmc_mean_kib(fetch_dir, PREFILL_KERNEL, "FETCH_SIZE") * 1024.0 * f_cal
        write = _pmc_mean_kib(write_dir, PREFILL_KERNEL, "WRITE_SIZE") * 1024.0 * w_cal
        print(f"hbm_fetch_bytes_per_launch: {fetch:.0f}")
        print(f"hbm_write_bytes_per_launch: {write:.0f}")
        print(f"hbm_bytes_per_launch: {fetch + write:.0f}")
        print(f"kernel_sources_sha: {sources_sha(TILE_KERNEL_SOURCES)}")
        return
    total = 0.0
    for kern in kernels:
        fetch = _pmc_mean_kib(fetch_dir, kern, "FETCH_SIZE") * 1024.0 * f_cal
        write = _pmc_mean_kib(write_dir, kern, "WRITE_SIZE") * 1024.0 * w_cal
        total += fetch + write
        print(f"[{kern}] hbm_fetch_bytes_per_launch: {fetch:.0f}")
        print(f"[{kern}] hbm_write_bytes_per_launch: {write:.0f}")
    print(f"hbm_bytes_all_listed_kernels: {total:.0f}")


# ----------------------------------------------------------------------------- the benchmark

def read_traffic():
    """HBM bytes per prefill launch from the committed rocprofv3 counter summary,
    or None when the tile kernel's sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for ln in f:
            if ":" in ln and not ln.startswith("#"):
                k, v = ln.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha") != sources_sha(TILE_KERNEL_SOURCES):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(x, case, seconds: float):
    """The C++ fp64 oracle as it stands (S and P materialised per row panel,
    two-pass softmax, plain loops, OpenMP over (batch, head, panel)) on a
    bounded sample of the prefill workload: whole (b, h) heads, all rows, one
    head per host thread per call, until about `seconds` of compute; then the
    d=64 causal prefill (B=1, H=32, N=4096) on one thread for about a quarter
    of that.  Converting the bf16 inputs to fp64 is not timed."""
    import numpy as np

    import oracle
    from oracle import cpp as ocpp
    from synthgen import workloads as W

    threads = ocpp.max_threads()
    per_head = prefill_flops(1, 1, case.N, case.d, case.causal)
    group = case.H // case.Hkv
    done, el = 0, 0.0
    while done < case.B * case.H and el < seconds:
        b, h0 = divmod(done, case.H)
        h1 = min(case.H, h0 + threads)
        q = x.f64("q", (slice(b, b + 1), slice(h0, h1)))
        kv_heads = [h // group for h in range(h0, h1)]  # one kv head per query head, in order
        k = x.f64("k", (slice(b, b + 1), kv_heads))
        v = x.f64("v", (slice(b, b + 1), kv_heads))
        ts = time.perf_counter()
        oracle.attention_forward(q, k, v, case.scale, case.causal)
        el += time.perf_counter() - ts
        done += h1 - h0
    c1 = W.PREFILL_D64
    x1 = W.dense_inputs(c1)
    per_head1 = prefill_flops(1, 1, c1.N, c1.d, True)
    done1, el1 = 0, 0.0
    ocpp.set_threads(1)
    try:
        while done1 < c1.H and el1 < seconds / 4:
            q, k, v = (np.ascontiguousarray(x1.f64(n, (slice(0, 1), slice(done1, done1 + 1)))) for n in "qkv")
            ts = time.perf_counter()
            oracle.attention_forward(q, k, v, c1.scale, True)
            el1 += time.perf_counter() - ts
            done1 += 1
    finally:
        ocpp.set_threads(threads)
    return {
        "value": round(done * per_head / el / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {case.B * case.H} (b,h) heads of the B={case.B} H={case.H} N={case.N} d={case.d} "
                  f"{'causal' if case.causal else 'non-causal'} prefill, all rows, C++ fp64 oracle on {threads} "
                  f"threads, {el:.1f} s of compute",
        "one_core": {"value": round(done1 * per_head1 / el1 / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
                     "sample": f"{done1} of {c1.H} heads of the B=1 H=32 N=4096 d=64 causal prefill, C++ fp64 "
                               f"oracle on 1 thread, {el1:.1f} s of compute"},
        "cpu_model": _cpu_model(),
        "host_cpus": os.cpu_count(),
    }


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _time_calls(fn, stream, warmup: int = 3, reps: int = 10) -> float:
    """Mean milliseconds per call of fn from HIP events on `stream`."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _smi_sample(exe: str):
    """One `amd-smi metric` reading of GPU 0: (per-XCD shader clocks in MHz, socket power in W)."""
    import subprocess

    r = subprocess.run([exe, "metric", "-g", "0", "--clock", "--power", "--json"], capture_output=True, text=True,
                       timeout=20)
    text = r.stdout
    start = min(i for i in (text.find("{"), text.find("[")) if i >= 0)
    d = json.loads(text[start:])
    g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
    clocks = []
    for key in sorted(k for k in g["clock"] if k.startswith("gfx_")):
        v = g["clock"][key]["clk"]["value"]
        if isinstance(v, (int, float)):
            clocks.append(float(v))
    power = g["power"]["socket_power"]["value"]
    return clocks, (float(power) if isinstance(power, (int, float)) else None)


def clock_under_load(launch, samples: int = 2) -> dict:
    """Shader clock and socket power while the headline prefill runs: a thread keeps
    launching it while `amd-smi` (a child process) reads the GPU, then the
    launches stop and the stream drains."""
    import shutil
    import threading

    import torch

    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    stop = threading.Event()

    def keep_busy():
        while not stop.is_set():
            for _ in range(50):
                launch()
            torch.cuda.current_stream().synchronize()

    t = threading.Thread(target=keep_busy, daemon=True)
    t.start()
    time.sleep(0.5)
    got = []
    err = None
    for _ in range(samples):
        try:
            got.append(_smi_sample(exe))
        except Exception as e:  # a missing or unparsable tool leaves the fields empty
            err = f"{type(e).__name__}: {e}"
    stop.set()
    t.join()
    torch.cuda.synchronize()
    clocks = sorted(c for cl, _ in got for c in cl)
    powers = [p for _, p in got if p is not None]
    if not clocks:
        return {"sclk_mhz": None, "socket_power_w": None, "note": err or "no clock reading"}
    return {"sclk_mhz": clocks[len(clocks) // 2], "sclk_mhz_range": [clocks[0], clocks[-1]],
            "socket_power_w": max(powers) if powers else None, "samples": len(got),
            "source": "amd-smi metric while the prefill ran (median over XCDs and samples)"}


def context_measurements(fa, W, bf16, dev, stream, q, k, v, o, lse, pc, dx, dc, dq, dk, dv, dsl, do, dlse):
    """Other prefill shapes and a decode split sweep, each timed with HIP events
    after the timed step."""
    import torch

    ctx = {}
    # the headline shape without the causal mask: 4 n^2 d per (b, h)
    f = prefill_flops(pc.B, pc.H, pc.N, pc.d, False)
    ms_nc = _time_calls(lambda: fa.attn_fwd(q, k, v, o, lse, pc.B, pc.H, pc.Hkv, pc.N, pc.d, pc.scale, 0), stream)
    ctx["prefill_noncausal"] = {"workload": "B=8 H=32 N=4096 d=128 bf16 non-causal", "ms_per_call": round(ms_nc, 4),
                                "TFLOP/s": round(f / (ms_nc * 1e-3) / 1e12, 2),
                                "frac_bf16_peak": round(f / (ms_nc * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    for key, c, label in (("prefill_long", W.PREFILL_LONG, "B=1 H=32 N=32768 d=128 bf16 causal"),
                          ("prefill_d64", W.PREFILL_D64, "B=1 H=32 N=4096 d=64 bf16 causal"),
                          ("prefill_d256", W.PREFILL_D256, "B=4 H=32 N=4096 d=256 bf16 causal")):
        x = W.dense_inputs(c)
        cq, ck, cv = bf16(x.q), bf16(x.k), bf16(x.v)
        del x
        co = torch.empty_like(cq)
        cl = torch.empty((c.B, c.H, c.N), dtype=torch.float32, device=dev)
        ms_c = _time_calls(lambda: fa.attn_fwd(cq, ck, cv, co, cl, c.B, c.H, c.Hkv, c.N, c.d, c.scale, 1), stream)
        fc = prefill_flops(c.B, c.H, c.N, c.d, True)
        ctx[key] = {"workload": label, "ms_per_call": round(ms_c, 4), "TFLOP/s": round(fc / (ms_c * 1e-3) / 1e12, 2),
                    "frac_bf16_peak": round(fc / (ms_c * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del cq, ck, cv, co, cl
    # decode at fixed split counts (the timed step uses the automatic count)
    ssum = int(dx.seqlens.sum())
    nbytes = decode_bytes(dx.seqlens, dc.B, dc.H, dc.Hkv, dc.d)
    wsb = fa.attn_decode_workspace_bytes(dc.B, dc.H, dc.d, 8)
    ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
    sweep = {}
    for sp in (4, 8):
        ms_d = _time_calls(lambda: fa.attn_decode(dq, dk, dv, dsl, do, dlse, dc.B, dc.H, dc.Hkv, dc.Lmax, dc.d,
                                                  dc.scale, sp, ws, wsb), stream, reps=20)
        sweep[str(sp)] = {"GB/s": round(nbytes / (ms_d * 1e-3) / 1e9, 1), "ms_per_call": round(ms_d, 4)}
    ctx["decode_splits"] = sweep
    return ctx


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return 0
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return 0
    if args.counters:
        counters_report(args.counters, args.counter_kernel or "", args.counter_trace)
        return 0
    if args.traffic:
        traffic_summary(*args.traffic, kernels=args.traffic_kernel)
        return 0
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the kernels are measured on one GPU's "
              "share at its real shape; sharding over several GPUs is not built.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import exact_attention_11_amd as fa
    from synthgen import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    dev = "cuda"

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    if args.copy_calib:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n, "launches": 3}))
        return 0

    parts = [args.only] if args.only else ["prefill", "decode", "hstu", "backward", "decode_paged", "hstu_padded",
                                           "prefill_fp8"]
    print(f"bench: preparing inputs for {parts}", file=sys.stderr, flush=True)

    pc = W.PREFILL_D128_CAUSAL
    need_dense = "prefill" in parts or "backward" in parts
    px = W.dense_inputs(pc) if need_dense or not args.no_cpu_baseline else None
    calls = {}
    if need_dense:
        q, k, v = bf16(px.q), bf16(px.k), bf16(px.v)
        o = torch.empty((pc.B, pc.H, pc.N, pc.d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((pc.B, pc.H, pc.N), dtype=torch.float32, device=dev)
        calls["prefill"] = lambda: fa.attn_fwd(q, k, v, o, lse, pc.B, pc.H, pc.Hkv, pc.N, pc.d, pc.scale, 1)
    if "backward" in parts:
        from synthgen import TENSOR_DO, normal_bf16

        gout = bf16(normal_bf16(pc.seed, TENSOR_DO, (pc.B, pc.H, pc.N, pc.d)))
        gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bwsb = fa.attn_bwd_workspace_bytes(pc.B, pc.H, pc.N)
        bws = torch.empty(bwsb // 4, dtype=torch.float32, device=dev)
        calls["prefill"]()  # the backward reads the forward's O and LSE
        calls["backward"] = lambda: fa.attn_bwd(q, k, v, o, lse, gout, gq, gk, gv, pc.B, pc.H, pc.Hkv, pc.N, pc.d,
                                                pc.scale, 1, bws, bwsb)
    if "prefill_d64" in parts:
        c64 = W.PREFILL_D64
        x64 = W.dense_inputs(c64)
        q64, k64, v64 = bf16(x64.q), bf16(x64.k), bf16(x64.v)
        del x64
        o64 = torch.empty_like(q64)
        l64 = torch.empty((c64.B, c64.H, c64.N), dtype=torch.float32, device=dev)
        calls["prefill_d64"] = lambda: fa.attn_fwd(q64, k64, v64, o64, l64, c64.B, c64.H, c64.Hkv, c64.N, c64.d,
                                                   c64.scale, 1)
    if "prefill_fp8" in parts:
        fc = W.PREFILL_FP8
        fx = W.fp8_dense_inputs(fc)
        dev_arr = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
        fq, fk, fv = dev_arr(fx.q), dev_arr(fx.k), dev_arr(fx.v)
        fdq, fdk, fdv = dev_arr(fx.descale_q), dev_arr(fx.descale_k), dev_arr(fx.descale_v)
        fo = torch.empty((fc.B, fc.H, fc.N, fc.d), dtype=torch.bfloat16, device=dev)
        flse = torch.empty((fc.B, fc.H, fc.N), dtype=torch.float32, device=dev)
        calls["prefill_fp8"] = lambda: fa.attn_fwd_fp8(fq, fk, fv, fo, flse, fdq, fdk, fdv, fc.B, fc.H, fc.Hkv, fc.N,
                                                       fc.d, fc.scale, 1)
        del fx
    dc = W.DECODE_GQA
    dx = None
    if "decode" in parts or "decode_paged" in parts:
        dx = W.decode_inputs(dc)
    if "decode_paged" in parts:
        page = 16
        pdx = W.paged_from_decode(dx, page)
        pq, pk, pv = bf16(dx.q), bf16(pdx.k_pages), bf16(pdx.v_pages)
        ptab = torch.from_numpy(pdx.block_table).to(dev)
        psl = torch.from_numpy(dx.seqlens).to(dev)
        pmp = pdx.block_table.shape[1]
        pnp = pdx.num_pages
        po = torch.empty((dc.B, dc.H, dc.d), dtype=torch.bfloat16, device=dev)
        plse = torch.empty((dc.B, dc.H), dtype=torch.float32, device=dev)
        pwsb = fa.attn_decode_workspace_bytes(dc.B, dc.H, dc.d, args.splits)
        pws = torch.empty(pwsb // 4, dtype=torch.float32, device=dev)
        calls["decode_paged"] = lambda: fa.attn_decode_paged(pq, pk, pv, ptab, psl, po, plse, dc.B, dc.H, dc.Hkv, page,
                                                             pmp, pnp, dc.d, dc.scale, args.splits, pws,
                                                             pwsb)
        del pdx
    if "decode" in parts:
        dq, dk, dv = bf16(dx.q), bf16(dx.k), bf16(dx.v)
        dsl = torch.from_numpy(dx.seqlens).to(dev)
        do = torch.empty((dc.B, dc.H, dc.d), dtype=torch.bfloat16, device=dev)
        dlse = torch.empty((dc.B, dc.H), dtype=torch.float32, device=dev)
        wsb = fa.attn_decode_workspace_bytes(dc.B, dc.H, dc.d, args.splits)
        ws = torch.empty(wsb // 4, dtype=torch.float32, device=dev)
        calls["decode"] = lambda: fa.attn_decode(dq, dk, dv, dsl, do, dlse, dc.B, dc.H, dc.Hkv, dc.Lmax, dc.d,
                                                 dc.scale, args.splits, ws, wsb)
    jc = W.HSTU_JAGGED
    jx = None
    if "hstu" in parts or "hstu_padded" in parts:
        jx = W.jagged_inputs(jc)
    if "hstu_padded" in parts:
        # every sequence zero-padded to len_hi rows: silu(alpha q.0) = 0, so the
        # padding adds nothing to the valid rows but is computed like them
        Np = jc.len_hi
        nseq_p = len(jx.lengths)
        padded = {}
        for name in ("q", "k", "v"):
            src = getattr(jx, name)
            dst = np.zeros((nseq_p * Np, jc.H, jc.d), dtype=np.uint16)
            for b in range(nseq_p):
                s0, s1 = int(jx.offsets[b]), int(jx.offsets[b + 1])
                dst[b * Np:b * Np + (s1 - s0)] = src[s0:s1]
            padded[name] = bf16(dst)
        poff = torch.arange(0, (nseq_p + 1) * Np, Np, dtype=torch.int32, device=dev)
        po_h = torch.empty((nseq_p * Np, jc.H, jc.d), dtype=torch.bfloat16, device=dev)
        calls["hstu_padded"] = lambda: fa.attn_hstu_jagged(padded["q"], padded["k"], padded["v"], po_h, poff, nseq_p,
                                                           jc.H, jc.d, Np, jc.alpha, jc.inv_n, 1)
    if "hstu" in parts:
        T = int(jx.offsets[-1])
        jq, jk, jv = bf16(jx.q), bf16(jx.k), bf16(jx.v)
        joff = torch.from_numpy(jx.offsets).to(dev)
        jo = torch.empty((T, jc.H, jc.d), dtype=torch.bfloat16, device=dev)
        nseq = len(jx.lengths)
        calls["hstu"] = lambda: fa.attn_hstu_jagged(jq, jk, jv, jo, joff, nseq, jc.H, jc.d, jx.max_seqlen,
                                                    jc.alpha, jc.inv_n, 1)

    stream = torch.cuda.current_stream()

    def step(record):
        for name in parts:
            if record is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                calls[name]()
                e1.record(stream)
                record[name].append((e0, e1))
            else:
                calls[name]()

    print(f"bench: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    rec = {name: [] for name in parts}
    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch = {name: sorted(a.elapsed_time(b) for a, b in rec[name]) for name in parts}
    ms = {name: sum(v) / max(1, len(v)) for name, v in per_launch.items()}
    med = {name: (v[len(v) // 2] if v else float("nan")) for name, v in per_launch.items()}

    out = {
        "metric": "attn fwd TFLOPS & % bf16 MFMA peak (N=4096,d=128 causal); decode HBM GB/s",
        "value": None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / max(1, args.steps), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "causal prefill B=8 H=32 N=4096 d=128 bf16 (+ GQA decode, jagged HSTU in the step)",
                   "global_batch": pc.B, "seq_len": pc.N, "parallelism": "none (1 GPU)"},
    }
    if "prefill" in parts:
        flops = prefill_flops(pc.B, pc.H, pc.N, pc.d, True)
        tflops = flops / (ms["prefill"] * 1e-3) / 1e12
        out["value"] = round(tflops, 2)
        traffic = read_traffic()
        out["roofline"] = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                           "kernel": "tile_kernel<128,causal,softmax>", "flops_per_launch": flops,
                           "ms_per_launch": round(ms["prefill"], 4), "median_ms_per_launch": round(med["prefill"], 4),
                           "launches": len(per_launch["prefill"])}
    if "decode" in parts:
        ssum = int(dx.seqlens.sum())
        nbytes = decode_bytes(dx.seqlens, dc.B, dc.H, dc.Hkv, dc.d)
        gbs = nbytes / (ms["decode"] * 1e-3) / 1e9
        out["decode"] = {"GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                         "ms_per_call": round(ms["decode"], 4), "median_ms_per_call": round(med["decode"], 4),
                         "algorithmic_bytes": nbytes, "sum_L": ssum, "splits": args.splits or "auto"}
        if out["value"] is None:
            out.update({"value": round(gbs, 1), "unit": "GB/s"})
    if "decode" in parts and not args.only:
        # the same decode at 16, 32 and 64 chunks per sequence (the automatic
        # count above is 768 work items in all, 6 chunks per sequence here);
        # left out of single-part runs, whose counter profiles then cover the
        # automatic split alone
        sweep = {}
        swsb = fa.attn_decode_workspace_bytes(dc.B, dc.H, dc.d, 64)
        sws = torch.empty(swsb // 4, dtype=torch.float32, device=dev)
        for sp in (16, 32, 64):
            ms_s = _time_calls(lambda: fa.attn_decode(dq, dk, dv, dsl, do, dlse, dc.B, dc.H, dc.Hkv, dc.Lmax, dc.d,
                                                      dc.scale, sp, sws, swsb), stream, reps=20)
            sweep[str(sp)] = {"GB/s": round(nbytes / (ms_s * 1e-3) / 1e9, 1),
                              "frac_hbm_peak": round(nbytes / (ms_s * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                              "ms_per_call": round(ms_s, 4)}
        out["decode"]["splits_sweep"] = sweep
        del sws
    if "decode_paged" in parts:
        ssum = int(dx.seqlens.sum())
        # same algorithmic bytes as the contiguous decode (the block-table reads,
        # 4 bytes per 16-row page, are under 0.01 % and not counted)
        nbytes = decode_bytes(dx.seqlens, dc.B, dc.H, dc.Hkv, dc.d)
        gbs = nbytes / (ms["decode_paged"] * 1e-3) / 1e9
        out["decode_paged"] = {"GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                               "ms_per_call": round(ms["decode_paged"], 4),
                               "median_ms_per_call": round(med["decode_paged"], 4), "algorithmic_bytes": nbytes,
                               "page_size": 16, "splits": args.splits or "auto"}
        if out["value"] is None:
            out.update({"value": round(gbs, 1), "unit": "GB/s"})
    if "hstu" in parts:
        hf = hstu_flops(jx.lengths, jc.H, jc.d)
        ht = hf / (ms["hstu"] * 1e-3) / 1e12
        # transcendental bound: two per score (exp2 and rcp of the SiLU weight),
        # scores counted by the same causal convention (flops / 4d)
        scores = hf / (4 * jc.d)
        trans_ms = 2 * scores / 64 * TRANS_CYCLES_PER_WAVE_OP / (SIMDS * SPEC_CLOCK_HZ) * 1e3
        # vector-issue bound of the whole weight: the transcendentals plus the
        # plain instructions each score needs
        silu_ms = trans_ms + 2.5 * scores / 64 * VALU_CYCLES_PER_WAVE_OP / (SIMDS * SPEC_CLOCK_HZ) * 1e3
        out["hstu"] = {"TFLOP/s": round(ht, 2), "frac_bf16_peak": round(ht / PEAK_BF16_TFLOPS, 4),
                       "ms_per_call": round(ms["hstu"], 4), "median_ms_per_call": round(med["hstu"], 4),
                       "flops": hf, "trans_bound_ms": round(trans_ms, 4),
                       "frac_trans_bound": round(trans_ms / ms["hstu"], 4),
                       "silu_valu_bound_ms": round(silu_ms, 4),
                       "frac_silu_valu_bound": round(silu_ms / ms["hstu"], 4)}
        if out["value"] is None:
            out.update({"value": round(ht, 2), "unit": "TFLOP/s"})
    if "backward" in parts:
        bf = backward_flops(pc.B, pc.H, pc.N, pc.d, True)
        bt = bf / (ms["backward"] * 1e-3) / 1e12
        out["backward"] = {"TFLOP/s": round(bt, 2), "frac_bf16_peak": round(bt / PEAK_BF16_TFLOPS, 4),
                           "ms_per_call": round(ms["backward"], 4), "median_ms_per_call": round(med["backward"], 4),
                           "flops": bf}
        if out["value"] is None:
            out.update({"value": round(bt, 2), "unit": "TFLOP/s"})
    if "prefill_fp8" in parts:
        ff = prefill_flops(fc.B, fc.H, fc.N, fc.d, True)
        ft = ff / (ms["prefill_fp8"] * 1e-3) / 1e12
        out["prefill_fp8"] = {"TFLOP/s": round(ft, 2), "frac_fp8_peak": round(ft / PEAK_FP8_TFLOPS, 4),
                              "ms_per_call": round(ms["prefill_fp8"], 4),
                              "median_ms_per_call": round(med["prefill_fp8"], 4), "flops": ff}
        if out["value"] is None:
            out.update({"value": round(ft, 2), "unit": "TFLOP/s"})
    if "prefill_d64" in parts:
        f64_ = prefill_flops(c64.B, c64.H, c64.N, c64.d, True)
        t64 = f64_ / (ms["prefill_d64"] * 1e-3) / 1e12
        out["prefill_d64"] = {"TFLOP/s": round(t64, 2), "frac_bf16_peak": round(t64 / PEAK_BF16_TFLOPS, 4),
                              "ms_per_call": round(ms["prefill_d64"], 4), "flops": f64_}
        if out["value"] is None:
            out.update({"value": round(t64, 2), "unit": "TFLOP/s"})
    if "hstu_padded" in parts:
        out["hstu_padded"] = {"ms_per_call": round(ms["hstu_padded"], 4), "padded_to": jc.len_hi,
                              "sequences": len(jx.lengths)}
        if "hstu" in parts:
            out["hstu_padded"]["jagged_speedup"] = round(ms["hstu_padded"] / ms["hstu"], 3)
        if out["value"] is None:
            out.update({"value": round(ms["hstu_padded"], 4), "unit": "ms", "higher_is_better": False})
    if not args.only and not args.no_context and "prefill" in parts:
        print("bench: shader clock and power under the prefill", file=sys.stderr, flush=True)
        clk = clock_under_load(calls["prefill"])
        if clk.get("sclk_mhz"):
            peak_at = PEAK_BF16_TFLOPS * clk["sclk_mhz"] / (SPEC_CLOCK_HZ / 1e6)
            clk["peak_at_sclk"] = round(peak_at, 1)
            clk["frac_at_sclk"] = round(out["roofline"]["achieved"] / peak_at, 4)
        out["roofline"]["clock"] = clk
    if not args.only and not args.no_context:
        print("bench: context measurements", file=sys.stderr, flush=True)
        out["context"] = context_measurements(fa, W, bf16, dev, stream, q, k, v, o, lse, pc, dx, dc, dq, dk, dv, dsl,
                                              do, dlse)
    if not args.no_cpu_baseline:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(px, pc, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

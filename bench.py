"""Benchmark of the Momentum-Mamba selective scan on one MI355X.

One step = one msm_scan_fwd call over the Mamba-1.4B layer shape (Bt=4, L=4096, D=4096, N=16,
bf16 I/O with fp32 state, beta=0.9, alpha=1) with inputs already resident in HBM.  The line
reports its HBM roofline (algorithmic bytes over the kernel's time against 8 TB/s) and, as a
second figure, its VALU issue share; the median and minimum over 50 calls with the last-level
cache warm and flushed; the backward on its own workload (Bt=4, L=2048, D=2048, N=16, fp32);
one decode step (msm_scan_step, Bt=1024 sequences of the same layer shape) with its HBM
roofline; the tiny workload's latency; every other configuration of the measurement plan with
its workspace and device memory; and the fp64 oracle timed on the host cores (all of them, and
one) on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload m1p4b] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "fwd/bwd selective-scan state-updates/sec (Bt·L·D·N) + achieved HBM GB/s"
HBM_PEAK_GBS = 8000.0
# VALU issue slots per second from the published fp32 vector peak, 157.3 TFLOP/s: halved because
# packed FP32 is not used, halved again because an FMA counts two flops (= 256 CUs x 4 SIMDs x
# 16 lanes x 2.4 GHz)
FP32_VECTOR_PEAK_TFLOPS = 157.3
VALU_PEAK_TSLOTS = FP32_VECTOR_PEAK_TFLOPS / 2 / 2
# Issue slots the recurrence needs per state update: exp2 (v_exp_f32, half rate: 2 slots) plus
# delta*A, the write c*B, the velocity FMA, the hidden-state FMA and the readout FMA; the
# velocity FMA disappears when beta = 0.
SLOTS_PER_UPDATE = {True: 6, False: 7}


def alg_bytes_fwd(w: workloads.Workload, last_state: bool = False) -> int:
    s = 2 if w.io == "bf16" else 4
    b = w.Bt * w.L * (3 * w.D * s + 2 * w.N * s) + 4 * w.D * w.N
    if w.dskip:
        b += 4 * w.D
    if last_state:
        b += 8 * w.Bt * w.D * w.N
    return b


def alg_bytes_bwd(w: workloads.Workload) -> int:
    s = 2 if w.io == "bf16" else 4
    b = w.Bt * w.L * (5 * w.D * s + 4 * w.N * s) + 8 * w.D * w.N
    if w.dskip:
        b += 8 * w.D
    return b


def alg_bytes_step(w: workloads.Workload) -> int:
    """One decode step: the fp32 h and v states read and written, x / delta / z read and y
    written per channel, B and C per batch row, A, Dskip and the delta bias once."""
    s = 2 if w.io == "bf16" else 4
    return (16 * w.Bt * w.D * w.N + 4 * w.Bt * w.D * s + 2 * w.Bt * w.N * s + 4 * w.D * w.N
            + 8 * w.D)


def source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "selective_state_space_msm_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str):
    """HBM bytes per launch from the committed rocprof counter summary, if it was taken on the
    current kernel sources (else None)."""
    p = os.path.join(ROOT, "profiles", "traffic_%s.json" % name)
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


WARM_SECONDS = 0.2
last_warmup = 0  # warm-up calls run by the latest timed()


def timed(fn, stream, steps, warmup):
    """Run fn at least `warmup` times and for at least WARM_SECONDS of sustained work (the GPU
    raises its clocks only under sustained load: after an idle gap, a few milliseconds of
    warm-up time the kernels at lower clocks), then time `steps` calls with HIP events on
    `stream`.  Returns the mean duration per call in ms and the list of per-call durations;
    the number of warm-up calls run is left in last_warmup."""
    import torch
    n = 0
    for _ in range(warmup):
        fn()
        n += 1
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < WARM_SECONDS:
        for _ in range(8):
            fn()
        n += 8
        torch.cuda.synchronize()
    global last_warmup
    last_warmup = n
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    with torch.cuda.stream(stream):
        evs[0].record(stream)
        for i in range(steps):
            fn()
            evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    total = evs[0].elapsed_time(evs[-1])
    return total / steps, per


def per_call_ms(fn, stream, calls, flush=None):
    """Duration of each of `calls` calls of fn, from HIP events recorded on `stream` right
    before and after it.  flush: a function run before each call, outside the timed interval
    (it evicts the inputs from the last-level cache)."""
    import torch
    out = []
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    with torch.cuda.stream(stream):
        for a, b in ev:
            if flush is not None:
                flush()
            a.record(stream)
            fn()
            b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


_flush_buf = None


def cache_flush():
    """Write 1 GiB on the device: more than the 256 MB last-level cache holds."""
    import torch
    global _flush_buf
    if _flush_buf is None:
        _flush_buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    _flush_buf.fill_(1.0)


def timing_record(fn, stream, calls=50):
    """Median and minimum per-call time over `calls` calls, warm (back to back) and with the
    last-level cache flushed before each call."""
    warm = per_call_ms(fn, stream, calls)
    cold = per_call_ms(fn, stream, calls, flush=cache_flush)
    return {"calls": calls,
            "warm": {"median_ms": float(np.median(warm)), "min_ms": float(np.min(warm))},
            "flushed": {"median_ms": float(np.median(cold)), "min_ms": float(np.min(cold))}}


def nbytes_of(t):
    return 0 if t is None else t.numel() * t.element_size()


def to_dev(inp):
    import torch
    dt = torch.float32 if inp["io"] == "f32" else torch.bfloat16
    d = {}
    for k in ("x", "delta", "B", "C", "dy"):
        if inp.get(k) is not None:
            d[k] = torch.from_numpy(inp[k]).to("cuda").to(dt)
    d["A"] = torch.from_numpy(inp["A"]).to("cuda")
    d["Dskip"] = None if inp["Dskip"] is None else torch.from_numpy(inp["Dskip"]).to("cuda")
    return d


def bench_fwd(w, steps, warmup, stream, a_kind="s4d", fused=False, zoh=False):
    """Time msm_scan_fwd on workload w (fused: msm_selective_scan_fwd with a delta bias,
    softplus and the gate, on the raw-delta recipe of the fused op; zoh: also the zero-order
    hold)."""
    import torch
    import selective_state_space_msm_amd as msm
    inp = workloads.make_inputs(w, a_kind=a_kind, with_dy=False)
    g = to_dev(inp)
    if fused:
        ex = workloads.make_fused_extras(w, w.seed + 7)
        dt = g["x"].dtype
        g["delta"] = torch.from_numpy(ex["delta_raw"]).to("cuda").to(dt)
        g["z"] = torch.from_numpy(ex["z"]).to("cuda").to(dt)
        g["delta_bias"] = torch.from_numpy(ex["delta_bias"]).to("cuda")
    y = torch.empty_like(g["x"])
    nbytes = msm.msm_scan_fwd_workspace_bytes(w.Bt, w.L, w.D, w.N, w.io)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    plan = msm.msm_scan_fwd_plan(w.Bt, w.L, w.D, w.N, w.io, w.beta)

    def step():
        if fused:
            msm.msm_selective_scan_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], w.beta,
                                       w.alpha, g["Dskip"], z=g["z"], delta_bias=g["delta_bias"],
                                       delta_softplus=True, zero_order_hold=zoh, y=y,
                                       workspace=ws, stream=stream)
        else:
            msm.msm_scan_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], w.beta, w.alpha,
                             g["Dskip"], y=y, workspace=ws, stream=stream)

    ms, per = timed(step, stream, steps, warmup)
    mem = {"workspace_bytes": int(nbytes),
           "device_bytes": int(sum(nbytes_of(t) for t in list(g.values()) + [y]) + nbytes)}
    return ms, per, plan, step, mem


def bench_bwd(w, steps, warmup, stream, fused=False, zoh=False):
    """Time msm_scan_bwd on workload w (fused: msm_selective_scan_bwd with the fused op's extras,
    zoh: also the zero-order hold)."""
    import torch
    import selective_state_space_msm_amd as msm
    inp = workloads.make_inputs(w, with_dy=True)
    g = to_dev(inp)
    if fused:
        ex = workloads.make_fused_extras(w, w.seed + 7)
        dt = g["x"].dtype
        g["delta"] = torch.from_numpy(ex["delta_raw"]).to("cuda").to(dt)
        g["z"] = torch.from_numpy(ex["z"]).to("cuda").to(dt)
        g["delta_bias"] = torch.from_numpy(ex["delta_bias"]).to("cuda")
    nbytes = msm.msm_scan_bwd_workspace_bytes(w.Bt, w.L, w.D, w.N, w.io)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    out = {"dx": torch.empty_like(g["x"]), "ddelta": torch.empty_like(g["x"]),
           "dA": torch.empty_like(g["A"]), "dB": torch.empty_like(g["B"]),
           "dC": torch.empty_like(g["C"])}
    plan = msm.msm_scan_bwd_plan(w.Bt, w.L, w.D, w.N, w.io, w.beta)
    if zoh and 5 <= w.N <= 16:
        # the zero-order hold's documented choice: two states per wavefront half at 5-16 states
        # (the fused backward without it takes the plain backward's plan)
        plan = dict(plan, states_per_wave=2)

    if fused:
        out["dz"] = torch.empty_like(g["x"])
        out["ddelta_bias"] = torch.empty_like(g["delta_bias"])

    def step():
        if fused:
            msm.msm_selective_scan_bwd(g["x"], g["delta"], g["A"], g["B"], g["C"], g["dy"],
                                       w.beta, w.alpha, g["Dskip"], z=g["z"],
                                       delta_bias=g["delta_bias"], delta_softplus=True,
                                       zero_order_hold=zoh, out=out, workspace=ws, stream=stream)
        else:
            msm.msm_scan_bwd(g["x"], g["delta"], g["A"], g["B"], g["C"], g["dy"], w.beta,
                             w.alpha, g["Dskip"], out=out, workspace=ws, stream=stream)

    ms, per = timed(step, stream, steps, warmup)
    mem = {"workspace_bytes": int(nbytes),
           "device_bytes": int(sum(nbytes_of(t) for t in list(g.values()) + list(out.values()))
                               + nbytes)}
    return ms, per, plan, step, mem


def bench_step(w, steps, warmup, stream):
    import torch
    import selective_state_space_msm_amd as msm
    si = workloads.make_step_inputs(w)
    dt = torch.float32 if w.io == "f32" else torch.bfloat16
    g = {k: torch.from_numpy(si[k]).to("cuda").to(dt) for k in ("x", "delta", "z", "B", "C")}
    for k in ("A", "Dskip", "delta_bias", "h", "v"):
        g[k] = torch.from_numpy(si[k]).to("cuda")
    y = torch.empty_like(g["x"])

    def step():
        msm.msm_scan_step(g["x"], g["delta"], g["A"], g["B"], g["C"], g["h"], g["v"], w.beta,
                          w.alpha, g["Dskip"], z=g["z"], delta_bias=g["delta_bias"],
                          delta_softplus=True, y=y, stream=stream)

    return timed(step, stream, steps, warmup)


def bench_complex(w, steps, warmup, stream, direction):
    """Time msm_scan_complex_fwd or msm_scan_complex_bwd on workload w (complex A, B, C)."""
    import torch
    import selective_state_space_msm_amd as msm
    inp = workloads.make_complex_inputs(w, with_dy=direction == "bwd")
    dt = torch.float32 if w.io == "f32" else torch.bfloat16
    g = {k: torch.from_numpy(inp[k]).to("cuda").to(dt) for k in ("x", "delta", "B", "C")}
    g["A"] = torch.from_numpy(inp["A"]).to("cuda")
    if direction == "fwd":
        y = torch.empty_like(g["x"])

        def step():
            msm.msm_scan_complex_fwd(g["x"], g["delta"], g["A"], g["B"], g["C"], w.beta, w.alpha,
                                     y=y, stream=stream)
    else:
        g["dy"] = torch.from_numpy(inp["dy"]).to("cuda").to(dt)
        nbytes = msm.msm_scan_complex_bwd_workspace_bytes(w.Bt, w.L, w.D, w.N, w.io)
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        out = {"dx": torch.empty_like(g["x"]), "ddelta": torch.empty_like(g["x"]),
               "dA": torch.empty_like(g["A"]), "dB": torch.empty_like(g["B"]),
               "dC": torch.empty_like(g["C"])}

        def step():
            msm.msm_scan_complex_bwd(g["x"], g["delta"], g["A"], g["B"], g["C"], g["dy"], w.beta,
                                     w.alpha, out=out, workspace=ws, stream=stream)

    return timed(step, stream, steps, warmup)


def alg_bytes_complex(w: workloads.Workload, direction: str) -> int:
    """Bytes a complex call must move at least: x, delta, y (fwd) or x, delta, dy, dx, ddelta
    (bwd) per (b, t, d); B, C (fwd) or B, C, dB, dC (bwd) as (re, im) pairs per (b, t, n)."""
    es = 4 if w.io == "f32" else 2
    rows_d = w.Bt * w.L * w.D
    rows_n = w.Bt * w.L * w.N * 2
    if direction == "fwd":
        return es * (3 * rows_d + 2 * rows_n) + 8 * w.D * w.N
    return es * (5 * rows_d + 4 * rows_n) + 16 * w.D * w.N


def bench_configs(steps, warmup, stream, only=None):
    """Every other configuration the measurement plan lists, one line each: the complex scan
    forward and backward, the forward at each forward shape (both beta where listed), the
    forward with an unstructured A, the fused forward, and the README benchmark shape forward
    and backward."""
    W = workloads.WORKLOADS
    # (workload, direction, overrides, A, fused extras, zero-order hold)
    runs = [("m130m", "fwd", {}, "s4d", False, False),
            ("m130m", "fwd", {"beta": 0.0}, "s4d", False, False),
            ("m130m", "fwd", {}, "random", False, False),
            ("m1p4b", "fwd", {}, "random", False, False),
            ("m1p4b", "fwd", {}, "s4d", True, False), ("m1p4b", "fwd", {}, "s4d", True, True),
            ("long", "fwd", {}, "s4d", False, False),
            ("bwd", "bwd", {}, "s4d", True, False), ("bwd", "bwd", {}, "s4d", True, True),
            ("pages", "fwd", {}, "s4d", False, False),
            ("pages", "fwd", {"beta": 0.0}, "s4d", False, False),
            ("pages", "bwd", {}, "s4d", False, False),
            ("pages", "bwd", {"beta": 0.0}, "s4d", False, False)]
    out = []
    # the complex-valued scan (A = -1/2 + i pi n, complex B and C), forward and backward
    for direction in ("fwd", "bwd") if only is None or "complex" in only else ():
        w = W["complex"]
        ms, per = bench_complex(w, steps, warmup, stream, direction)
        out.append({"workload": "complex", "direction": direction, "beta": w.beta, "A": "s4d_lin",
                    "complex": True, "Bt": w.Bt, "L": w.L, "D": w.D, "N": w.N, "io": w.io,
                    "ms": ms, "ms_min": min(per), "state_updates_per_s": w.updates / (ms / 1e3),
                    "algorithmic_GBs": alg_bytes_complex(w, direction) / (ms / 1e3) / 1e9})
        import torch
        torch.cuda.empty_cache()
    for name, direction, kw, a_kind, fused, zoh in runs:
        if only is not None and name not in only:
            continue
        w = W[name].replace(**kw)
        if direction == "fwd":
            ms, per, plan, fn, mem = bench_fwd(w, steps, warmup, stream, a_kind=a_kind,
                                               fused=fused, zoh=zoh)
            nb = alg_bytes_fwd(w)
        else:
            ms, per, plan, fn, mem = bench_bwd(w, steps, warmup, stream, fused=fused, zoh=zoh)
            nb = alg_bytes_bwd(w)
        out.append({"workload": name, "direction": direction, "beta": w.beta, "A": a_kind,
                    "fused_extras": fused, "zero_order_hold": zoh, "Bt": w.Bt, "L": w.L,
                    "D": w.D, "N": w.N, "io": w.io,
                    "ms": ms, "ms_min": min(per), "state_updates_per_s": w.updates / (ms / 1e3),
                    "algorithmic_GBs": nb / (ms / 1e3) / 1e9, "hbm_frac":
                    nb / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, "plan": plan, "memory": mem})
        import torch
        torch.cuda.empty_cache()
    return out


def cpu_baseline(w, target_s=12.0):
    """The fp64 oracle, as it stands, on a bounded slice of the workload: every batch row and
    every step of a block of channels sized for roughly target_s seconds on the host cores."""
    import oracle
    threads = oracle.max_threads()
    inp = workloads.make_inputs(w.replace(D=64, L=min(w.L, 1024)), seed=w.seed + 7)
    t0 = time.perf_counter()
    oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], w.beta, w.alpha,
               Dskip=inp["Dskip"], threads=threads)
    probe_rate = w.Bt * inp["x"].shape[1] * 64 * w.N / (time.perf_counter() - t0)
    # channels so that the timed sample takes about target_s
    dsel = int(max(threads, min(w.D, target_s * probe_rate / (w.Bt * w.L * w.N))))
    sw = w.replace(D=dsel)
    inp = workloads.make_inputs(sw, seed=w.seed + 8)
    t0 = time.perf_counter()
    oracle.fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], w.beta, w.alpha,
               Dskip=inp["Dskip"], threads=threads)
    dt = time.perf_counter() - t0
    # one thread on the first batch row, a few channels sized for about a fifth of target_s
    ch1 = int(max(1, min(w.D, target_s / 5 * probe_rate / threads / (w.L * w.N))))
    w1 = w.replace(Bt=1, D=ch1)
    inp1 = workloads.make_inputs(w1, seed=w.seed + 9)
    t0 = time.perf_counter()
    oracle.fwd(inp1["x"], inp1["delta"], inp1["A"], inp1["B"], inp1["C"], w.beta, w.alpha,
               Dskip=inp1["Dskip"], threads=1)
    dt1 = time.perf_counter() - t0
    return {"value": sw.updates / dt, "unit": "state-updates/s", "cores": threads,
            "kind": "oracle",
            "sample": "fp64 C oracle forward, Bt=%d L=%d N=%d over %d of the %d channels "
                      "(%.3g state updates in %.1f s, OpenMP over channels)"
                      % (sw.Bt, sw.L, sw.N, dsel, w.D, sw.updates, dt),
            "one_thread": {"value": w1.updates / dt1, "unit": "state-updates/s", "cores": 1,
                           "sample": "batch row 0, L=%d N=%d, %d channels (%.3g state updates "
                                     "in %.1f s)" % (w1.L, w1.N, ch1, w1.updates, dt1)}}


def pmc_summary(fetch_csv, write_csv, kernel_substr, name, command):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) of
    `bench.py --calib-copy` into profiles/traffic_<name>.json.  Each counter is scaled by what
    it reads for the plain 256 MiB device copy of the same run (known bytes / counter)."""
    import csv

    def per_kernel(path, counter):
        vals, copies = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if kernel_substr in r["Kernel_Name"]:
                vals.append(v)
            elif "copyBuffer" in r["Kernel_Name"]:
                copies.append((int(r["Grid_Size"]), v))
        # the calibration copies are the largest copy dispatches of the run (small host-to-device
        # staging copies use the same kernel)
        big = max(g for g, _ in copies)
        return vals, [v for g, v in copies if g == big]

    fk, fcopy = per_kernel(fetch_csv, "FETCH_SIZE")
    wk, wcopy = per_kernel(write_csv, "WRITE_SIZE")
    copy_kib = (256 << 20) / 1024.0
    fscale = copy_kib / (sum(fcopy) / len(fcopy))
    wscale = copy_kib / (sum(wcopy) / len(wcopy))
    fetch = sum(fk) / len(fk) * fscale * 1024
    write = sum(wk) / len(wk) * wscale * 1024
    rec = {"kernel": kernel_substr, "source_hash": source_hash(),
           "fetch_KiB_per_dispatch": sum(fk) / len(fk), "write_KiB_per_dispatch": sum(wk) / len(wk),
           "fetch_scale": fscale, "write_scale": wscale, "hbm_bytes_per_launch": fetch + write,
           "dispatches": [len(fk), len(wk)], "command": command}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "traffic_%s.json" % name), "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="m1p4b", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--bwd-workload", default="bwd", choices=sorted(workloads.WORKLOADS) + ["none"])
    ap.add_argument("--step-workload", default="decode",
                    choices=[k for k, v in workloads.WORKLOADS.items() if v.direction == "step"]
                    + ["none"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations (m130m, long, README shape, ...)")
    ap.add_argument("--configs-only", default=None,
                    help="comma-separated workload names: run only their configuration lines")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=5, metavar=("FETCH_CSV", "WRITE_CSV", "KERNEL", "NAME",
                                                       "COMMAND"),
                    help="summarise two rocprofv3 counter runs into profiles/ and exit (no GPU)")
    args = ap.parse_args(argv)
    if args.pmc_summary:
        print(json.dumps(pmc_summary(*args.pmc_summary), indent=1))
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    stream = torch.cuda.current_stream()

    w = workloads.WORKLOADS[args.workload]
    if w.direction != "fwd":
        raise SystemExit("--workload must be a forward workload")
    ms, per, plan, fwd_fn, fwd_mem = bench_fwd(w, args.steps, args.warmup, stream)
    fwd_warmup_run = last_warmup
    sec = ms / 1e3
    beta0 = w.beta == 0.0
    slots = w.updates * SLOTS_PER_UPDATE[beta0]
    achieved_slots = slots / sec / 1e12
    abytes = alg_bytes_fwd(w)
    kname = "fwd_%s" % w.name
    rec = {
        "metric": METRIC,
        "value": w.updates / sec,
        "unit": "state-updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_run": fwd_warmup_run,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic the path computes in; the I/O dtype is config.io
        "dtype": "f32",
        "data": "synthetic (seeded; distributions of the workload recipe)",
        "config": {"workload": "%s: forward scan, Mamba-1.4B layer shape" % w.name if w.name == "m1p4b"
                   else "%s: forward scan" % w.name,
                   "Bt": w.Bt, "L": w.L, "D": w.D, "N": w.N, "io": w.io, "state": "f32",
                   "beta": w.beta, "alpha": w.alpha, "dskip": w.dskip, "plan": plan},
        # the forward is one kernel at this shape: the call's time on its stream is the kernel's
        "roofline": {"bound": "hbm", "achieved": abytes / sec / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": abytes / sec / 1e9 / HBM_PEAK_GBS,
                     "traffic": measured_traffic(kname), "algorithmic_bytes": abytes,
                     "kernel_ms_mean": ms, "kernel_ms_min": min(per)},
        "alu": {"achieved": achieved_slots, "peak": VALU_PEAK_TSLOTS,
                "unit": "T VALU lane-slots/s", "frac": achieved_slots / VALU_PEAK_TSLOTS,
                "slots_per_update": SLOTS_PER_UPDATE[beta0],
                "peak_from": "157.3 TFLOP/s fp32 vector / 2 (no packed FP32) / 2 (FMA)"},
        "memory": fwd_mem,
    }
    rec["timing"] = timing_record(fwd_fn, stream)
    if args.bwd_workload != "none":
        wb = workloads.WORKLOADS[args.bwd_workload]
        bms, bper, bplan, bwd_fn, bwd_mem = bench_bwd(wb, max(3, args.steps // 2),
                                                      max(1, args.warmup // 2), stream)
        bbytes = alg_bytes_bwd(wb)
        rec["bwd"] = {"workload": "%s: backward, Bt=%d L=%d D=%d N=%d io=%s beta=%g"
                                  % (wb.name, wb.Bt, wb.L, wb.D, wb.N, wb.io, wb.beta),
                      "ms_per_call": bms, "state_updates_per_s": wb.updates / (bms / 1e3),
                      "algorithmic_GBs": bbytes / (bms / 1e3) / 1e9,
                      "hbm_frac": bbytes / (bms / 1e3) / 1e9 / HBM_PEAK_GBS, "plan": bplan,
                      "traffic": measured_traffic("bwd_%s" % wb.name), "memory": bwd_mem,
                      "timing": timing_record(bwd_fn, stream)}
        del bwd_fn
        import torch
        torch.cuda.empty_cache()
    # latency of the smallest workload (launch-bound): median and minimum over 50 calls
    wt = workloads.WORKLOADS["tiny"]
    _, tper, tplan, tiny_fn, tiny_mem = bench_fwd(wt, 10, 10, stream)
    tt = per_call_ms(tiny_fn, stream, 50)
    rec["latency_tiny"] = {"workload": "tiny: forward, Bt=1 L=64 D=4 N=4 io=f32 beta=0.9",
                           "median_ms": float(np.median(tt)), "min_ms": float(np.min(tt)),
                           "calls": 50, "plan": tplan, "memory": tiny_mem}
    if args.step_workload != "none":
        ws_ = workloads.WORKLOADS[args.step_workload]
        sms, sper = bench_step(ws_, max(5, args.steps), max(2, args.warmup // 2), stream)
        sbytes = alg_bytes_step(ws_)
        rec["decode"] = {"workload": "%s: one decode step with bias, softplus and gate, Bt=%d D=%d "
                                     "N=%d io=%s" % (ws_.name, ws_.Bt, ws_.D, ws_.N, ws_.io),
                         "ms_per_call": sms, "state_updates_per_s": ws_.Bt * ws_.D * ws_.N / (sms / 1e3),
                         "roofline": {"bound": "hbm", "achieved": sbytes / (sms / 1e3) / 1e9,
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": sbytes / (sms / 1e3) / 1e9 / HBM_PEAK_GBS,
                                      "traffic": measured_traffic("step_%s" % ws_.name),
                                      "algorithmic_bytes": sbytes}}
    if not args.calib_copy:
        # practical streaming rate of the box: a 1 GiB device-to-device copy (read + write),
        # a second denominator next to the 8 TB/s peak (left out of counter runs, whose only
        # copy must be the calibration copy)
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        cms, _ = timed(lambda: dst.copy_(src), stream, 10, 3)
        rec["roofline"]["copy_probe_GBs"] = 2 * src.numel() / (cms / 1e3) / 1e9
        del src, dst
        torch.cuda.empty_cache()
    if not args.no_configs:
        only = None if args.configs_only is None else set(args.configs_only.split(","))
        rec["configs"] = bench_configs(max(5, args.steps // 2), max(3, args.warmup // 2), stream,
                                       only)
    if args.calib_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        rec["calib_copy_bytes"] = 2 * src.numel()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

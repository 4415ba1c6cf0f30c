#!/usr/bin/env python3
"""Benchmark of the Axon-SSM selective-scan prefill on one MI355X.

One step = one call of axon_ssm_prefill over one batch of synthetic input (every step of the hot
path: conv, dt, scan, readout, gate, cache/state outputs). The default workload is the Axon-SSM
layer shape the metric is quoted on: batch 1, L = 2048, E = 7680, N = 16, K = 4, fp32.
Inputs are resident in HBM before timing starts; several input sets are rotated so that each step
reads data that is not left in the 256 MB last-level (Infinity) cache by the previous step.

Prints one JSON line (rank 0). Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "selective-scan tokens/s at E=7680,N=16,L=2048 + % of HBM peak GB/s"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E peak, 8 TB/s
N_STATE, K_CONV = 16, 4
COPY_BYTES = 512 << 20  # calibration copy: 512 MiB read + 512 MiB written per dispatch


def algorithmic_bytes(Bsz, L, E, elt, with_cache_in=False, with_state_in=False):
    """Bytes the method itself must move for one prefill: x, z, dt_raw, B, C read once, y written
    once, parameters read once, final state and conv cache written (and read when given)."""
    act = 3 * Bsz * L * E * elt + 2 * Bsz * L * N_STATE * elt + Bsz * L * E * elt
    prm = 4 * (E * N_STATE + 3 * E + E * K_CONV)
    out = 4 * (Bsz * E * N_STATE + Bsz * (K_CONV - 1) * E)
    inn = (4 * Bsz * (K_CONV - 1) * E if with_cache_in else 0) + \
        (4 * Bsz * E * N_STATE if with_state_in else 0)
    return act + prm + out + inn


def decode_algorithmic_bytes(Bsz, E, elt):
    """Bytes one decode step must move: x, z, dt_raw read and y written (B, E); B, C (B, N);
    the conv cache and the state read and written in place (fp32); parameters read once."""
    act = 4 * Bsz * E * elt + 2 * Bsz * N_STATE * elt
    caches = 2 * 4 * (Bsz * (K_CONV - 1) * E + Bsz * E * N_STATE)
    prm = 4 * (E * N_STATE + 3 * E + E * K_CONV)
    return act + caches + prm


def calibrate_copy(steps):
    """A plain device-to-device copy of a known size, for scaling rocprofv3's FETCH_SIZE and
    WRITE_SIZE counters (KiB per dispatch) into bytes: each dispatch reads and writes
    COPY_BYTES."""
    import torch

    dev = torch.device("cuda:0")
    n = COPY_BYTES // 4
    src = torch.arange(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_dispatch": COPY_BYTES,
                      "bytes_written_per_dispatch": COPY_BYTES, "dispatches": steps}), flush=True)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, min_seconds=10.0, single_seconds=3.0):
    """The oracle as it is (test infrastructure), timed on the host cores over whole passes of the
    same workload until min_seconds have elapsed, with as many threads as the process may use (at
    most 16, a one-GPU share of the host); then single-threaded on each of the first two cores
    the process may use, over the leading channels of the workload (the oracle's cost is linear
    in channels), for about single_seconds each."""
    import oracle

    avail = sorted(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else []
    nproc = len(avail) or (os.cpu_count() or 1)
    threads = min(16, nproc)
    Bsz, L, E = inp["x"].shape
    oracle.prefill({k: (v[:, :8] if k in ("x", "z", "dt_raw", "B", "C") else v)
                    for k, v in inp.items()}, threads=threads)  # load / warm up
    passes = 0
    t0 = time.perf_counter()
    while True:
        oracle.prefill(inp, threads=threads)
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    out = {"value": passes * Bsz * L / el, "unit": "tokens/s", "cores": threads,
           "kind": "oracle",
           "sample": f"whole workload ({Bsz}x{L}x{E}), {passes} passes in {el:.1f} s, "
                     f"{threads} threads over channels, double precision",
           "nproc": nproc, "os_cpu_count": os.cpu_count(), "cpu_model": _cpu_model()}

    # Single thread, pinned: time a slice of channels, grown until it takes single_seconds.
    def channel_slice(ec):
        d = dict(inp)
        for k in ("x", "z", "dt_raw"):
            d[k] = np.ascontiguousarray(inp[k][:, :, :ec])
        for k in ("A_log", "D", "dt_bias", "conv_w", "conv_b"):
            d[k] = np.ascontiguousarray(inp[k][:ec])
        return d

    single = {}
    cores = avail[:2] if len(avail) >= 2 else avail
    if cores and hasattr(os, "sched_setaffinity"):
        try:
            for cpu in cores:
                os.sched_setaffinity(0, {cpu})
                ec = max(1, min(E, 8))
                while True:
                    d = channel_slice(ec)
                    t0 = time.perf_counter()
                    oracle.prefill(d, threads=1)
                    el = time.perf_counter() - t0
                    if el >= single_seconds or ec == E:
                        break
                    ec = min(E, max(ec * 2, int(ec * single_seconds / max(el, 1e-3))))
                # tokens/s of the whole workload: the slice's rate scaled by its share of channels
                single[f"c{cpu}"] = {"value": Bsz * L * (ec / E) / el, "unit": "tokens/s",
                                     "sample": f"{Bsz}x{L}x{ec} (of {E} channels), {el:.2f} s, "
                                               f"1 thread pinned to CPU {cpu}"}
        finally:
            os.sched_setaffinity(0, set(avail))
    out["single_thread"] = single
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 50; a decode workload: its step count, 256)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="axon_prefill_f32_b1_l2048_e7680")
    ap.add_argument("--rotate", type=int, default=3, help="input sets cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run only a plain device copy of known size (counter calibration)")
    ap.add_argument("--conv-activation", default="none", choices=["none", "silu"],
                    help="variant: SiLU on the convolution output (Mamba block)")
    ap.add_argument("--discretization", default="first_order", choices=["first_order", "zoh"],
                    help="variant: exact zero-order hold")
    ap.add_argument("--layer", type=int, default=0, metavar="D_MODEL",
                    help="time the whole layer (projections + path) with this d_model instead")
    ap.add_argument("--ssd", default="", metavar="WORKLOAD",
                    help="time the Mamba-2 SSD core instead (e.g. mamba2_ssd_f32_b1_l2048_h64)")
    ap.add_argument("--micro", action="store_true",
                    help="run only the instruction and HBM microbenchmarks (libaxonmicro.so)")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per launch (from rocprofv3 counters), if present")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); every (b, e) channel "
              "is independent, so the path shards over batch and channels with no exchange; run "
              "one process per GPU on its own share.", file=sys.stderr)
        sys.exit(2)

    if args.steps is None:
        wl = None if args.ssd else workloads.workload(args.workload)
        args.steps = wl.decode_steps if wl is not None and wl.kind == "decode" else 50
    if args.calibrate_copy:
        calibrate_copy(args.steps)
        return
    if args.micro:
        bench_micro()
        return

    import torch

    import selective_state_space_depthwise_amd as axon

    if args.ssd:
        bench_ssd(args, next(x for x in workloads.SSD_WORKLOADS if x.name == args.ssd))
        return
    w = workloads.workload(args.workload)
    if args.layer:
        bench_layer(args, w)
        return
    if w.kind == "decode":
        bench_decode(args, w)
        return
    variant = {"conv_activation": args.conv_activation, "discretization": args.discretization}
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    adt = torch.bfloat16 if w.act == "bf16" else torch.float32
    elt = 2 if w.act == "bf16" else 4
    Bsz, L, E = w.batch, w.seqlen, w.d_inner

    inp0 = workloads.prefill_inputs(w)
    prm = {k: torch.from_numpy(inp0[k]).to(dev) for k in ("A_log", "D", "dt_bias", "conv_w",
                                                         "conv_b")}
    sets = []
    for r in range(args.rotate):
        inp = inp0 if r == 0 else workloads.prefill_inputs(w, seed_offset=r)
        s = {k: torch.from_numpy(inp[k]).to(dev).to(adt) for k in ("x", "z", "dt_raw", "B", "C")}
        s["y"] = torch.empty_like(s["x"])
        s["cache"] = torch.empty((Bsz, K_CONV - 1, E), dtype=torch.float32, device=dev)
        s["state"] = torch.empty((Bsz, E, N_STATE), dtype=torch.float32, device=dev)
        sets.append(s)
    ws_bytes = axon.prefill_workspace_bytes(Bsz, L, E, w.act == "bf16")
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s = sets[i % len(sets)]
        axon.prefill(s["x"], s["z"], s["dt_raw"], s["B"], s["C"], prm["A_log"], prm["D"],
                     prm["dt_bias"], prm["conv_w"], prm["conv_b"], dt_min=inp0["dt_min"],
                     dt_max=inp0["dt_max"], y=s["y"], conv_cache_out=s["cache"],
                     ssm_state_out=s["state"], workspace=ws, stream=stream, **variant)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region: K steps, bracketed by synchronisation, with one pair of HIP events on the
    # launch stream around them: the mean launch duration is their span over K (events around
    # every call would put their own packets between the calls).
    e_start = torch.cuda.Event(enable_timing=True)
    e_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = e_start.elapsed_time(e_end)

    ms_per_step = wall * 1e3 / args.steps
    # After the timed region: the spread of single calls (events around each, same rotation).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(args.warmup + args.steps + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ev_ms = np.array([a.elapsed_time(b) for a, b in ev])
    # After the timed region: the same input set back to back, so its inputs may sit in the
    # 256 MB last-level cache (reported beside, never as the value).
    warm = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(10)]
    for i in range(10):
        warm[i][0].record(stream)
        step(0)
        warm[i][1].record(stream)
    torch.cuda.synchronize()
    warm_ms = float(np.median([a.elapsed_time(b) for a, b in warm]))
    tokens = Bsz * L
    value = tokens / (ms_per_step / 1e3)
    alg = algorithmic_bytes(Bsz, L, E, elt)
    launch_ms = region_ms / args.steps
    achieved = alg / (launch_ms / 1e3) / 1e9
    traffic = None
    if os.path.exists(args.traffic_json):
        with open(args.traffic_json) as f:
            tj = json.load(f)
        entry = tj.get(w.name)
        default_variant = variant == {"conv_activation": "none", "discretization": "first_order"}
        if entry and default_variant and entry.get("kernel_source_sha") == _kernel_source_sha():
            traffic = entry.get("bytes_per_launch")
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.act,
        "data": "synthetic (seeded normal draws, Axon-SSM init for A_log and dt bias)",
        "config": {"workload": w.name, "batch": Bsz, "seq_len": L, "d_inner": E,
                   "d_state": N_STATE, "d_conv": K_CONV, "act_dtype": w.act,
                   "input_sets_rotated": args.rotate, **variant},
        "hbm_gbps": round(achieved, 1),
        "pct_hbm_peak": round(100.0 * achieved / HBM_PEAK_GBPS, 2),
        "event_ms": {"mean": round(launch_ms, 5),
                     "single_call": {"mean": round(float(ev_ms.mean()), 5),
                                     "min": round(float(ev_ms.min()), 5),
                                     "median": round(float(np.median(ev_ms)), 5)},
                     "warm_same_inputs_median": round(warm_ms, 5)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": alg},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp0)
    print(json.dumps(line), flush=True)


def bench_decode(args, w):
    """One step = one axon_ssm_decode_step over the whole batch (one token per sequence); the
    caches are seeded by a prefill of the workload's prompt length and updated in place."""
    import torch

    import selective_state_space_depthwise_amd as axon

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    adt = torch.bfloat16 if w.act == "bf16" else torch.float32
    elt = 2 if w.act == "bf16" else 4
    Bsz, E = w.batch, w.d_inner
    inp0 = workloads.prefill_inputs(w)
    t = {k: torch.from_numpy(inp0[k]).to(dev) for k in ("A_log", "D", "dt_bias", "conv_w",
                                                       "conv_b")}
    pre = {k: torch.from_numpy(inp0[k]).to(dev).to(adt) for k in ("x", "z", "dt_raw", "B", "C")}
    _, cache, state = axon.prefill(pre["x"], pre["z"], pre["dt_raw"], pre["B"], pre["C"],
                                   t["A_log"], t["D"], t["dt_bias"], t["conv_w"], t["conv_b"],
                                   dt_min=inp0["dt_min"], dt_max=inp0["dt_max"])
    nsets = max(1, min(args.rotate * 8, w.decode_steps or 1))
    steps_in = []
    for s_ in range(nsets):
        st = workloads.decode_step_inputs(w, s_)
        steps_in.append({k: torch.from_numpy(st[k]).to(dev).to(adt) for k in st})
    y = torch.empty((Bsz, E), dtype=adt, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        st = steps_in[i % nsets]
        axon.decode_step(st["x"], st["z"], st["dt_raw"], st["B"], st["C"], t["A_log"], t["D"],
                         t["dt_bias"], t["conv_w"], t["conv_b"], cache, state,
                         dt_min=inp0["dt_min"], dt_max=inp0["dt_max"], y=y, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The same K steps issued one call at a time (host-bound: each call costs more host time than
    # the kernel takes), reported beside the graph figure.
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # A serving loop issues decode steps back to back; one call costs more host time than GPU
    # time, so the K timed steps are captured once in a HIP graph (one kernel per step, no
    # memset or allocation inside) and replayed: the events then time the kernels, not Python.
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream(dev)
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.steps):
                st = steps_in[(args.warmup + i) % nsets]
                axon.decode_step(st["x"], st["z"], st["dt_raw"], st["B"], st["C"], t["A_log"],
                                 t["D"], t["dt_bias"], t["conv_w"], t["conv_b"], cache, state,
                                 dt_min=inp0["dt_min"], dt_max=inp0["dt_max"], y=y, stream=cap)
    stream.wait_stream(cap)
    graph.replay()  # untimed: first replay
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = np.array([e0.elapsed_time(e1) / args.steps])
    ms_per_step = wall * 1e3 / args.steps
    alg = decode_algorithmic_bytes(Bsz, E, elt)
    launch_ms = float(ev_ms.mean())
    achieved = alg / (launch_ms / 1e3) / 1e9
    line = {
        "metric": "decode tokens/s (one token per sequence per step)",
        "value": round(Bsz / (ms_per_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.act,
        "data": "synthetic (seeded normal draws; caches from a seeded prefill)",
        "config": {"workload": w.name, "batch": Bsz, "d_inner": E, "d_state": N_STATE,
                   "d_conv": K_CONV, "prompt_tokens": w.seqlen, "act_dtype": w.act},
        "event_ms": {"mean": round(launch_ms, 5), "min": round(float(ev_ms.min()), 5),
                     "median": round(float(np.median(ev_ms)), 5)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": alg,
                     "note": "state and cache (B E (N + 3) fp32) stay in the last-level cache "
                             "between steps; steps replayed from one captured HIP graph, event "
                             "time of the replay / steps"},
        "eager_ms_per_step": round(eager_ms, 5),
    }
    print(json.dumps(line), flush=True)


def bench_layer(args, w):
    """One step = one forward of the whole layer (input projection, convolution, selection
    projection, scan and gate, output projection) over the workload's batch and sequence, with
    random-initialised weights of the Axon-SSM layer configuration (d_model = --layer)."""
    import torch

    import selective_state_space_depthwise_amd as axon

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    adt = torch.bfloat16 if w.act == "bf16" else torch.float32
    Dm = args.layer
    inp = workloads.layer_inputs(w, Dm)
    d = {k: torch.from_numpy(inp[k]).to(dev).to(adt) for k in ("x_in", "W_in", "W_f", "W_out")}
    d.update({k: torch.from_numpy(inp[k]).to(dev) for k in ("A_log", "D", "dt_bias", "conv_w",
                                                            "conv_b")})
    Bsz, L, E = w.batch, w.seqlen, w.d_inner
    out = torch.empty_like(d["x_in"])
    cache = torch.empty((Bsz, K_CONV - 1, E), dtype=torch.float32, device=dev)
    state = torch.empty((Bsz, E, N_STATE), dtype=torch.float32, device=dev)
    layer = axon.Layer()
    stream = torch.cuda.current_stream(dev)
    variant = {"conv_activation": args.conv_activation, "discretization": args.discretization}

    def step():
        layer.forward(d["x_in"], d["W_in"], d["W_f"], d["W_out"], d["A_log"], d["D"],
                      d["dt_bias"], d["conv_w"], d["conv_b"], dt_min=inp["dt_min"],
                      dt_max=inp["dt_max"], out=out, conv_cache_out=cache, ssm_state_out=state,
                      stream=stream, **variant)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = np.array([a.elapsed_time(b) for a, b in ev])
    M = Bsz * L
    flops = 2.0 * M * (2 * E * Dm + (2 * N_STATE + E) * E + Dm * E)
    launch_ms = float(ev_ms.mean())
    tflops = flops / (launch_ms / 1e3) / 1e12
    peak = 2500.0 if w.act == "bf16" else 157.3
    ms_per_step = wall * 1e3 / args.steps
    line = {
        "metric": "Axon-SSM layer forward tokens/s (projections + selective-scan path)",
        "value": round(M / (ms_per_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.act,
        "data": "synthetic (seeded normal draws, random-initialised projection weights)",
        "config": {"workload": w.name + "_layer", "batch": Bsz, "seq_len": L, "d_model": Dm,
                   "d_inner": E, "d_state": N_STATE, "d_conv": K_CONV, **variant},
        "event_ms": {"mean": round(launch_ms, 5), "min": round(float(ev_ms.min()), 5),
                     "median": round(float(np.median(ev_ms)), 5)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(tflops / peak, 4), "traffic": None,
                     "flops_per_launch": flops,
                     "note": "projection GEMM flops over the whole layer's time"},
    }
    layer.close()
    print(json.dumps(line), flush=True)


def ssd_algorithmic_flops(Bsz, L, H, P=64, N=128, Q=64):
    """Multiply-add flops (2 per product) of the chunked SSD form per call: per (batch, chunk)
    the lower block triangle of C B^T (10 of 16 16x16 blocks over N); per (batch, head, chunk)
    the chunk state x^T diag(w) B (P x N over Q), the incoming-state readout C H^T (Q x P over
    N) and the lower block triangle of the masked (C B^T) times x (10 of 16 blocks, over Q)."""
    nc = -(-L // Q)
    gram = 10 * 16 * 16 * N * 2
    per_head = P * N * Q * 2 + Q * P * N * 2 + 10 * 16 * 16 * P * 2
    return Bsz * nc * (gram + H * per_head)


def bench_ssd(args, w):
    """One step = one axon_ssd_scan call (four kernels: C B^T per chunk, chunk states, the
    recurrence over chunks, outputs) over the workload's batch, from a zero state."""
    import torch

    import selective_state_space_depthwise_amd as axon

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    adt = torch.bfloat16 if w.act == "bf16" else torch.float32
    elt = 2 if w.act == "bf16" else 4
    Bsz, L, H = w.batch, w.seqlen, w.heads
    inp0 = workloads.ssd_inputs(w)
    prm = {k: torch.from_numpy(inp0[k]).to(dev) for k in ("A_log", "D", "dt_bias")}
    sets = []
    for r in range(args.rotate):
        inp = inp0 if r == 0 else workloads.ssd_inputs(w, seed_offset=r)
        s = {k: torch.from_numpy(inp[k]).to(dev).to(adt) for k in ("x", "dt_raw", "B", "C")}
        s["y"] = torch.empty_like(s["x"])
        s["state"] = torch.empty((Bsz, H, 64, 128), dtype=torch.float32, device=dev)
        sets.append(s)
    ws = torch.empty(max(axon.ssd_workspace_bytes(Bsz, L, H, w.act == "bf16"), 1),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        s = sets[i % len(sets)]
        axon.ssd_scan(s["x"], s["dt_raw"], s["B"], s["C"], prm["A_log"], prm["D"],
                      prm["dt_bias"], dt_min=inp0["dt_min"], dt_max=inp0["dt_max"], y=s["y"],
                      state_out=s["state"], workspace=ws, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(args.warmup + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = np.array([a.elapsed_time(b) for a, b in ev])
    launch_ms = float(ev_ms.mean())
    flops = ssd_algorithmic_flops(Bsz, L, H)
    tflops = flops / (launch_ms / 1e3) / 1e12
    hbm = elt * (2 * Bsz * L * H * 64 + Bsz * L * H + 2 * Bsz * L * 128) + 4 * Bsz * H * 64 * 128
    ms_per_step = wall * 1e3 / args.steps
    line = {
        "metric": "Mamba-2 SSD core tokens/s (64 heads x 64, d_state 128)",
        "value": round(Bsz * L / (ms_per_step / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded normal draws, A in [-16, -1], dt in [1e-3, 0.1] + N(0,1) raw)",
        "config": {"workload": w.name, "batch": Bsz, "seq_len": L, "n_heads": H, "head_dim": 64,
                   "d_state": 128, "chunk": 64, "act_dtype": w.act,
                   "input_sets_rotated": args.rotate},
        "event_ms": {"mean": round(launch_ms, 5), "min": round(float(ev_ms.min()), 5),
                     "median": round(float(np.median(ev_ms)), 5)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": 157.3,
                     "unit": "TFLOP/s", "frac": round(tflops / 157.3, 4),
                     "traffic": _measured_traffic(args.traffic_json, w.name, _ssd_source_sha()),
                     "flops_per_launch": flops,
                     "note": "fp32 matrix-core flops of the chunked form over the whole call "
                             "(four kernels)"},
        "hbm_gbps_of_call": round(hbm / (launch_ms / 1e3) / 1e9, 1),
    }
    if not args.no_cpu_baseline:
        import oracle

        threads = min(16, os.cpu_count() or 1)
        Ls = 128
        sample = {k: (v[:, :Ls] if k in ("x", "dt_raw", "B", "C") else v) for k, v in inp0.items()}
        oracle.ssd_scan({k: (v[:, :4] if k in ("x", "dt_raw", "B", "C") else v)
                         for k, v in inp0.items()}, threads=threads)
        passes, t0 = 0, time.perf_counter()
        while True:
            oracle.ssd_scan(sample, threads=threads)
            passes += 1
            el = time.perf_counter() - t0
            if el >= 10.0:
                break
        line["cpu_baseline"] = {
            "value": round(passes * Bsz * Ls / el, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "sample": f"first {Ls} tokens of the workload, all {H} heads, "
                                        f"{passes} passes in {el:.1f} s, double precision"}
    print(json.dumps(line), flush=True)


MICRO_KINDS = ["fma", "exp", "dpp_row_newbcast_mul", "permlane32_swap", "state_update_mix",
               "exp_1_per_4_fma", "fma_plus_salu", "fma_dependent_chain", "exp_dependent_chain",
               "permlane16_swap", "exp_1_per_1_fma", "exp_1_per_2_fma", "exp_1_per_8_fma",
               "lane_per_channel_update", "lane_per_channel_update_exp_as_mul",
               "16_exp_then_48_fma", "8_exp_then_24_fma_twice", "16_exp_then_48_fma_vop3",
               "fma_sgpr_operand", "one_chain_update_exp_read_2_later",
               "one_chain_update_decay_one_token_ahead", "one_chain_exps_grouped_then_dpp",
               "one_chain_exps_grouped_then_plain"]


def bench_micro():
    """Issue cost per wave64 instruction on one SIMD (cycles at the clock measured in the kernel
    and at the nominal 2.4 GHz) for 1, 2 and 4 waves per SIMD, and HBM GB/s of a plain copy and a
    plain read (libaxonmicro.so). One JSON line."""
    import ctypes

    from selective_state_space_depthwise_amd import build as _b

    if not os.path.exists(_b.MICRO_LIB):
        raise RuntimeError(f"{_b.MICRO_LIB} is missing: run python -m "
                           "selective_state_space_depthwise_amd.build")
    lib = ctypes.CDLL(_b.MICRO_LIB)
    lib.axon_micro_alu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_double)]
    lib.axon_micro_hbm.argtypes = [ctypes.c_int, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_double)]
    simds = 256 * 4
    out = (ctypes.c_double * 3)()
    alu = {}
    clock_ghz = []
    for kind, name in enumerate(MICRO_KINDS):
        per = lib.axon_micro_alu_instrs_per_iter(kind)
        alu[name] = {}
        for wps in (1, 2, 4):
            iters = 2000
            rc = lib.axon_micro_alu(kind, wps, iters, out)
            if rc:
                raise RuntimeError(f"micro {name} wps {wps}: hip error {rc}")
            ms, tick, rtick = out[0], out[1], out[2]
            ghz = tick / (rtick / 100e6) / 1e9 if rtick else float("nan")
            clock_ghz.append(ghz)
            instrs = iters * per * wps  # wave64 instructions issued per SIMD
            ns = ms * 1e6 / instrs
            alu[name][f"{wps}_wave_per_simd"] = {
                "ns_per_instr": round(ns, 4), "cycles_at_2.4GHz": round(ns * 2.4, 3),
                "cycles_at_measured_clock": round(ns * ghz, 3), "ms": round(ms, 4)}
        print(f"micro {name} done", file=sys.stderr, flush=True)
    hbm = {}
    for kind, name in ((0, "copy"), (1, "read")):
        nbytes = 1 << 30
        for blocks in (2048, 8192):
            rc = lib.axon_micro_hbm(kind, nbytes, 10, blocks, out)
            if rc:
                raise RuntimeError(f"micro hbm {name}: hip error {rc}")
            moved = nbytes * (2 if kind == 0 else 1)
            hbm[f"{name}_{blocks}_workgroups"] = {
                "GB_per_s": round(moved / (out[0] / 1e3) / 1e9, 1), "ms": round(out[0], 4),
                "bytes_moved": moved}
    # The row scan's activation reads: lane rows of 16 lanes reading 64-, 128- or 256-byte
    # segments of one token, 240 workgroups of 8 waves, 2048 x 7680 fp32 (and the same bytes
    # at 2 and 4 x the channels).
    for kind, seg in ((2, 64), (3, 128), (4, 256)):
        nbytes = 2048 * 7680 * 4
        rc = lib.axon_micro_hbm(kind, nbytes, 20, 1, out)
        if rc:
            raise RuntimeError(f"micro hbm segment {seg}: hip error {rc}")
        hbm[f"row_pattern_read_{seg}B_segments"] = {
            "GB_per_s": round(nbytes / (out[0] / 1e3) / 1e9, 1), "ms": round(out[0], 4),
            "bytes_moved": nbytes}
    # LDS: bytes delivered per CU clock (the measured clock) for each lane pattern.
    lib.axon_micro_lds.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.POINTER(ctypes.c_double)]
    ghz = float(np.median(clock_ghz))
    lds = {}
    for kind, name, nbytes in ((0, "read_b128_distinct", 1024), (1, "read_b128_row_broadcast", 1024),
                               (2, "read_b128_all_same", 1024), (3, "write_b128_distinct", 1024)):
        lds[name] = {}
        for wps in (1, 2, 4):
            iters = 4000
            rc = lib.axon_micro_lds(kind, wps, iters, out)
            if rc:
                raise RuntimeError(f"micro lds {name}: hip error {rc}")
            instrs_per_cu = iters * 16 * 4 * wps
            cycles = out[0] * 1e-3 * ghz * 1e9
            lds[name][f"{wps}_wave_per_simd"] = {
                "cu_cycles_per_instr": round(cycles / instrs_per_cu, 3),
                "bytes_per_cu_cycle": round(nbytes * instrs_per_cu / cycles, 1),
                "ms": round(out[0], 4)}
    print(json.dumps({"micro": "gfx950 instruction issue, LDS and HBM streaming",
                      "s_memtime_clock_GHz": round(float(np.median(clock_ghz)), 4),
                      "simds": simds, "alu": alu, "lds": lds, "hbm": hbm}), flush=True)


def _measured_traffic(path, name, sha):
    """HBM bytes per call measured by rocprofv3 counters (profiles/traffic.json), if they were
    taken on the current kernel sources; else None."""
    if not os.path.exists(path):
        return None
    with open(path) as f:
        entry = json.load(f).get(name)
    if entry and entry.get("kernel_source_sha") == sha:
        return entry.get("bytes_per_launch")
    return None


def _ssd_source_sha():
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_depthwise_amd", "csrc")
    for name in ("axon_device.h", "axon_ssd.hip"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def _kernel_source_sha():
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_depthwise_amd", "csrc")
    # the sources the prefill kernels are built from
    for name in ("axon_device.h", "axon_internal.h", "axon_kernels.hip", "axon_rowscan.hip",
                 "axon_chanscan.hip", "axonscan_api.cpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()

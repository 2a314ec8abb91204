#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

One step = one full-sequence scan (mamba_scan_fwd) of the Mamba-2.8B-shaped
prefill layer: batch 8, 5,120 channels, 2,048 tokens, 16 states, bf16 inputs,
fp32 state, with bias, softplus, D skip and silu(z) gate. Inputs are seeded
synthetic tensors already resident in HBM; the timed region holds exactly
--steps calls bracketed by device synchronisation.

Two input sets are alternated between calls, so consecutive calls do not
find their inputs in the caches.

Prints one JSON line. `value` is elem-steps/s (batch * L * channels per
second). `roofline` relates the scan call's algorithmic fp32 operations to
the published fp32 vector-ALU peak (the scan is bound by vector-ALU issue),
from its average time per call: two HIP events on the launch stream bracket
the timed region (no events between its calls); the median and interquartile
range come from a second pass with an event pair around each call. `traffic`
is the HBM bytes per call that rocprofv3 measured for the same kernel
sources (profiles/, null once the sources change); `hbm` gives the
same call's algorithmic HBM bytes (every input read once, y and the final
state written once) against the HBM peak; `flushed` times the call with
512 MB written between calls (more than the 256 MB last-level cache).
`cpu_baseline` is the fp64 oracle timed on this host on every core of the
process's affinity set over the whole workload (plus one thread on a sample).
Measured in the same run, each with its own roofline: the scan on the
130M-shaped layer (`fwd_130m`) and on 131,072 tokens (`fwd_131k`), both with
flushed caches and alternated inputs; the backward call on the 2.8B layer
(`bwd`), the decode step (64 one-token updates of a 4,096 x 5,120 x 16 fp32
state, `decode`), the causal convolution front-end (`conv`) and the Mamba-2
SSD layer (80 heads of 64, N = 128, 8 x 2048, `ssd`, against the bf16
matrix-core peak), and the same forward scan through the opt-in state-split
kernel (`fwd_split`), for comparison with the default kernel. `--parts`
selects a subset (profiling runs use one part each).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
# fp32 vector peak: 256 CUs x 4 SIMDs x 2 wave64 instructions per 4 clocks
# (x 64 lanes = 32 lane-operations per clock) x 2 flops per FMA x 2.4 GHz =
# 157.3 TFLOP/s, the published figure. These kernels use unpacked fp32
# arithmetic only; on gfx950 a SIMD issues two unpacked fp32 add/multiply/FMA
# wave instructions per four clocks when two waves have one ready (measured
# up to 1.76 per four clocks with eight waves per SIMD), so the published peak
# is the roofline they are held to.
ALU_PEAK_TFLOPS = 256 * 4 * 32 * 2 * 2.4e9 / 1e12
# one wave instruction per SIMD per four clocks, the rate the scan kernels
# reach in practice (reported beside the roofline)
SINGLE_ISSUE_TFLOPS = ALU_PEAK_TFLOPS / 2
FLUSH_BYTES = 512 << 20    # written between flushed calls: more than the 256 MB MALL
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "scan": ["scan_fwd.hip", "tile_io.h", "device_math.h", "kernels.h"],
    "decode": ["state_update.hip", "device_math.h", "kernels.h"],
    "conv": ["conv1d.hip", "device_math.h", "conv.h"],
    "conv_update": ["conv1d.hip", "device_math.h", "conv.h"],
    "bwd": ["scan_bwd.hip", "scan_fwd.hip", "tile_io.h", "device_math.h", "kernels.h"],
    "ssd": ["ssd.hip", "device_math.h", "kernels.h"],
    "split": ["scan_split.hip", "scan_split.h", "tile_io.h", "device_math.h", "kernels.h"],
}
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak


def source_hash(kind: str) -> str:
    """sha256 over the kernel sources of one entry point (to tell whether HBM
    byte counts recorded under profiles/ still describe the built kernels)."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "selective_state_space_56_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def recorded_traffic(kind: str, workload: str):
    """HBM bytes per call measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
    (scaled by a plain copy's counts) and stored in profiles/, or None when
    there is no record or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, f"{kind}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != source_hash(kind):
        return None
    return rec.get("hbm_bytes_per_call")
METRIC = "scan fwd: (batch·L·D_inner) elem-steps/s + achieved HBM GB/s (% of peak)"


def scan_bytes(w) -> int:
    """Algorithmic HBM bytes of one scan: x, Delta_raw, z read and y written
    (io dtype, once per element), B and C read once per token, A, D and bias
    read once per channel, the fp32 final state written once."""
    eb = 2 if w.io == "bf16" else 4
    elems = w.batch * w.seqlen * w.dim
    io_tensors = 3 if w.gate else 2
    return (elems * eb * (io_tensors + 1) + 2 * w.batch * w.seqlen * w.dstate * eb
            + w.dim * w.dstate * 4 + 2 * w.dim * 4 + w.batch * w.dim * w.dstate * 4)


def scan_flops(w) -> int:
    """Algorithmic fp32 operations of one scan, counting each transcendental
    as one: per (step, state) Delta*A, exp, Delta*x*B (Delta*x once per
    step), two FMAs = 7; per (step, channel) bias add, softplus (exp, add,
    log), Delta*x, D*x + y (2), and with the gate silu (exp, add, divide,
    multiply) and the gate multiply (5)."""
    per_row_step = 7 * w.dstate + 7 + (5 if w.gate else 0)
    return w.batch * w.seqlen * w.dim * per_row_step


def bwd_bytes(w) -> int:
    """Algorithmic HBM bytes of one backward call: x, Delta_raw, z and dy read
    and dx, dDelta_raw, dz written (io dtype, once per element), B and C read
    and the fp32 dB and dC written once per token, A, D and bias read and dA,
    dD, dbias written once per channel, the fp32 final-state gradient read
    and the initial-state gradient written once per row."""
    eb = 2 if w.io == "bf16" else 4
    elems = w.batch * w.seqlen * w.dim
    io_in = 4 if w.gate else 3
    io_out = 3 if w.gate else 2
    tok = w.batch * w.seqlen * w.dstate
    rows = w.batch * w.dim * w.dstate
    return (elems * eb * (io_in + io_out) + tok * (2 * eb + 2 * 4) + 2 * (w.dim * w.dstate * 4 + 2 * w.dim * 4)
            + 2 * rows * 4)


def bwd_flops(w) -> int:
    """Algorithmic fp32 operations of one backward call (an FMA counts as 2,
    a transcendental as 1), the recomputation of the states included (the
    method recomputes rather than stores them). Per (step, state): decay
    Delta*A and exp (2), state Delta*x*B and FMA (3), adjoint C*ds + (2),
    abar*h_{t-1}*lam (2), dA, A-term of dDelta, lam*B, C*h read-out FMAs (8),
    dB and dC products and their sums over channels (4), abar*lam (1) = 22.
    Per (step, channel): softplus (3), sigmoid of the Delta input (3),
    silu(z) and its sigmoid (4), ds (1), dx (3), dDelta_raw (3), dz (5), the
    dD and dbias sums (3) = 25."""
    return w.batch * w.seqlen * w.dim * (22 * w.dstate + 25)


def ssd_flops(w) -> int:
    """Algorithmic matrix-core work of one SSD call (the chunked algorithm, FMA
    = 2 flops), per (batch row, head, chunk of Q steps): the causal half of the
    scores C B^T (Q^2 N), the masked scores times X (Q^2 P), the chunk state
    (2 Q N P) and the inherited state's read-out C S_in (2 Q N P)."""
    Q = 256
    chunks = -(-w.seqlen // Q)
    per = Q * Q * (w.dstate + w.headdim) + 4 * Q * w.dstate * w.headdim
    return w.batch * w.nheads * chunks * per


def ssd_bytes(w) -> int:
    """Algorithmic HBM bytes of one SSD call: x read and y written (bf16), dt
    (bf16, one per head and step), B and C (bf16, per group and step) read
    once, A, D and bias per head."""
    return (2 * w.batch * w.seqlen * w.nheads * w.headdim * 2 + w.batch * w.seqlen * w.nheads * 2
            + 2 * w.batch * w.seqlen * w.ngroups * w.dstate * 2 + 3 * w.nheads * 4)


def decode_bytes(w) -> int:
    """Per decode step: the fp32 state read and written, x, Delta_raw, z read,
    y written, B and C per sequence, A, D and bias per channel."""
    eb = 2 if w.io == "bf16" else 4
    rows = w.batch * w.dim
    return (2 * rows * w.dstate * 4 + rows * eb * 4 + 2 * w.batch * w.dstate * eb
            + w.dim * w.dstate * 4 + 2 * w.dim * 4)


def conv_bytes(w, width=4) -> int:
    """Algorithmic HBM bytes of one conv1d_fwd call: xin read and out written
    once (io dtype), the state in and out, taps and bias once per channel."""
    eb = 2 if w.io == "bf16" else 4
    elems = w.batch * w.seqlen * w.dim
    return 2 * elems * eb + 2 * w.batch * w.dim * (width - 1) * eb + w.dim * (width + 1) * 4


def conv_update_bytes(w, width=4) -> int:
    """Per decode token: the state read and written, xin read, out written,
    taps and bias."""
    eb = 2 if w.io == "bf16" else 4
    rows = w.batch * w.dim
    return 2 * rows * (width - 1) * eb + 2 * rows * eb + w.dim * (width + 1) * 4


def time_calls(fn, n, stream):
    """Run fn n times on `stream`, timing each call with HIP events recorded on
    that stream. Returns the list of per-call milliseconds."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    with torch.cuda.stream(stream):
        for a, b in evs:
            a.record(stream)
            fn()
            b.record(stream)
    stream.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, nthreads):
    """The fp64 oracle on the whole workload on this host's cores, and on one
    thread over every 16th channel (rows are independent, so the work scales
    exactly with the channel count)."""
    import numpy as np
    from oracle import default_oracle
    from selective_state_space_56_amd.workloads import to_f64_numpy
    orc = default_oracle()
    args = [to_f64_numpy(inp[k]) for k in ("x", "delta", "A", "B", "C")]
    kw = {k: to_f64_numpy(inp[k]) for k in ("D", "z", "delta_bias")}
    t0 = time.perf_counter()
    orc.scan(*args, **kw, nthreads=nthreads)
    dt = time.perf_counter() - t0
    ch = np.arange(0, w.dim, 16)
    sub = [np.ascontiguousarray(args[0][:, :, ch]), np.ascontiguousarray(args[1][:, :, ch]),
           np.ascontiguousarray(args[2][ch]), args[3], args[4]]
    skw = {"D": np.ascontiguousarray(kw["D"][ch]), "z": np.ascontiguousarray(kw["z"][:, :, ch]),
           "delta_bias": np.ascontiguousarray(kw["delta_bias"][ch])}
    t1 = time.perf_counter()
    orc.scan(*sub, **skw, nthreads=1)
    dt1 = time.perf_counter() - t1
    one = w.batch * w.seqlen * len(ch) / dt1
    return {"value": w.elem_steps / dt, "unit": "elem-steps/s", "cores": nthreads, "kind": "oracle",
            "sample": f"whole workload ({w.batch}x{w.seqlen}x{w.dim}, N={w.dstate}), fp64, "
                      f"{dt:.2f} s wall on {nthreads} threads; one thread on every 16th channel: "
                      f"{one:.3g} elem-steps/s ({dt1:.2f} s)",
            "single_thread_value": one, "cpu_model": cpu_model()}


def flushed_calls(fns, n, stream):
    """Per-call milliseconds of n calls, cycling through fns (one per resident
    input set), each call preceded by an untimed write of FLUSH_BYTES so that
    no input is served from the MALL or L2; HIP events on `stream` bracket the
    call alone."""
    import torch
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    with torch.cuda.stream(stream):
        for i, (a, b) in enumerate(evs):
            scratch.fill_(i & 0xff)
            a.record(stream)
            fns[i % len(fns)]()
            b.record(stream)
    stream.synchronize()
    del scratch
    return [a.elapsed_time(b) for a, b in evs]


def call_stats(ms):
    """median, min and interquartile range of per-call times (ms)."""
    import numpy as np
    q1, med, q3 = np.percentile(ms, [25, 50, 75])
    return {"median_launch_ms": float(med), "min_launch_ms": float(min(ms)),
            "iqr_launch_ms": [float(q1), float(q3)]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="mamba2p8b_prefill")
    ap.add_argument("--segments", type=int, default=0, help="force time segments (0 = library plan)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-conv", action="store_true")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-ssd", action="store_true")
    ap.add_argument("--parts", default="fwd,c1,c3,bwd,decode,conv,ssd,split",
                    help="comma list of the parts to run (profiling runs take one family at a time); "
                         "without fwd only the other parts' objects are printed")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (to scale HBM byte counters)")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "launches": 3}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows are independent, so batch/channel sharding would need no communication; "
              "see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from selective_state_space_56_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from selective_state_space_56_amd.build import build
        build()
    from selective_state_space_56_amd import scan_fwd
    from selective_state_space_56_amd.workloads import WORKLOADS, make_scan_inputs

    parts = set(args.parts.split(","))
    run_fwd = "fwd" in parts
    run_bwd = "bwd" in parts and not args.no_bwd
    run_decode = "decode" in parts and not args.no_decode
    run_conv = "conv" in parts and not args.no_conv
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    w = WORKLOADS[args.workload]
    inp = make_scan_inputs(w, device=dev)
    stream = torch.cuda.current_stream(dev)
    rec = {}
    if run_fwd:
        rec = fwd_part(args, w, inp, stream, scan_fwd, binding)
    # the other forward workloads (per-call, flushed): the 130M layer and the
    # 131k-token long context
    if "c1" in parts:
        rec["fwd_130m"] = scan_case_part(args, "mamba130m_layer", stream, 30)
    if "c3" in parts:
        rec["fwd_131k"] = scan_case_part(args, "long_context_131k", stream, 6)
    if run_bwd:
        rec["bwd"] = bwd_part(args, w, inp, stream, binding)
    if run_decode:
        rec["decode"] = decode_part(stream)
    if run_conv:
        rec["conv"] = conv_part(args, w, stream)
    if "ssd" in parts and not args.no_ssd:
        rec["ssd"] = ssd_part(args, stream)
    if "split" in parts:
        rec["fwd_split"] = split_part(args, w, inp, stream)
    if run_fwd and not args.no_cpu_baseline:
        nthreads = max(1, len(os.sched_getaffinity(0)))
        rec["cpu_baseline"] = cpu_baseline(w, inp, nthreads)
    print(json.dumps(rec), flush=True)


def fwd_part(args, w, inp, stream, scan_fwd, binding):
    """The headline: K back-to-back mamba_scan_fwd calls on the 2.8B prefill
    layer, alternating between two resident input sets (so consecutive calls
    cannot reuse each other's inputs from the MALL), timed on the wall clock
    (value, ms_per_step) and per call with HIP events (roofline); then the
    same call with the MALL and L2 flushed before each call."""
    import torch
    from selective_state_space_56_amd.workloads import make_scan_inputs
    dev = inp["x"].device
    inp2 = make_scan_inputs(w, device=dev, seed=1)
    out = torch.empty((w.batch, w.seqlen, w.dim), dtype=w.torch_io, device=dev)
    last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)

    def make_step(i):
        def step():
            scan_fwd(i["x"], i["delta"], i["A"], i["B"], i["C"], D=i["D"], z=i["z"],
                     delta_bias=i["delta_bias"], out=out, last_state=last, segments=args.segments)
        return step
    steps = [make_step(inp), make_step(inp2)]
    it = iter(range(10 ** 9))

    def step():
        steps[next(it) % 2]()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed region: K back-to-back calls, bracketed by two HIP events on
    # the calls' stream (their difference / K is the per-call GPU time the
    # roofline uses) and by the wall clock (value, ms_per_step)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    region_ms = ev0.elapsed_time(ev1) / args.steps
    # then the per-call distribution (median, IQR), an event pair around each call
    per_call = time_calls(step, args.steps, stream)
    flushed = flushed_calls(steps, max(20, min(args.steps, 50)), stream)
    del inp2

    value = w.elem_steps * args.steps / elapsed
    kern_ms = region_ms
    nbytes = scan_bytes(w)
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    nflops = scan_flops(w)
    tflops = nflops / (kern_ms * 1e-3) / 1e12
    ws_bytes = binding.workspace_size(w.batch, w.seqlen, w.dim, w.dstate, w.torch_io, args.segments)
    fl = call_stats(flushed)
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "elem-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.io == "bf16" else "f32",
        "data": "synthetic (seeded; shapes of a Mamba-2.8B layer; two input sets alternated)",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "d_inner": w.dim,
                   "d_state": w.dstate, "io": w.io, "state": "f32", "gate": w.gate,
                   "parallelism": "single GPU"},
        # The scan is bound by vector-instruction issue, so the roofline is the
        # ALU one; the HBM view (the metric's GB/s) rides along.
        "roofline": {"bound": "alu", "achieved": tflops, "peak": ALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / ALU_PEAK_TFLOPS,
                     "traffic": recorded_traffic("scan", w.name),
                     "kernel": "mamba_scan_fwd call (aggregate, fold and output kernels)",
                     "algorithmic_flops_per_launch": nflops, "avg_launch_ms": kern_ms,
                     "avg_launch_ms_method": "HIP events bracketing the timed region, / steps",
                     **call_stats(per_call),
                     "per_call_method": "second pass of the same calls, HIP events around each",
                     "workspace_bytes": ws_bytes,
                     "single_issue_peak": SINGLE_ISSUE_TFLOPS,
                     "frac_of_single_issue": tflops / SINGLE_ISSUE_TFLOPS},
        "hbm": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nbytes,
                "achieved_at_median": nbytes / (call_stats(per_call)["median_launch_ms"] * 1e-3) / 1e9},
        "flushed": {"method": f"{FLUSH_BYTES >> 20} MB written before each call (untimed), "
                              "two input sets alternated; HIP events around the call",
                    "calls": len(flushed), **fl,
                    "hbm_frac_at_median": nbytes / (fl["median_launch_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "alu_frac_at_median": nflops / (fl["median_launch_ms"] * 1e-3) / 1e12 / ALU_PEAK_TFLOPS},
    }
    return rec


def scan_case_part(args, name, stream, calls):
    """Another workload of the forward scan (the 130M layer, the 131k-token
    long context): per-call times with the MALL and L2 flushed before each
    call (two input sets alternated where both fit comfortably), with the
    elem-steps/s, HBM and ALU fractions at the median."""
    import torch
    from selective_state_space_56_amd import binding, scan_fwd
    from selective_state_space_56_amd.workloads import WORKLOADS, make_scan_inputs
    w = WORKLOADS[name]
    dev = torch.device("cuda", 0)
    sets = [make_scan_inputs(w, device=dev, seed=s) for s in range(2 if w.elem_steps < 1e9 else 1)]
    out = torch.empty((w.batch, w.seqlen, w.dim), dtype=w.torch_io, device=dev)
    last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)

    def make_step(i):
        return lambda: scan_fwd(i["x"], i["delta"], i["A"], i["B"], i["C"], D=i["D"], z=i["z"],
                                delta_bias=i["delta_bias"], out=out, last_state=last)
    fns = [make_step(i) for i in sets]
    for f in fns:
        f()
    torch.cuda.synchronize()
    ms = flushed_calls(fns, calls, stream)
    st = call_stats(ms)
    med = st["median_launch_ms"] * 1e-3
    nb, nf = scan_bytes(w), scan_flops(w)
    res = {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "d_inner": w.dim,
           "d_state": w.dstate, "io": w.io, "input_sets": len(sets), "calls": calls,
           "flush_bytes": FLUSH_BYTES, **st, "avg_launch_ms": sum(ms) / len(ms),
           "value_at_median": w.elem_steps / med, "unit": "elem-steps/s",
           "hbm": {"achieved": nb / med / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": nb / med / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": nb},
           "alu": {"achieved": nf / med / 1e12, "peak": ALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                   "frac": nf / med / 1e12 / ALU_PEAK_TFLOPS, "algorithmic_flops_per_launch": nf},
           "workspace_bytes": binding.workspace_size(w.batch, w.seqlen, w.dim, w.dstate, w.torch_io)}
    del sets, out, last
    return res


def bwd_part(args, w, inp, stream, binding):
    import torch
    from selective_state_space_56_amd import scan_bwd
    from selective_state_space_56_amd.workloads import make_bwd_grads
    dev = inp["x"].device
    gr = make_bwd_grads(w, device=dev)

    def bstep():
        scan_bwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], gr["dout"], D=inp["D"],
                 z=inp["z"], delta_bias=inp["delta_bias"], dlast=gr["dlast"])

    for _ in range(3):
        bstep()
    torch.cuda.synchronize()
    nb = max(5, args.steps // 5)
    bcalls = time_calls(bstep, nb, stream)
    bms = sum(bcalls) / len(bcalls)
    bfl = bwd_flops(w)
    bby = bwd_bytes(w)
    out = {
        "op": "mamba_scan_bwd (all gradients, states recomputed)", "workload": w.name,
        "calls": nb, "avg_launch_ms": bms, **call_stats(bcalls),
        "value": w.elem_steps / (bms * 1e-3), "unit": "elem-steps/s",
        "roofline": {"bound": "alu", "achieved": bfl / (bms * 1e-3) / 1e12,
                     "peak": ALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": bfl / (bms * 1e-3) / 1e12 / ALU_PEAK_TFLOPS,
                     "traffic": recorded_traffic("bwd", w.name),
                     "algorithmic_flops_per_launch": bfl},
        "hbm": {"achieved": bby / (bms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": bby / (bms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "algorithmic_bytes_per_launch": bby},
        "workspace_bytes": binding.bwd_workspace_size(w.batch, w.seqlen, w.dim, w.dstate,
                                                      w.torch_io),
    }
    del gr
    return out


def decode_part(stream):
    import torch
    from selective_state_space_56_amd import state_update
    from selective_state_space_56_amd.workloads import (WORKLOADS, make_decode_state,
                                                        make_decode_token, make_params)
    dev = torch.device("cuda", 0)
    wd = WORKLOADS["decode_4096"]
    params = make_params(wd, device=dev)
    state = make_decode_state(wd, device=dev)
    toks = [make_decode_token(wd, s, device=dev) for s in range(wd.decode_steps)]
    outd = torch.empty((wd.batch, wd.dim), dtype=wd.torch_io, device=dev)
    it = iter(range(10 ** 9))

    def dstep():
        t = toks[next(it) % wd.decode_steps]
        state_update(state, t["x"], t["delta"], params["A"], t["B"], t["C"], D=params["D"],
                     z=t["z"], delta_bias=params["delta_bias"], out=outd)

    for _ in range(4):
        dstep()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dcalls = time_calls(dstep, wd.decode_steps, stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t1
    dms = sum(dcalls) / len(dcalls)
    db = decode_bytes(wd)
    out = {
        "workload": wd.name, "steps": wd.decode_steps, "ms_total": dt * 1e3,
        "value": wd.batch * wd.dim * wd.decode_steps / dt, "unit": "elem-steps/s",
        "avg_launch_ms": dms, **call_stats(dcalls),
        "roofline": {"bound": "hbm", "achieved": db / (dms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": db / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": recorded_traffic("decode", wd.name),
                     "algorithmic_bytes_per_launch": db},
    }
    del toks, state
    return out


def conv_part(args, w, stream):
    import torch
    from selective_state_space_56_amd import conv1d_fwd, conv1d_update
    from selective_state_space_56_amd.workloads import WORKLOADS, make_conv_inputs
    dev = torch.device("cuda", 0)
    ci = make_conv_inputs(w, 4, device=dev)
    cout = torch.empty_like(ci["xin"])
    cst = torch.empty_like(ci["state"])

    def cstep():
        conv1d_fwd(ci["xin"], ci["weight"], ci["bias"], ci["state"], out=cout, state_out=cst)

    for _ in range(args.warmup):
        cstep()
    torch.cuda.synchronize()
    ccalls = time_calls(cstep, args.steps, stream)
    cms = sum(ccalls) / len(ccalls)
    cb = conv_bytes(w)
    out = {
        "op": "mamba_conv1d_fwd (causal depthwise conv, width 4, + SiLU)", "workload": w.name,
        "avg_launch_ms": cms, **call_stats(ccalls),
        "value": w.elem_steps / (cms * 1e-3), "unit": "elem-steps/s",
        "roofline": {"bound": "hbm", "achieved": cb / (cms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": cb / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": recorded_traffic("conv", w.name),
                     "algorithmic_bytes_per_launch": cb},
    }
    wd = WORKLOADS["decode_4096"]
    cd = make_conv_inputs(wd.with_shape(seqlen=1), 4, device=dev)
    cstate = cd["state"].clone()
    cx = cd["xin"][:, 0].contiguous()
    cdo = torch.empty_like(cx)
    for _ in range(4):
        conv1d_update(cstate, cx, cd["weight"], cd["bias"], out=cdo)
    torch.cuda.synchronize()
    ucalls = time_calls(lambda: conv1d_update(cstate, cx, cd["weight"], cd["bias"], out=cdo),
                        wd.decode_steps, stream)
    ums = sum(ucalls) / len(ucalls)
    ub = conv_update_bytes(wd)
    out["decode"] = {
        "op": "mamba_conv1d_update", "workload": wd.name, "avg_launch_ms": ums,
        **call_stats(ucalls),
        "roofline": {"bound": "hbm", "achieved": ub / (ums * 1e-3) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": ub / (ums * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "traffic": recorded_traffic("conv_update", wd.name),
                     "algorithmic_bytes_per_launch": ub},
    }
    del ci, cout, cst, cd, cstate
    return out


def ssd_part(args, stream):
    import torch
    from selective_state_space_56_amd import ssd_fwd
    from selective_state_space_56_amd.workloads import SSD_WORKLOADS, make_ssd_inputs
    dev = torch.device("cuda", 0)
    ws = SSD_WORKLOADS["mamba2_2p7b_layer"]
    si = make_ssd_inputs(ws, device=dev)
    out = torch.empty_like(si["x"])
    last = torch.empty((ws.batch, ws.nheads, ws.dstate, ws.headdim), dtype=torch.float32, device=dev)

    def sstep():
        ssd_fwd(si["x"], si["dt"], si["A"], si["B"], si["C"], D=si["D"], dt_bias=si["dt_bias"],
                out=out, last_state=last)

    for _ in range(args.warmup):
        sstep()
    torch.cuda.synchronize()
    calls = time_calls(sstep, args.steps, stream)
    ms = sum(calls) / len(calls)
    fl, by = ssd_flops(ws), ssd_bytes(ws)
    res = {
        "op": "mamba_ssd_fwd (Mamba-2 SSD, chunked on the matrix cores)", "workload": ws.name,
        "config": {"batch": ws.batch, "seq_len": ws.seqlen, "heads": ws.nheads,
                   "head_dim": ws.headdim, "d_state": ws.dstate, "groups": ws.ngroups, "chunk": 256,
                   "io": "bf16"},
        "avg_launch_ms": ms, **call_stats(calls),
        "value": ws.elem_steps / (ms * 1e-3), "unit": "elem-steps/s",
        "roofline": {"bound": "mfma", "achieved": fl / (ms * 1e-3) / 1e12,
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": fl / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": recorded_traffic("ssd", ws.name),
                     "algorithmic_flops_per_launch": fl},
        "hbm": {"achieved": by / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": by},
    }
    del si, out, last
    return res


def split_part(args, w, inp, stream):
    """The same forward scan through the opt-in state-split kernel
    (MAMBA_SCAN_SPLIT_STATES): timed beside the default for comparison."""
    import torch
    from selective_state_space_56_amd import scan_fwd
    dev = inp["x"].device
    out = torch.empty((w.batch, w.seqlen, w.dim), dtype=w.torch_io, device=dev)
    last = torch.empty((w.batch, w.dim, w.dstate), dtype=torch.float32, device=dev)

    def step():
        scan_fwd(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], D=inp["D"], z=inp["z"],
                 delta_bias=inp["delta_bias"], out=out, last_state=last, split_states=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    calls = time_calls(step, args.steps, stream)
    ms = sum(calls) / len(calls)
    fl, by = scan_flops(w), scan_bytes(w)
    return {
        "op": "mamba_scan_fwd with MAMBA_SCAN_SPLIT_STATES (one scan_split_kernel launch; not the default)",
        "workload": w.name, "avg_launch_ms": ms, **call_stats(calls),
        "value": w.elem_steps / (ms * 1e-3), "unit": "elem-steps/s",
        "roofline": {"bound": "alu", "achieved": fl / (ms * 1e-3) / 1e12, "peak": ALU_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": fl / (ms * 1e-3) / 1e12 / ALU_PEAK_TFLOPS,
                     "traffic": recorded_traffic("split", w.name), "algorithmic_flops_per_launch": fl},
        "hbm": {"achieved": by / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes_per_launch": by},
    }


if __name__ == "__main__":
    main()

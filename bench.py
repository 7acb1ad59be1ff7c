#!/usr/bin/env python3
"""Benchmark: KDA chunked prefill tokens/s on one MI355X (plus decode tok/s).

One step = one kda_chunk_fwd call over the prefill workload (B=4, H=16,
T=2048, d_k=d_v=128, bf16 q/k/v, fp32 gates, chunk 64), inputs resident in
HBM.  Steps rotate over NSETS independently seeded input sets (about 0.8 GB
in total, well above the 256 MB Infinity Cache) so each call reads its inputs
from HBM rather than from a cache warmed by the previous call.

Printed: ONE JSON line with the headline prefill rate, the roofline of the
prefill call (compulsory HBM bytes / measured call time against 8 TB/s), the
decode workload (256 sequences x 32 heads, 512 MiB fp32 state, 1024 steps),
the long-context workload (B=1 H=32 T=65536) and the packed-batch workload
(64 sequences, H=16), each with its own roofline, and the fp64 CPU oracle
timed on this host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
METRIC = "KDA chunked prefill tokens/s at H=16,d=128; decode tok/s; % of roofline"
NSETS = 4

# HBM traffic per call from two rocprofv3 passes (TCC FETCH_SIZE, then
# WRITE_SIZE), calibrated against a plain device copy of known size: FETCH_SIZE
# reads half the bytes moved (x2.0), WRITE_SIZE reads them exactly (x1.0).
# Each figure belongs to the kernel source with the given sha256 prefix and is
# reported as null once that source has changed.
MEASURED_TRAFFIC = {
    "prefill": ("kda_prefill.hip", "3277a6bfc4657d66", 467_075_141),
    "decode": ("kda_decode.hip", "00e70acbccc2d272", 1_086_896_743),
    "decode_tokens": ("kda_decode.hip", "00e70acbccc2d272", 1_125_807_616),
    # measured under the two-phase schedule: counter collection serialises
    # kernels, which the overlapped schedule cannot run under
    "long_context": ("kda_prefill.hip", "3277a6bfc4657d66", 7_466_443_120),
    "long_share": ("kda_prefill.hip", "3277a6bfc4657d66", 1_202_456_800),
    "varlen": ("kda_prefill.hip", "3277a6bfc4657d66", 16_085_273_910),
}


def measured_traffic(key):
    import hashlib
    fname, sha, nbytes = MEASURED_TRAFFIC[key]
    if nbytes is None:
        return None
    path = os.path.join(ROOT, "linear_attention_kda_amd", "csrc", fname)
    with open(path, "rb") as f:
        cur = hashlib.sha256(f.read()).hexdigest()
    return nbytes if cur.startswith(sha) else None


def prefill_bytes(B, T, H, dk, dv, esize=2, s0=False, gate_form="channel"):
    """Compulsory HBM bytes of one prefill call: q, k, v, o at their dtype,
    alpha fp32 (per key channel, or one per token and head, or none), beta
    fp32, S_final (and S0) fp32."""
    tok = B * T * H
    alpha = {"channel": tok * dk * 4, "scalar": tok * 4, "none": 0,
             "log_channel": tok * dk * 4, "log_scalar": tok * 4,
             "softplus_channel": tok * dk * 4, "softplus_scalar": tok * 4}[gate_form]
    return (tok * (2 * dk + 2 * dv) * esize + alpha + tok * 4
            + (2 if s0 else 1) * B * H * dv * dk * 4)


def prefill_flops(B, T, H, dk, dv, C=64):
    """Algorithmic flops of the chunked form per head-token, as executed:
    6 dk dv + 2C(3dk + 2dv) + C^2/3."""
    return B * T * H * (6 * dk * dv + 2 * C * (3 * dk + 2 * dv) + C * C / 3)


def packed_bytes(T, N, H, dk, dv, esize=2):
    """Compulsory bytes of one packed-batch call of T tokens in N sequences:
    per head-token q, k, v, o at their dtype, alpha fp32 per key channel and
    beta fp32; S0 and S_final fp32 once per (sequence, head)."""
    return T * H * ((2 * dk + 2 * dv) * esize + dk * 4 + 4) + 2 * N * H * dv * dk * 4


def decode_bytes(N, H, dk, dv, esize=2):
    units = N * H
    return units * (2 * dv * dk * 4 + (2 * dk + 2 * dv) * esize + dk * 4 + 4)


def bench_prefill(args, torch, kda, inputs, gate_form="channel", steps=None, act=0, module=False):
    w = inputs.WORKLOADS["prefill"]
    B, T, H, dk, dv = w["B"], w["T"], w["H"], w["dk"], w["dv"]
    steps = steps or args.steps
    dev = torch.device("cuda:0")
    sets = []
    # one workspace, as a caller running layer after layer would hold
    ws = torch.empty(kda.chunk_fwd_workspace_size(B, T, H, dk, dv, -1, kda.KDA_BF16),
                     dtype=torch.uint8, device=dev)
    for s in range(NSETS):
        if gate_form == "channel":
            inp = inputs.workload("prefill", seed=s, device=dev)
        else:
            inp = inputs.dense(B, T, H, dk, dv, w["dtype"], w["gate"], seed=s, device=dev,
                               gate_form=gate_form)
        o = torch.empty_like(inp["v"])
        S = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
        ops = {}
        if module:
            # random module weights (no trained ones): convolution taps, norm
            # gains, and gate logits shaped like the output
            g = torch.Generator(device=dev).manual_seed(100 + s)
            ops = dict(conv=tuple(torch.randn((H, d, 4), generator=g, device=dev) * 0.5 for d in (dk, dk, dv)),
                       norm_weight=1.0 + 0.1 * torch.randn(dv, generator=g, device=dev), norm_eps=1e-6,
                       out_gate=torch.randn(inp["v"].shape, generator=g, device=dev).to(w["dtype"]))
        sets.append((inp, ws, o, S, ops))
    torch.cuda.synchronize()

    def step(i):
        inp, ws, o, S, ops = sets[i % NSETS]
        kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], gate=gate_form, out=o,
                      S_final=S, workspace=ws, act=act, **ops)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # one pair of HIP events on the library's stream around all timed calls:
    # events between the calls would add their own gaps to every step
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_ms = e0.elapsed_time(e1) / steps
    # the spread of single calls, from a separate short run with events
    # around each call (not used for the throughput)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        step(i)
        b.record(stream)
    torch.cuda.synchronize()
    single = sorted(a.elapsed_time(b) for a, b in ev)
    return dict(B=B, T=T, H=H, dk=dk, dv=dv, wall_s=wall, ms_per_step=wall * 1e3 / steps,
                call_ms_mean=mean_ms, call_ms_median=single[len(single) // 2], call_ms_min=single[0],
                tokens=B * T)


def bench_long_context(args, torch, kda, inputs, steps=10, warmup=2, name="long",
                       others=("two_phase",), first="auto"):
    """A long-context workload (S0 given): one chunk chain of 1024 steps per
    (sequence, head).  `long` (B=1, H=32, T=65536) under the automatic
    schedule (which overlaps prep and scan for this shape) and under
    two-phase; `long_share` (its 4-head share) under the automatic schedule
    (split-sequence) and the others for comparison."""
    w = inputs.WORKLOADS[name]
    B, T, H, dk, dv = w["B"], w["T"], w["H"], w["dk"], w["dv"]
    dev = torch.device("cuda:0")
    inp = inputs.workload(name, seed=0, device=dev)
    o = torch.empty_like(inp["v"])
    S = torch.empty((B, H, dv, dk), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.chunk_fwd_workspace_size(B, T, H, dk, dv, -1, kda.KDA_BF16), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    out, status = {}, {}
    for sched in (first,) + tuple(others):
        prev = kda.set_schedule(sched)
        for _ in range(warmup):
            kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"], out=o,
                          S_final=S, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"], out=o,
                          S_final=S, workspace=ws)
        e1.record(stream)
        torch.cuda.synchronize()
        kda.set_schedule(prev)
        out[sched] = e0.elapsed_time(e1) * 1e3 / steps
        # which schedule the timed calls ran, and that none reported an error
        status[sched] = kda.chunk_fwd_status(ws)
        if status[sched][1]:
            raise RuntimeError(f"long-context {sched}: schedule error bits {status[sched][1]:#x}")
    nbytes = prefill_bytes(B, T, H, dk, dv, s0=True)
    ach = nbytes / (out[first] * 1e-6) / 1e9
    res = {"workload": f"long-context prefill B={B} H={H} T={T} d_k=d_v={dk} bf16, S0 given",
           "calls": steps, "call_us_mean": round(out[first], 1),
           "schedule": status[first][0]}
    for sched in others:
        res[f"call_us_{sched}"] = round(out[sched], 1)
    res.update({"tokens_per_s": round(B * T / (out[first] * 1e-6), 1),
                "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(ach / HBM_PEAK_GBS, 4),
                             "traffic": measured_traffic("long_context" if name == "long" else name),
                             "traffic_schedule": "two_phase" if name == "long" else "split",
                             "algorithmic_bytes": nbytes}})
    return res


def bench_varlen(args, torch, kda, inputs, steps=20, warmup=3):
    """The packed-batch workload: 64 sequences of lognormal lengths in one
    buffer with int32 offsets, 16 heads, per-sequence S0, the slow-gate and
    beta = 1 head groups."""
    w = inputs.WORKLOADS["varlen"]
    H, dk, dv = w["H"], w["dk"], w["dv"]
    dev = torch.device("cuda:0")
    inp = inputs.workload("varlen", seed=0, device=dev)
    T = int(inp["cu_seqlens"][-1])
    N = int(inp["lengths"].numel())
    o = torch.empty_like(inp["v"])
    S = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.chunk_fwd_workspace_size(1, T, H, dk, dv, N, kda.KDA_BF16), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)

    def call():
        kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0=inp["S0"],
                      cu_seqlens=inp["cu_seqlens"], out=o, S_final=S, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / steps
    lens = inp["lengths"]
    nbytes = packed_bytes(T, N, H, dk, dv)
    ach = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"packed batch of {N} sequences (lengths {int(lens.min())}..{int(lens.max())}, "
                        f"total {T} tokens) H={H} d_k=d_v={dk} bf16, S0 given",
            "calls": steps, "call_us_mean": round(us, 1), "tokens": T,
            "chunks": int(((lens + 63) // 64).sum()) * H,
            "tokens_per_s": round(T / (us * 1e-6), 1),
            "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": measured_traffic("varlen"),
                         "algorithmic_bytes": nbytes}}


def decode_tokens_bytes(N, H, dk, dv, Tk, esize=2):
    """One multi-token launch: the state is read and written once, each of the
    Tk tokens brings its q, k, v, alpha, beta and writes its output row."""
    units = N * H
    return units * (2 * dv * dk * 4 + Tk * ((2 * dk + 2 * dv) * esize + dk * 4 + 4))


def bench_decode_tokens(args, torch, kda, inputs, Tk=4):
    """Draft verification: Tk tokens per sequence per launch over the decode
    workload's state, the same 1024 tokens per sequence as the decode line."""
    w = inputs.WORKLOADS["decode"]
    N, H, dk, dv = w["N"], w["H"], w["dk"], w["dv"]
    launches = max(1, args.decode_steps // Tk)
    dev = torch.device("cuda:0")
    S = inputs.decode_state(N, H, dk, dv, w["s0_std"], seed=0, device=dev)
    blocks = []                      # 32 distinct input blocks (1.3 GiB), cycled
    for b in range(min(32, launches)):
        toks = [inputs.decode_token(N, H, dk, dv, w["dtype"], w["alpha_lo"], step=b * Tk + t, device=dev)
                for t in range(Tk)]
        blocks.append({key: torch.stack([t[key] for t in toks], 1).contiguous() for key in toks[0]})
    o = torch.empty((N, Tk, H, dv), dtype=w["dtype"], device=dev)
    S_w = S.clone()
    for b in range(min(4, launches)):
        t = blocks[b % len(blocks)]
        kda.decode_tokens(t["q"], t["k"], t["v"], t["alpha"], t["beta"], S_w, S_out=S_w, out=o)
    del S_w
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for b in range(launches):
        t = blocks[b % len(blocks)]
        kda.decode_tokens(t["q"], t["k"], t["v"], t["alpha"], t["beta"], S, S_out=S, out=o)
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    launch_us = total_ms * 1e3 / launches
    nbytes = decode_tokens_bytes(N, H, dk, dv, Tk)
    achieved = nbytes / (launch_us * 1e-6) / 1e9
    return {"workload": f"decode_tokens N={N} H={H} d_k=d_v={dk} bf16, Tk={Tk} tokens per launch, "
                        f"fp32 state {N * H * dv * dk * 4 >> 20} MiB updated in place",
            "launches": launches, "tokens_per_s": N * Tk * launches / (total_ms * 1e-3),
            "us_per_launch": launch_us,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode_tokens"), "bytes_per_launch": nbytes}}


def bench_decode(args, torch, kda, inputs):
    w = inputs.WORKLOADS["decode"]
    N, H, dk, dv, steps = w["N"], w["H"], w["dk"], w["dv"], args.decode_steps
    dev = torch.device("cuda:0")
    S = inputs.decode_state(N, H, dk, dv, w["s0_std"], seed=0, device=dev)
    toks = [inputs.decode_token(N, H, dk, dv, w["dtype"], w["alpha_lo"], step=s, device=dev)
            for s in range(steps)]
    o = torch.empty((N, H, dv), dtype=w["dtype"], device=dev)
    # warm-up on a copy of the state (the timed run starts from the seeded state)
    S_w = S.clone()
    for s in range(min(8, steps)):
        t = toks[s]
        kda.decode_step(t["q"], t["k"], t["v"], t["alpha"], t["beta"], S_w, out=o)
    del S_w
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(steps):
        t = toks[s]
        kda.decode_step(t["q"], t["k"], t["v"], t["alpha"], t["beta"], S, out=o)
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    step_us = total_ms * 1e3 / steps
    nbytes = decode_bytes(N, H, dk, dv)
    achieved = nbytes / (step_us * 1e-6) / 1e9
    return {"workload": f"decode N={N} H={H} d_k=d_v={dk} bf16, fp32 state {N * H * dv * dk * 4 >> 20} MiB",
            "steps": steps, "tokens_per_s": N * steps / (total_ms * 1e-3), "us_per_step": step_us,
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                         "traffic": measured_traffic("decode"), "bytes_per_step": nbytes}}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inputs, torch):
    """The fp64 oracle on the prefill workload, timed on this host's cores:
    all 64 (sequence, head) units x 2048 tokens with OpenMP over units, and one
    unit-slice (4 units) on a single thread."""
    import oracle
    inp = inputs.workload("prefill", seed=0, device="cpu")
    args = [oracle._to_f64(inp[n]) for n in ("q", "k", "v", "alpha", "beta")]
    threads = oracle.default_threads()
    orc = oracle.get()
    w = inputs.WORKLOADS["prefill"]
    tokens = w["B"] * w["T"]
    reps, t_all = 3, []
    for _ in range(reps):
        t0 = time.perf_counter()
        orc.fwd(*args, n_threads=threads)
        t_all.append(time.perf_counter() - t0)
    dt = min(t_all)
    # single thread on sequence 0, heads 0..3 (4 of 64 units), scaled per unit
    one = [a[:1, :, :4].copy() for a in args]
    t0 = time.perf_counter()
    orc.fwd(*one, n_threads=1)
    dt1 = (time.perf_counter() - t0) * (w["B"] * w["H"] / 4)
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"whole prefill workload (B=4 x T=2048 tokens, 16 heads, d=128) in fp64, "
                      f"best of {reps}: {dt:.3f} s on {threads} threads ({os.cpu_count()} visible "
                      f"CPUs, {_cpu_model()}); one thread on 4 of the 64 units, scaled: "
                      f"{tokens / dt1:.1f} tokens/s",
            "single_thread_value": round(tokens / dt1, 1)}


def copy_calib(args, torch):
    """One plain device copy of --copy-calib-mib MiB, whose counter readings
    calibrate FETCH_SIZE and WRITE_SIZE."""
    n = args.copy_calib_mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    return n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-gate-forms", action="store_true",
                    help="skip the scalar-gate prefill line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the long-context workload (B=1 H=32 T=65536, timed under both schedules)")
    ap.add_argument("--long-only", action="store_true",
                    help="time only the long-context workload (for profiling); prints its object")
    ap.add_argument("--long-share-only", action="store_true",
                    help="time only the 4-head long-context share (split-sequence; for profiling)")
    ap.add_argument("--schedule", default="auto", choices=["auto", "two_phase", "overlap", "split"],
                    help="with --long-only / --long-share-only: the one schedule to time (counter "
                         "collection serialises kernels, which the overlapped schedule cannot run under)")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed-batch workload (64 sequences, H=16)")
    ap.add_argument("--varlen-only", action="store_true",
                    help="time only the packed-batch workload (for profiling); prints its object")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus "
              f"{args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_kda_amd as kda
    from linear_attention_kda_amd import inputs

    if args.long_only:
        out = {"long_context": bench_long_context(args, torch, kda, inputs, others=(), first=args.schedule)}
        if args.copy_calib_mib:
            out["copy_calib_bytes"] = copy_calib(args, torch)
        print(json.dumps(out), flush=True)
        return
    if args.long_share_only:
        out = {"long_context_share": bench_long_context(args, torch, kda, inputs, name="long_share", others=(),
                                                        first=args.schedule)}
        if args.copy_calib_mib:
            out["copy_calib_bytes"] = copy_calib(args, torch)
        print(json.dumps(out), flush=True)
        return
    if args.varlen_only:
        out = {"varlen": bench_varlen(args, torch, kda, inputs)}
        if args.copy_calib_mib:
            out["copy_calib_bytes"] = copy_calib(args, torch)
        print(json.dumps(out), flush=True)
        return
    pf = bench_prefill(args, torch, kda, inputs)
    nbytes = prefill_bytes(pf["B"], pf["T"], pf["H"], pf["dk"], pf["dv"])
    flops = prefill_flops(pf["B"], pf["T"], pf["H"], pf["dk"], pf["dv"])
    call_s = pf["call_ms_mean"] * 1e-3
    achieved = nbytes / call_s / 1e9
    result = {
        "metric": METRIC,
        "value": round(pf["tokens"] / (pf["ms_per_step"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pf["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill B=4 H=16 T=2048 d_k=d_v=128, bf16 q/k/v, fp32 gates, "
                               "chunk 64, S0=0", "B": pf["B"], "T": pf["T"], "H": pf["H"],
                   "d_k": pf["dk"], "d_v": pf["dv"], "chunk": 64, "input_sets": NSETS},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("prefill"),
                     "kernel": "kda_chunk_fwd call (chunk_prep_kernel + chunk_scan_kernel)",
                     "algorithmic_bytes": nbytes,
                     "call_us_mean": round(pf["call_ms_mean"] * 1e3, 2),
                     "single_call_us_median": round(pf["call_ms_median"] * 1e3, 2),
                     "single_call_us_min": round(pf["call_ms_min"] * 1e3, 2),
                     "mfma_frac": round(flops / call_s / 1e12 / BF16_PEAK_TFLOPS, 4)},
    }
    if not args.no_decode:
        result["decode"] = bench_decode(args, torch, kda, inputs)
        result["decode_tokens"] = bench_decode_tokens(args, torch, kda, inputs)
    if not args.no_gate_forms:
        # the same workload with the gate in other forms: one gate per (token,
        # head) (Gated DeltaNet), and per-channel gates given as log(alpha)
        forms = (("scalar", "prefill_scalar_gate", "one fp32 gate per (token, head)", 0),
                 ("log_channel", "prefill_log_gate", "per-channel fp32 gates given as log(alpha)", 0),
                 ("softplus_channel", "prefill_fused_inputs",
                  "raw q, k (SiLU and unit length applied on load), beta logits (sigmoid on load), "
                  "per-channel gate logits g with alpha = exp(-softplus(g))",
                  kda.KDA_ACT_QK_SILU_L2NORM | kda.KDA_ACT_BETA_SIGMOID),
                 ("softplus_channel", "prefill_module_ops",
                  "the fused inputs above after a short causal convolution of q, k and v (width 4, random taps), "
                  "outputs through an RMS norm and a sigmoid gate (gate logits bf16, shaped like o)",
                  kda.KDA_ACT_QK_SILU_L2NORM | kda.KDA_ACT_BETA_SIGMOID))
        for form, key, what, act in forms:
            module = key == "prefill_module_ops"
            sg = bench_prefill(args, torch, kda, inputs, gate_form=form, steps=max(20, args.steps // 4), act=act,
                               module=module)
            sb = prefill_bytes(sg["B"], sg["T"], sg["H"], sg["dk"], sg["dv"], gate_form=form)
            if module:  # the gate logits are read once; the weights are a few KB
                sb += sg["B"] * sg["T"] * sg["H"] * sg["dv"] * 2
            ach = sb / (sg["call_ms_mean"] * 1e-3) / 1e9
            result[key] = {
                "workload": f"prefill B=4 H=16 T=2048 d=128 bf16, {what}",
                "tokens_per_s": round(sg["tokens"] / (sg["ms_per_step"] * 1e-3), 1),
                "call_us_mean": round(sg["call_ms_mean"] * 1e3, 2),
                "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(ach / HBM_PEAK_GBS, 4), "algorithmic_bytes": sb}}
    if not args.no_long_context:
        result["long_context"] = bench_long_context(args, torch, kda, inputs)
        result["long_context_share"] = bench_long_context(args, torch, kda, inputs, name="long_share",
                                                          others=("two_phase", "overlap"))
    if not args.no_varlen:
        result["varlen"] = bench_varlen(args, torch, kda, inputs)
    if args.copy_calib_mib:
        result["copy_calib_bytes"] = copy_calib(args, torch)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inputs, torch)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

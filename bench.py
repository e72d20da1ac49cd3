"""Benchmark of the delta-rule operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one chunkwise Gated DeltaNet prefill of the workload
B=4, H=8, T=2048, d_k=d_v=128, bf16 (seeded synthetic inputs resident in HBM),
i.e. dn_chunk_fwd = the chunk-parallel UT/WY phase followed by the sequential
inter-chunk scan. The JSON line reports whole-job token-heads/s (B*H*T per
second) as `value` (K steps back to back between two synchronisations), the
median step and the median cold step (MALL and L2s flushed before each call),
the roofline of the dominant kernel (timed live with HIP events on the stream
it runs on), the fp64 CPU oracle timed on this host as `cpu_baseline`, and the
parity of the timed outputs against it. `long_context` holds the same record
for the largest single-GPU workload, B=1, H=16, T=65536 (the one-launch form).
`decode` holds the fused decode step of B=256 x H=16, d=128 (1000 steps, fp32
state updated in place) in state-HBM GB/s against the HBM peak. The other
workloads (KDA prefill, the fp32 DeltaNet recurrent and chunked forms) are timed
under `workloads`, the serving forms and variants under `serving_forms`, and
the gated layer's kernels around the rule under `layer`.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill tokens/s (B*H*T/s) at d=128 + decode state HBM GB/s, % of peak"
PEAK_BF16_TFLOPS = 2516.6     # dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0         # HBM3E
C = 64

# Algorithmic work per token and head at d_k = d_v = d (full 64 x 64 tiles, as
# the chunk algorithm is written): the chunk-parallel phase does K K^T, Q K^T,
# W = T X and u = T V (4 x 2*C*d); the scan does W S, Q~ S, K~^T U (3 x 2*d*d)
# and attn U (2*C*d).
def flops_prep(d):
    return 4 * 2 * C * d


def flops_scan(d):
    return 3 * 2 * d * d + 2 * C * d


def bytes_prefill(B, H, T, d, esize=2):
    """Compulsory HBM bytes: q, k, v, beta, g read, o written, S_final written."""
    return B * H * T * (4 * d * esize + 2 * esize) + B * H * d * d * 4


def decode_bytes_per_step(B, H, d, esize=2):
    """State read + write, q, k, v, beta, g read, o written."""
    return B * H * (2 * d * d * 4 + 3 * d * esize + 2 * esize + d * esize)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# HBM traffic per launch from rocprofv3 counter runs (FETCH_SIZE and WRITE_SIZE in
# KiB per dispatch, each in a run of its own, averaged over the dispatches of the
# kernel at the workload's grid size) on the workloads timed here:
#   rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -- python3 bench.py --no-cpu
#       --no-workloads --steps 5 --warmup 2 --cold-reps 2 --decode-steps 20
# A plain device copy of 512 MiB (bench.py --copy-mib 512) reads FETCH_SIZE =
# 262,159 KiB and WRITE_SIZE = 524,288 KiB, so FETCH_SIZE is scaled by 2.0 and
# WRITE_SIZE by 1.0. Each entry carries the SHA-256 of the kernel sources it was
# taken on; when they have changed since, the figure no longer describes the
# kernel and is reported as null.
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0
CHUNK_SOURCES = ("delta_rule_recurrent_amd/csrc/chunk.hip", "delta_rule_recurrent_amd/csrc/dn_chunk.h",
                 "delta_rule_recurrent_amd/csrc/dn_device.h", "delta_rule_recurrent_amd/csrc/dn_launch.h",
                 "delta_rule_recurrent_amd/csrc/dn_kda_prep.h", "delta_rule_recurrent_amd/build.py")
DECODE_SOURCES = ("delta_rule_recurrent_amd/csrc/decode.hip", "delta_rule_recurrent_amd/csrc/dn_device.h",
                  "delta_rule_recurrent_amd/csrc/dn_launch.h")
TRAFFIC = {
    # B=4 H=8 T=2048 d=128 (grid 1024 x 128 threads; 3750 / 3990 dispatches)
    "chunk_prep2_kernel": {"fetch_kib": 29217.2, "write_kib": 58112.0, "sources": CHUNK_SOURCES,
                           "sha256": "87099bb4c798a6b8ed7d39510f1a473bd23d8cd85533d5a2f712a9f0248da651"},
    # B=4 H=8 T=2048 d=128 (grid 256 x 256 threads; 3750 / 3990 dispatches)
    "chunk_scan_kernel": {"fetch_kib": 37107.0, "write_kib": 18432.0, "sources": CHUNK_SOURCES,
                          "sha256": "87099bb4c798a6b8ed7d39510f1a473bd23d8cd85533d5a2f712a9f0248da651"},
    # B=1 H=16 T=65536 d=128 (grid 240 x 256 threads; 810 / 830 dispatches)
    "chunk_fused_kernel": {"fetch_kib": 987842.3, "write_kib": 1193988.6, "sources": CHUNK_SOURCES,
                           "sha256": "87099bb4c798a6b8ed7d39510f1a473bd23d8cd85533d5a2f712a9f0248da651"},
    # KDA B=2 H=16 T=8192 d=128 (grid 512 x 256 threads; 54 / 54 dispatches), from
    #   rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) -- python3 bench.py --no-cpu
    #       --no-prefill --no-long --no-decode
    "chunk_fused_kda_kernel": {"fetch_kib": 283280.2, "write_kib": 366915.4, "sources": CHUNK_SOURCES,
                               "sha256": "87099bb4c798a6b8ed7d39510f1a473bd23d8cd85533d5a2f712a9f0248da651"},
    # B=256 H=16 d=128, one token (311 dispatches each)
    "decode_step_kernel": {"fetch_kib": 136307.8, "write_kib": 263168.0, "sources": DECODE_SOURCES,
                           "sha256": "f4ef3522c6770c548689c443524ee18ffe39ad6d04accfc58b54f4519dfe8c8a"},
}


def sources_sha256(sources):
    import hashlib

    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_bytes(kernel):
    """Measured HBM bytes per launch (read + write, calibrated), or None when the
    kernel sources changed after the counters were taken."""
    t = TRAFFIC.get(kernel)
    if t is None or t["sha256"] != sources_sha256(t["sources"]):
        return None
    return int(round((t["fetch_kib"] * FETCH_SCALE + t["write_kib"] * WRITE_SCALE) * 1024))


def event_time_ms(torch, fn, reps):
    """Average duration of one fn() (one kernel launch): `reps` launches back to
    back on the current stream between one pair of HIP events, after one
    untimed launch. Matches the per-dispatch average of a kernel trace."""
    fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def call_times_ms(torch, fn, reps, flush=None):
    """Durations in ms of `reps` calls of fn, each between its own pair of HIP
    events on the current stream (the stream every entry point here launches
    on). Warm (flush None): the calls run back to back. Cold: before each call,
    outside its events, `flush` (a copy through two 512 MiB buffers, twice the
    256 MB MALL) evicts what the earlier calls left in the MALL and the L2s."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for e0, e1 in evs:
        if flush is not None:
            flush()
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def launch_means_ms(torch, fn, groups, per_group):
    """Mean duration of one fn() (one kernel launch) in each of `groups` groups of
    `per_group` launches back to back between one pair of HIP events on the
    current stream, after one untimed launch. Back to back, the launches run
    one after the other with no gap, so a group's mean matches the per-dispatch
    average of a kernel trace (events around single launches would add each
    launch's start-up latency)."""
    fn()
    out = []
    for _ in range(groups):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(per_group):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / per_group)
    return out


def median(xs):
    s = sorted(xs)
    n = len(s)
    return s[n // 2] if n % 2 else 0.5 * (s[n // 2 - 1] + s[n // 2])


def make_flush(torch, dev):
    a = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    a.fill_(1)
    return lambda: b.copy_(a)


def settle(torch, step, seconds):
    """Untimed calls, after the warmup steps, until `seconds` of wall time have
    passed: the timed region then starts with the GPU's clocks already up (a
    few warmup steps of tens of microseconds leave it at its idle clocks).
    Returns the number of calls."""
    t0, n = time.perf_counter(), 0
    while True:
        for _ in range(20):
            step()
        torch.cuda.synchronize()
        n += 20
        if time.perf_counter() - t0 >= seconds:
            return n


def timed_steps(torch, step, steps):
    """The contract's timing: `steps` calls back to back between a barrier and a
    device synchronisation on both sides, one HIP event before each call and one
    after the last. Returns (mean ms per call over the whole bracket, median of
    the per-call event intervals, wall seconds)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(steps):
        evs[i].record()
        step()
    evs[steps].record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[steps]) / steps, median(per), t_wall


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100,
                    help="timed steps of the headline prefill (the long-context one takes a fifth)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the CPU oracle on the workload until this much time has passed")
    ap.add_argument("--no-workloads", action="store_true", help="skip the secondary workloads")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode workload")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the headline prefill (for profiling the other kernels alone)")
    ap.add_argument("--no-long", action="store_true",
                    help="skip the long-context prefill (B=1, H=16, T=65536)")
    ap.add_argument("--settle", type=float, default=1.0,
                    help="seconds of untimed calls after the warmup steps of each prefill workload")
    ap.add_argument("--cold-reps", type=int, default=10,
                    help="calls timed after a flush of the MALL and L2s (0: none)")
    ap.add_argument("--serving-only", action="store_true",
                    help="only time the serving forms and variants (for profiling their kernels)")
    ap.add_argument("--layer-only", action="store_true",
                    help="only time the gated layer's prologue / epilogue kernels (for profiling them)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (three times) and exit: "
                         "the reference kernel for scaling memory-traffic counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: the operator shards over (sequence, head) with "
              "no communication, and no multi-GPU path is implemented (got --gpus %d)"
              % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import delta_rule_recurrent_amd as dn
    import synthetic

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    def to_dev(d):
        return {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}

    if args.copy_mib:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "copies": 3}), flush=True)
        return

    if args.serving_only:
        print(json.dumps({"serving_forms": run_serving(torch, dn, synthetic, to_dev, dev)}), flush=True)
        return

    if args.layer_only:
        print(json.dumps({"layer": run_layer(torch, dn, synthetic, to_dev, dev)}), flush=True)
        return

    flush = make_flush(torch, dev) if args.cold_reps else None

    # ------------------------------------------------------------------ prefill
    result = {}
    if not args.no_prefill:
        result = run_prefill(args, torch, np, dn, synthetic, to_dev, dev,
                             "gdn_prefill_b4_h8_t2048_d128", flush)
    if not args.no_long:
        # the largest single-GPU workload, with its own roofline and CPU baseline
        result["long_context"] = run_prefill(args, torch, np, dn, synthetic, to_dev, dev,
                                             "gdn_prefill_b1_h16_t65536_d128", flush)
    del flush

    # ------------------------------------------------------------------- decode
    if not args.no_decode:
        result["decode"] = run_decode(args, torch, dn, synthetic, to_dev)

    # ---------------------------------------------------------- other workloads
    if not args.no_workloads:
        result["workloads"] = run_workloads(torch, dn, synthetic, to_dev, dev)
        result["serving_forms"] = run_serving(torch, dn, synthetic, to_dev, dev)
        result["layer"] = run_layer(torch, dn, synthetic, to_dev, dev)

    print(json.dumps(result), flush=True)


def cpu_oracle(args, np, inp_cpu, o, S_final, label):
    """The fp64 oracle on the whole workload, repeated until args.cpu_seconds of
    wall time have passed, and the parity of the timed GPU outputs against it."""
    import oracle

    nthreads = len(os.sched_getaffinity(0))
    log("cpu oracle on %d threads (%s)" % (nthreads, label))
    reps, t = 0, 0.0
    while reps == 0 or t < args.cpu_seconds:
        t0 = time.perf_counter()
        o_ref, S_ref = oracle.recurrent(inp_cpu["q"], inp_cpu["k"], inp_cpu["v"],
                                        inp_cpu["beta"], inp_cpu["g"], None, nthreads=nthreads)
        t += time.perf_counter() - t0
        reps += 1
    tokens = int(np.prod(inp_cpu["q"].shape[:3]))
    base = {
        "value": round(tokens * reps / t, 1), "unit": "tokens/s",
        "cores": oracle.max_threads(nthreads), "kind": "oracle",
        "sample": "the whole workload (%s; fp64 token-by-token recurrence) run %d times back "
                  "to back, %.2f s in total" % (label, reps, t),
    }
    og = o.float().cpu().double().numpy()
    sg = S_final.cpu().double().numpy()
    parity = {
        "o": float(np.abs(og - o_ref).max() / np.abs(o_ref).max()),
        "S_final": float(np.abs(sg - S_ref).max() / np.abs(S_ref).max()),
        "bound": 2e-2, "metric": "max|gpu-ref|/max|ref|",
    }
    log("cpu oracle %.2f s, parity %s" % (t, parity))
    return base, parity


def kernel_entry(ms_list, flop, per_group):
    """ms: mean launch duration over all groups; median_ms: median of the groups' means."""
    ms = sum(ms_list) / len(ms_list)
    tf = flop / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 5), "median_ms": round(median(ms_list), 5), "flop": flop,
            "launches": len(ms_list) * per_group,
            "timing": "%d groups of %d launches back to back" % (len(ms_list), per_group),
            "tflops": round(tf, 2), "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4)}


def roofline_block(name, e):
    return {
        "kernel": name, "bound": "mfma",
        "achieved": e["tflops"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": e["frac_mfma"],
        "traffic": traffic_bytes(name),
        "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x2.0 + WRITE_SIZE x1.0)",
        "algorithmic_flop_per_launch": e["flop"],
        "avg_launch_ms": e["ms"],
    }


def run_prefill(args, torch, np, dn, synthetic, to_dev, dev, name, flush):
    """One chunked Gated DeltaNet prefill workload: the contract's K-step timing,
    warm and cold medians, the dominant kernel's roofline from live event timing,
    and the CPU oracle beside it with the parity of the timed outputs.

    At 32 chunks per sequence dn_chunk_fwd runs the two phases (chunk_prep2 then
    chunk_scan), each timed alone back to back on the same stream; from 64
    chunks on it runs the one-launch form, whose call is chunk_fused_kernel plus
    two recomputation launches that return at once when the hand-off succeeded
    (about 2 us together), so the call's duration stands for the kernel's."""
    cfg = synthetic.CONFIGS[name]
    B, H, T, d = cfg["B"], cfg["H"], cfg["T"], cfg["dk"]
    nchunks = (T + C - 1) // C
    log("generating", name)
    inp_cpu = synthetic.make_config(name)
    inp = to_dev(inp_cpu)
    ws = torch.empty(dn.workspace_bytes(B, H, T, d, d, torch.bfloat16), dtype=torch.uint8, device=dev)
    o = torch.empty(B, H, T, d, dtype=torch.bfloat16, device=dev)
    S_final = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)

    def step():
        dn.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], None, o=o,
                     S_final=S_final, workspace=ws)

    steps = args.steps if nchunks < 64 else max(5, args.steps // 5)
    for _ in range(args.warmup):
        step()
    nsettle = settle(torch, step, args.settle)
    ms_step, med_step, t_wall = timed_steps(torch, step, steps)
    cold = call_times_ms(torch, step, args.cold_reps, flush=flush)
    tokens = B * H * T
    value = tokens / (ms_step * 1e-3)
    log("%s %.4f ms/step (median %.4f, cold median %.4f)  %.3e token-heads/s (wall %.3f s, %d steps)"
        % (name, ms_step, med_step, median(cold), value, t_wall, steps))

    groups, per = (5, 20) if nchunks < 64 else (5, 4)
    if nchunks < 64:
        kern = {
            "chunk_prep2_kernel": kernel_entry(launch_means_ms(torch, lambda: dn.chunk_prep(
                inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], ws), groups, per),
                flops_prep(d) * tokens, per),
            "chunk_scan_kernel": kernel_entry(launch_means_ms(torch, lambda: dn.chunk_scan(
                inp["q"], o, ws, None, S_final), groups, per), flops_scan(d) * tokens, per),
        }
    else:
        kern = {
            "chunk_fused_kernel": kernel_entry(launch_means_ms(torch, lambda: dn.chunk_fwd_fused(
                inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], None, o=o, S_final=S_final,
                workspace=ws), groups, per), (flops_prep(d) + flops_scan(d)) * tokens, per),
        }
        # DN_OK unless a hand-off wait of the latest call gave up (its results
        # were then recomputed by the two phases, and the time includes that)
        kern["chunk_fused_kernel"]["handoff_status"] = dn.chunk_fwd_handoff_status(
            ws, B, H, T, d, d, torch.bfloat16)
    for k_, v_ in kern.items():
        log("  %s %.4f ms (median %.4f)  %.1f TFLOP/s (%.2f%% of bf16 MFMA peak)"
            % (k_, v_["ms"], v_["median_ms"], v_["tflops"], 100 * v_["frac_mfma"]))
    dom = max(kern, key=lambda k_: kern[k_]["ms"])
    total_flop = (flops_prep(d) + flops_scan(d)) * tokens
    nbytes = bytes_prefill(B, H, T, d)
    path = lambda ms: {"ms": round(ms, 5),
                       "tflops": round(total_flop / (ms * 1e-3) / 1e12, 2),
                       "frac_mfma": round(total_flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "gbs_algorithmic": round(nbytes / (ms * 1e-3) / 1e9, 1),
                       "frac_hbm": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "settle": {"seconds": args.settle, "calls": nsettle,
                   "what": "untimed calls after the warmup steps, before the timed region"},
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "B": B, "H": H, "T": T, "d_k": d, "d_v": d, "chunk": C,
                   "variant": "gated_deltanet", "S0": "zeros",
                   "form": "two-phase" if nchunks < 64 else "one-launch"},
        "timing": {
            "mean_ms": round(ms_step, 5), "median_ms": round(med_step, 5),
            "cold_median_ms": round(median(cold), 5), "cold_reps": len(cold),
            "cold": "a copy of 512 MiB between two buffers (1 GiB of HBM traffic, four times the "
                    "256 MB MALL) before each cold call, outside its events",
            "warm_path": path(med_step), "cold_path": path(median(cold)),
            "algorithmic_flop": total_flop, "algorithmic_bytes": nbytes,
        },
        "roofline": roofline_block(dom, kern[dom]),
        "kernels": kern,
    }
    if not args.no_cpu:
        label = "B=%d, H=%d, T=%d, d=%d" % (B, H, T, d)
        result["cpu_baseline"], result["parity"] = cpu_oracle(args, np, inp_cpu, o, S_final, label)
    del inp, ws, o, S_final, inp_cpu
    return result


def run_decode(args, torch, dn, synthetic, to_dev):
    name_d = "gdn_decode_b256_h16_d128"
    cd = synthetic.CONFIGS[name_d]
    Bd, Hd, dd = cd["B"], cd["H"], cd["dk"]
    nsteps = args.decode_steps
    log("generating", name_d, nsteps, "steps")
    dinp = to_dev(synthetic.make_config(name_d, steps=nsteps))
    S = dinp["S0"].clone()
    od = torch.empty(Bd, Hd, dd, dtype=torch.bfloat16, device=S.device)
    xs = [(dinp["q"][s], dinp["k"][s], dinp["v"][s], dinp["beta"][s], dinp["g"][s])
          for s in range(nsteps)]

    def dstep(s):
        q_, k_, v_, b_, g_ = xs[s]
        dn.decode_step(q_, k_, v_, b_, g_, S, o=od)

    for s in range(min(10, nsteps)):
        dstep(s)
    torch.cuda.synchronize()
    runs = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for s in range(nsteps):
            dstep(s)
        e1.record()
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1))
    loop_ms = median(runs)
    per_launch = event_time_ms(torch, lambda: dstep(0), 200)
    bps = decode_bytes_per_step(Bd, Hd, dd)
    gbs_loop = bps * nsteps / (loop_ms * 1e-3) / 1e9
    gbs_kernel = bps / (per_launch * 1e-3) / 1e9
    log("decode %.2f us/step  %.1f GB/s loop, %.1f GB/s per launch"
        % (loop_ms * 1000 / nsteps, gbs_loop, gbs_kernel))
    return {
        "workload": name_d, "B": Bd, "H": Hd, "d": dd, "steps": nsteps,
        "runs_ms": [round(r, 4) for r in runs], "run": "median of 5 runs of the steps back to back",
        "ms_per_1000_steps": round(loop_ms * 1000.0 / nsteps, 3),
        "us_per_step": round(loop_ms * 1000.0 / nsteps, 2),
        "token_heads_per_s": round(Bd * Hd * nsteps / (loop_ms * 1e-3), 1),
        "state_gbs": round(gbs_loop, 1), "frac_hbm": round(gbs_loop / PEAK_HBM_GBS, 4),
        "bytes_per_step": bps,
        "roofline": {"kernel": "decode_step_kernel", "bound": "hbm",
                     "achieved": round(gbs_kernel, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs_kernel / PEAK_HBM_GBS, 4),
                     "traffic": traffic_bytes("decode_step_kernel"),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x2.0 + "
                                     "WRITE_SIZE x1.0)",
                     "algorithmic_bytes_per_launch": bps,
                     "avg_launch_ms": round(per_launch, 5)},
    }


def run_workloads(torch, dn, synthetic, to_dev, dev):
    wl = {}
    for wname, form in (("kda_prefill_b2_h16_t8192_d128", "chunk"),
                        ("deltanet_fp32_t512_d64", "chunk"),
                        ("deltanet_fp32_t512_d64", "recurrent")):
        c = synthetic.CONFIGS[wname]
        log("generating", wname)
        x = to_dev(synthetic.make_config(wname))
        Bw, Hw, Tw, dw = c["B"], c["H"], c["T"], c["dk"]
        dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
        kda = c["kind"] == "kda"
        wsw = torch.empty(max(dn.workspace_bytes(Bw, Hw, Tw, dw, dw, dt), 1), dtype=torch.uint8,
                          device=dev)
        ow = torch.empty(Bw, Hw, Tw, dw, dtype=dt, device=dev)
        Sw = torch.empty(Bw, Hw, dw, dw, dtype=torch.float32, device=dev)
        if form == "chunk":
            f = dn.kda_chunk_fwd if kda else dn.chunk_fwd
            run = lambda: f(x["q"], x["k"], x["v"], x["beta"], x["g"], None, o=ow, S_final=Sw,
                            workspace=wsw)
        else:
            run = lambda: dn.recurrent_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], None)
        for _ in range(3):
            run()
        # median of groups of launches back to back (50 calls in all)
        ms = median(launch_means_ms(torch, run, 5, 10))
        tok = Bw * Hw * Tw
        entry = {"form": form, "ms": round(ms, 4), "tokens_per_s": round(tok / (ms * 1e-3), 1)}
        if form == "chunk":
            tf = (flops_prep(dw) + flops_scan(dw)) * tok / (ms * 1e-3) / 1e12
            entry["tflops"] = round(tf, 2)
            entry["frac_mfma"] = round(tf / (PEAK_BF16_TFLOPS if dt == torch.bfloat16 else 157.3), 4)
            nb = bytes_prefill(Bw, Hw, Tw, dw, 2 if dt == torch.bfloat16 else 4)
            if kda:
                nb += Bw * Hw * Tw * (dw - 1) * (2 if dt == torch.bfloat16 else 4)   # g per key channel
            entry["gbs_algorithmic"] = round(nb / (ms * 1e-3) / 1e9, 1)
            entry["frac_hbm"] = round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
            if kda and dt == torch.bfloat16:
                # the one-launch form (the call's two guarded recomputation
                # launches return at once); counter traffic against the
                # compulsory bytes
                tb = traffic_bytes("chunk_fused_kda_kernel")
                entry["kernel"] = "chunk_fused_kda_kernel"
                entry["traffic"] = tb
                entry["traffic_vs_compulsory"] = round(tb / nb, 2) if tb else None
        wl["%s/%s" % (wname, form)] = entry
        log("  %s %s %.4f ms" % (wname, form, ms))
        del x, wsw, ow, Sw
    return wl


def run_serving(torch, dn, synthetic, to_dev, dev):
    """The serving forms of the prefill at the headline's size (32 value heads'
    worth of 2048 tokens at d = 128, bf16 Gated DeltaNet), each against the
    plain call it generalises:
      * chunk_fwd_states: every chunk-boundary state written (32 x 32 x 64 KiB);
      * chunk_fwd_gqa: 4 key heads shared by 8 value heads per sequence;
      * chunk_fwd_varlen: 8 heads over 8 sequences of 8192 tokens in all, with
        lengths 63 .. 3008 (the same 65536 token-heads as the headline);
    and decode_tokens (4 drafted tokens per sequence with a state snapshot after
    each) at the decode workload's 256 x 16 states; and the selective
    state-space kind (ssm_chunk_fwd at the headline size, ssm_decode_step at
    256 x 16 states) and the generalized delta rule's decode step (256 x 16)."""
    out = {}
    c = synthetic.CONFIGS["gdn_prefill_b4_h8_t2048_d128"]
    B, H, T, d = c["B"], c["H"], c["T"], c["dk"]
    x = to_dev(synthetic.make_config("gdn_prefill_b4_h8_t2048_d128"))
    tok = B * H * T

    def timed(name, run, extra=None):
        for _ in range(3):
            run()
        ms = event_time_ms(torch, run, 20)
        e = {"ms": round(ms, 4), "tokens_per_s": round(tok / (ms * 1e-3), 1)}
        e.update(extra or {})
        out[name] = e
        log("  serving %s %.4f ms" % (name, ms))

    ws = torch.empty(dn.workspace_bytes(B, H, T, d, d, torch.bfloat16), dtype=torch.uint8, device=dev)
    o = torch.empty(B, H, T, d, dtype=torch.bfloat16, device=dev)
    S = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)
    timed("chunk_fwd", lambda: dn.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["g"], None,
                                            o=o, S_final=S, workspace=ws))
    Sc = torch.empty(B, H, (T + 63) // 64, d, d, dtype=torch.float32, device=dev)
    timed("chunk_fwd_states", lambda: dn.chunk_fwd_states(x["q"], x["k"], x["v"], x["beta"], x["g"],
                                                          None, o=o, S_final=S, S_chunks=Sc,
                                                          workspace=ws),
          {"boundary_state_bytes": Sc.numel() * 4})
    qk = synthetic.make("gated", B, H // 2, T, d, d, dtype="bf16", seed=2001)
    qg, kg = qk["q"].to(dev), qk["k"].to(dev)
    timed("chunk_fwd_gqa", lambda: dn.chunk_fwd_gqa(qg, kg, x["v"], x["beta"], x["g"], None,
                                                    o=o, S_final=S, workspace=ws),
          {"key_heads": H // 2, "value_heads": H})
    lens = [3008, 64, 1536, 520, 1024, 77, 1900, 63]
    Tp = sum(lens)
    cu = torch.tensor([0] + [sum(lens[:i + 1]) for i in range(len(lens))], dtype=torch.int32,
                      device=dev)
    xp = to_dev(synthetic.make("gated", 1, H, Tp, d, d, dtype="bf16", seed=2002))
    wsp = torch.empty(int(dn.lib().dn_chunk_fwd_varlen_workspace(len(lens), H, Tp, d, d, 1)),
                      dtype=torch.uint8, device=dev)
    op = torch.empty(1, H, Tp, d, dtype=torch.bfloat16, device=dev)
    Sp = torch.empty(len(lens), H, d, d, dtype=torch.float32, device=dev)
    timed("chunk_fwd_varlen", lambda: dn.chunk_fwd_varlen(xp["q"], xp["k"], xp["v"], xp["beta"],
                                                          xp["g"], cu, None, o=op, S_final=Sp,
                                                          workspace=wsp),
          {"sequence_lengths": lens, "heads": H})
    # the selective state-space kind (no beta, no correction) on the same inputs
    timed("ssm_chunk_fwd", lambda: dn.ssm_chunk_fwd(x["q"], x["k"], x["v"], x["g"], None, o=o,
                                                    S_final=S, workspace=ws))
    # the generalized delta rule at the same size, chunked (fp32 maps) and token by token
    xg = to_dev(synthetic.make_gdr(B, H, T, d, "bf16", seed=2005))
    gargs = [xg[n] for n in ("q", "kw", "v", "kr", "a", "g")]
    wsg = torch.empty(int(dn.lib().dn_gdr_chunk_workspace(B, H, T, d, d, 1, 64)), dtype=torch.uint8,
                      device=dev)
    timed("gdr_chunk_fwd", lambda: dn.gdr_chunk_fwd(*gargs, None, o=o, S_final=S, workspace=wsg),
          {"workspace_bytes": wsg.numel()})
    timed("gdr_recurrent_fwd", lambda: dn.gdr_recurrent_fwd(*gargs, None))
    del xg, gargs, wsg
    # chunk-length sweep of the chunked generalized rule at T = 4096 (16 heads,
    # d = 128): the per-chunk triangular work grows with the length, the number
    # of sequential chunk steps falls with it
    Bs_, Hs_, Ts_ = 1, 16, 4096
    xs = to_dev(synthetic.make_gdr(Bs_, Hs_, Ts_, d, "bf16", seed=2006))
    sargs = [xs[n] for n in ("q", "kw", "v", "kr", "a", "g")]
    os_ = torch.empty(Bs_, Hs_, Ts_, d, dtype=torch.bfloat16, device=dev)
    Ss_ = torch.empty(Bs_, Hs_, d, d, dtype=torch.float32, device=dev)
    sweep = {}
    for ch in (16, 32, 64):
        wss = torch.empty(int(dn.lib().dn_gdr_chunk_workspace(Bs_, Hs_, Ts_, d, d, 1, ch)),
                          dtype=torch.uint8, device=dev)
        run = lambda: dn.gdr_chunk_fwd(*sargs, None, chunk=ch, o=os_, S_final=Ss_, workspace=wss)
        for _ in range(2):
            run()
        sweep[str(ch)] = round(event_time_ms(torch, run, 5), 4)
        del wss
    out["gdr_chunk_length_sweep_ms"] = {"B": Bs_, "H": Hs_, "T": Ts_, "d": d, "ms_by_chunk": sweep}
    log("  serving gdr chunk sweep %s" % sweep)
    del xs, sargs, os_, Ss_
    # the same sweep on the Gated DeltaNet prefill itself (two launches, chunk
    # lengths 32, 64, 128) at the same size
    xg2 = to_dev(synthetic.make("gated", Bs_, Hs_, Ts_, d, d, dtype="bf16", seed=2007))
    og2 = torch.empty(Bs_, Hs_, Ts_, d, dtype=torch.bfloat16, device=dev)
    Sg2 = torch.empty(Bs_, Hs_, d, d, dtype=torch.float32, device=dev)
    gsweep = {}
    for ch in (32, 64, 128):
        wsl = torch.empty(int(dn.lib().dn_chunk_fwd_len_workspace(Bs_, Hs_, Ts_, d, d, 1, ch)), dtype=torch.uint8,
                          device=dev)
        run = lambda: dn.chunk_fwd_len(xg2["q"], xg2["k"], xg2["v"], xg2["beta"], xg2["g"], None, chunk=ch,
                                       o=og2, S_final=Sg2, workspace=wsl)
        for _ in range(3):
            run()
        gsweep[str(ch)] = round(event_time_ms(torch, run, 20), 4)
        del wsl
    out["gdn_chunk_length_sweep_ms"] = {"B": Bs_, "H": Hs_, "T": Ts_, "d": d, "ms_by_chunk": gsweep,
                                        "form": "two launches (prep, scan)"}
    log("  serving gdn chunk sweep %s" % gsweep)
    del xg2, og2, Sg2
    del x, ws, o, S, Sc, qg, kg, xp, wsp, op, Sp
    # speculative decode: 4 drafted tokens for the decode workload's 256 x 16
    # states, the state after each kept (4 x 256 MiB of snapshots)
    Bd, Hd, K = 256, 16, 4
    xd = to_dev(synthetic.make("gated", Bd, Hd, K, d, d, dtype="bf16", seed=2003, s0_std=0.02))
    Sd = xd["S0"].clone()
    od = torch.empty(Bd, Hd, K, d, dtype=torch.bfloat16, device=dev)
    snap = torch.empty(Bd, Hd, K, d, d, dtype=torch.float32, device=dev)
    run = lambda: dn.decode_tokens(xd["q"], xd["k"], xd["v"], xd["beta"], xd["g"], Sd, o=od,
                                   S_snap=snap)
    for _ in range(2):
        run()
    ms = event_time_ms(torch, run, 5)
    state = Bd * Hd * d * d * 4
    moved = state * (2 + K)
    out["decode_tokens"] = {"ms": round(ms, 4), "B": Bd, "H": Hd, "tokens_per_call": K,
                            "state_bytes_moved": moved,
                            "gbs": round(moved / (ms * 1e-3) / 1e9, 1)}
    log("  serving decode_tokens %.4f ms" % ms)
    od1 = torch.empty(Bd, Hd, d, dtype=torch.bfloat16, device=dev)
    q1, k1, v1, g1 = (xd[n][:, :, 0].contiguous() for n in ("q", "k", "v", "g"))
    run = lambda: dn.ssm_decode_step(q1, k1, v1, g1, Sd, o=od1)
    for _ in range(2):
        run()
    ms = event_time_ms(torch, run, 20)
    out["ssm_decode_step"] = {"ms": round(ms, 4), "B": Bd, "H": Hd, "state_bytes_moved": 2 * state,
                              "gbs": round(2 * state / (ms * 1e-3) / 1e9, 1)}
    log("  serving ssm_decode_step %.4f ms" % ms)
    # generalized delta rule, one token for the same 256 x 16 states
    xg = to_dev(synthetic.make_gdr(Bd, Hd, 1, d, "bf16", seed=2004))
    gin = [xg[n][:, :, 0].contiguous() for n in ("q", "kw", "v", "kr", "a", "g")]
    run = lambda: dn.gdr_decode_step(*gin, Sd, o=od1)
    for _ in range(2):
        run()
    ms = event_time_ms(torch, run, 20)
    out["gdr_decode_step"] = {"ms": round(ms, 4), "B": Bd, "H": Hd, "state_bytes_moved": 2 * state,
                              "gbs": round(2 * state / (ms * 1e-3) / 1e9, 1)}
    log("  serving gdr_decode_step %.4f ms" % ms)
    del xd, Sd, od, snap, od1, xg, gin
    return out


def run_layer(torch, dn, synthetic, to_dev, dev):
    """The gated layer's kernels around the rule, at the headline's size (B=4,
    T=2048, 8 key and 8 value heads of d = 128, bf16) and at the decode
    workload's 256 sequences x 16 heads for one token:
      * prologue: convolution + SiLU with carried state, head split, L2 norm,
        gates, and the new convolution state;
      * epilogue: gated RMSNorm into token-major rows;
      * layer: prologue -> rule (chunked prefill / decode step) -> epilogue,
        i.e. the whole layer between its input and output projections.
    Bytes are the algorithmic HBM bytes of each kernel (every input read once,
    every output written once)."""
    out = {}

    def timed(name, run, nbytes, tokens, reps=20):
        for _ in range(3):
            run()
        ms = event_time_ms(torch, run, reps)
        e = {"ms": round(ms, 4), "tokens_per_s": round(tokens / (ms * 1e-3), 1)}
        if nbytes:
            e["bytes"] = nbytes
            e["gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
            e["frac_of_8000_gbs"] = round(nbytes / (ms * 1e-3) / 8e12, 3)
        out[name] = e
        log("  layer %s %.4f ms" % (name, ms))

    for tag, (B, T, Hk, Hv) in (("prefill_b4_t2048_h8", (4, 2048, 8, 8)),
                                ("decode_b256_h16", (256, 1, 16, 16))):
        d = 128
        x = to_dev(synthetic.make_layer(B, T, Hk, Hv, d, "bf16", seed=3001))
        C = (2 * Hk + Hv) * d
        tok = B * T * Hv
        q = torch.empty(B, Hk, T, d, dtype=torch.bfloat16, device=dev)
        k = torch.empty_like(q)
        v = torch.empty(B, Hv, T, d, dtype=torch.bfloat16, device=dev)
        beta = torch.empty(B, Hv, T, dtype=torch.bfloat16, device=dev)
        g = torch.empty_like(beta)
        cst = x["conv_state"].clone()
        act = B * T * C * 2 + 2 * B * T * Hv * 2   # qkv + (b, a), and as many written
        pro_bytes = 2 * act + 2 * B * C * 3 * 2 + C * 4 * 2
        # checked once through the binding, then timed as bare C-ABI calls with
        # the same arguments: at decode size the binding's per-call checks take
        # longer than the kernels
        dn.layer_prologue(x["qkv"], x["conv_w"], x["b"], x["a"], x["A_log"], x["dt_bias"], Hk, Hv,
                          conv_state=x["conv_state"], conv_state_out=cst, out=(q, k, v, beta, g))
        P = lambda t: t.data_ptr()   # noqa: E731
        st = torch.cuda.current_stream().cuda_stream
        pro_args = (P(x["qkv"]), P(x["conv_w"]), P(x["conv_state"]), P(cst), P(x["b"]), P(x["a"]),
                    P(x["A_log"]), P(x["dt_bias"]), P(q), P(k), P(v), P(beta), P(g), 0, B, T, Hk, Hv,
                    d, d, 1, st)
        lib = dn.lib()
        prologue = lambda: lib.dn_layer_prologue(*pro_args)   # noqa: E731
        timed(tag + "_prologue", prologue, pro_bytes, tok)
        o = torch.empty(B, Hv, T, d, dtype=torch.bfloat16, device=dev)
        y = torch.empty(B, T, Hv * d, dtype=torch.bfloat16, device=dev)
        dn.layer_epilogue(o, x["z"], x["norm_w"], 1e-6, out=y)
        epi_args = (P(o), P(x["z"]), P(x["norm_w"]), P(y), B, Hv, T, d, 1e-6, 1, st)
        epilogue = lambda: lib.dn_layer_epilogue(*epi_args)   # noqa: E731
        o.normal_()
        timed(tag + "_epilogue", epilogue, 3 * B * T * Hv * d * 2 + d * 2, tok)
        S = torch.zeros(B, Hv, d, d, dtype=torch.float32, device=dev)
        # the rule is likewise checked once through the binding and then timed as
        # a bare C-ABI call, so that the layer's figure is the GPU's time and not
        # the host's (three binding calls per layer at decode size outlast it)
        if T == 1:
            dn.decode_step_gqa(q[:, :, 0], k[:, :, 0], v[:, :, 0], beta[:, :, 0], g[:, :, 0], S,
                               o=o[:, :, 0])
            rule_args = (0, P(q), P(k), P(v), P(beta), P(g), P(S), P(o), B, Hk, Hv, d, d, 1, st)
            rule = lambda: lib.dn_decode_step_gqa(*rule_args)   # noqa: E731
        else:
            ws = torch.empty(dn.workspace_bytes(B, Hv, T, d, d, torch.bfloat16), dtype=torch.uint8,
                             device=dev)
            dn.chunk_fwd_gqa(q, k, v, beta, g, None, o=o, S_final=S, workspace=ws)
            rule_args = (0, P(q), P(k), P(v), P(beta), P(g), None, P(o), P(S), B, Hk, Hv, T, d, d, 1,
                         P(ws), ws.numel(), st)
            rule = lambda: lib.dn_chunk_fwd_gqa(*rule_args)   # noqa: E731

        def layer():
            prologue()
            assert rule() == 0
            epilogue()
        timed(tag + "_layer", layer, 0, tok)
        out[tag + "_layer"]["shape"] = {"B": B, "T": T, "key_heads": Hk, "value_heads": Hv, "d": d}
        if T > 1:
            # the same layer with the prologue inside the prefill's prep
            # (dn_layer_prefill): checked once through the binding, then timed as
            # a bare C-ABI call
            lws = dn.layer_prefill_workspace(B, T, Hk, Hv, d, torch.bfloat16, dev)
            cst3 = torch.empty_like(cst)
            dn.layer_prefill(x["qkv"], x["z"], x["b"], x["a"], x["conv_w"], x["A_log"], x["dt_bias"],
                             x["norm_w"], Hk, Hv, conv_state=x["conv_state"], conv_state_out=cst3,
                             S_final=S, out=y, workspace=lws)
            lp_args = (P(x["qkv"]), P(x["conv_w"]), P(x["conv_state"]), P(cst3), P(x["b"]), P(x["a"]),
                       P(x["A_log"]), P(x["dt_bias"]), P(x["z"]), P(x["norm_w"]), 1e-6, None, P(S),
                       P(y), 0, B, T, Hk, Hv, d, 1, P(lws), lws.numel(), st)
            lp = lambda: lib.dn_layer_prefill(*lp_args)   # noqa: E731
            timed(tag + "_layer_prologue_in_prep", lp, 0, tok)
            out[tag + "_layer_prologue_in_prep"]["what"] = (
                "dn_layer_prefill: the prologue formed in the prefill's prep (three launches: prep, "
                "scan, epilogue); bitwise the result of the three separate calls")
            del lws, cst3
        if T == 1:
            # the same layer step as one kernel (dn_layer_decode_step): checked
            # once through the binding, then timed as a bare C-ABI call
            cst2 = torch.empty_like(cst)
            dn.layer_decode_step(x["qkv"], x["z"], x["b"], x["a"], x["conv_w"], x["A_log"],
                                 x["dt_bias"], x["norm_w"], Hk, Hv, S, conv_state=x["conv_state"],
                                 conv_state_out=cst2, out=y)
            fused_args = (P(x["qkv"]), P(x["conv_w"]), P(x["conv_state"]), P(cst2), P(x["b"]),
                          P(x["a"]), P(x["A_log"]), P(x["dt_bias"]), P(x["z"]), P(x["norm_w"]), 1e-6,
                          P(S), P(y), 0, B, Hk, Hv, d, 1, st)
            fused = lambda: lib.dn_layer_decode_step(*fused_args)   # noqa: E731
            fused_bytes = (2 * B * Hv * d * d * 4 + pro_bytes - (2 * B * Hk + B * Hv) * d * 2
                           - 2 * B * Hv * 2 + 2 * B * Hv * d * 2)
            timed(tag + "_layer_one_kernel", lambda: fused() == 0 or None, fused_bytes, tok)
            out[tag + "_layer_one_kernel"]["what"] = (
                "dn_layer_decode_step: prologue, decode step and gated RMSNorm in one kernel; "
                "bytes: the state read and written once, qkv, b, a, z, conv_w, norm_w read, the "
                "two conv histories, out written")
            del cst2
        del x, q, k, v, beta, g, cst, o, y, S
    return out


if __name__ == "__main__":
    main()

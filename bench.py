#!/usr/bin/env python3
"""Benchmark of the Gated Delta Rule hot path on one MI355X (gfx950).

One step = one gdr_chunk_prefill call (chunk map, intra-chunk kernel, state
scan, output kernel) on the varlen prefill workload B=4, lengths
[1000, 4096, 300, 2796] (T = 8192), Nqk = 16, Nv = 32, D = 128, bf16
activations, fp32 states.  `value` is prefill tokens per second with inputs
resident in HBM.  The same run also times gdr_recurrent_decode on the decode
workload B=256 x 1 token, Nk=16, Nv=32, Dk=Dv=128, bf16 pool of 512 slots
(reported under "decode").

Timing: W untimed warm-up steps, then K steps bracketed by
torch.cuda.synchronize() on both sides, wall clock.  Inputs rotate over
--sets device copies (default 4, about 0.9 GB for prefill and 2 GiB of
pools for decode) so that the 256 MB Infinity Cache cannot hold one step's
inputs until the next.  Kernel durations come from hipEvents that the
library records around its kernels on the launch stream (gdr_timing_*).
Each event pair delays the stream by a few microseconds, so the timed
region records them around the dominant kernel only (its average is the
roofline's duration); the per-kernel breakdown comes from a short untimed
pass with every kernel's events, run before the timed region.  Kernels that
a call launches more than once (the phased scan and output) are reported
per call, summed over their launches.

Roofline: algorithmic flops per kernel (MFMA-bound kernels, fp16 dense peak
2.5 PFLOP/s) or algorithmic bytes (HBM-bound decode, 8 TB/s); the formulas
are in flops_prefill() / bytes_decode() below.  `traffic` is the HBM byte
count of the dominant kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE counter
runs recorded in profiles/counters.json, reported only while the kernel's
source file is unchanged since those counters were taken; for a contraction
kernel it is also given as a rate over the same duration and a fraction of
the 8 TB/s HBM peak (the prefill kernels move their workspace tiles through
HBM, and that, more than the matrix cores, bounds them).

cpu_baseline: the fp64 oracle (test infrastructure, one call on the full
workload, timed on this host's cores) -- a reported baseline, not a target.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_PEAK_FP16 = 2.5e15     # MI355X dense fp16/bf16 MFMA, FLOP/s
HBM_PEAK = 8.0e12           # MI355X HBM3E, B/s
D = 128
L = 128
KERNEL_SOURCES = {
    "gdr_chunkmap": "gated_delta_rule_chunk_amd/csrc/gdr_prefill.hip",
    "gdr_intra": "gated_delta_rule_chunk_amd/csrc/gdr_prefill.hip",
    "gdr_scan": "gated_delta_rule_chunk_amd/csrc/gdr_prefill.hip",
    "gdr_output": "gated_delta_rule_chunk_amd/csrc/gdr_prefill.hip",
    "gdr_decode": "gated_delta_rule_chunk_amd/csrc/gdr_decode.hip",
}


def chunk_rows(seq_lens):
    """Valid rows r of every 128-token chunk."""
    rows = []
    for n in seq_lens:
        rows += [min(L, n - s) for s in range(0, n, L)]
    return rows


def flops_prefill(seq_lens, Nqk, Nv):
    """Algorithmic flops of each prefill kernel, per call.

    Per chunk of r rows: intra  = Nv (2 r^2 D + r^3 / 3) + Nqk r^2 D
                                  (u, w: triangular r x r by r x D; the solve;
                                  lower half of the shared Gram k^ k^T)
                         scan   = Nv 4 r D^2   (w S and k^T v_new)
                         output = Nv (2 r D^2 + r^2 D) + Nqk r^2 D
                                  ((q^ e^g) S, P v_new, lower half of q^ k^T)
    Their sum is 6 r D^2 + 3 r^2 D + r^3/3 per value head plus 2 r^2 D per
    qk head.
    """
    f = {"gdr_chunkmap": 0.0, "gdr_intra": 0.0, "gdr_scan": 0.0, "gdr_output": 0.0}
    for r in chunk_rows(seq_lens):
        f["gdr_intra"] += Nv * (2 * r * r * D + r ** 3 / 3) + Nqk * r * r * D
        f["gdr_scan"] += Nv * 4 * r * D * D
        f["gdr_output"] += Nv * (2 * r * D * D + r * r * D) + Nqk * r * r * D
    return f


def bytes_prefill(T, B, Nqk, Nv, act_bytes=2):
    """Algorithmic HBM bytes of a prefill call: q, k, v, beta, out in the
    activation dtype, g fp32, state in and out fp32."""
    return (T * (2 * Nqk + 2 * Nv) * D + T * Nv) * act_bytes + T * Nv * 4 + 2 * B * Nv * D * D * 4


def bytes_decode(inp):
    """Algorithmic HBM bytes of a decode call: every read slab once, every
    distinct written slab once, plus the valid tokens' activations."""
    import numpy as np
    B, S, Nk, Nv, Dk, Dv = (inp[k] for k in ("B", "S", "Nk", "Nv", "Dk", "Dv"))
    sb = 4 if inp["state"] == "fp32" else 2
    ab = 4 if inp["act"] == "fp32" else 2
    idx = inp["idx"].numpy().reshape(B, S)
    lens = inp["lens"].numpy()
    slab = Nv * Dk * Dv * sb
    state = sum(slab * (1 + len(set(idx[b, :lens[b]].tolist()))) for b in range(B) if lens[b] > 0)
    ntok = int(lens.sum())
    act = ntok * (2 * Nk * Dk * ab + Nv * Dv * ab + Nv * ab + Nv * 4 + Nv * Dv * ab)
    if inp["gk"] is not None:
        act += ntok * Nv * Dk * 4
    return state + act + B * 4 + B * S * 4


def source_hash(path):
    return hashlib.sha256(open(os.path.join(ROOT, path), "rb").read()).hexdigest()[:16]


def counter_traffic(kernel):
    """HBM bytes per launch from the committed counter runs, or None if the
    kernel's source changed since they were taken."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(kernel)
    if not rec or rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("hbm_bytes_per_launch")


def timed(fn, steps, warmup, gdr, torch):
    """Warm up; take the per-kernel breakdown in an untimed pass with every
    kernel's events; then time `steps` steps with events around the dominant
    kernel (the most time per call) only.  Returns (seconds, breakdown
    {name: (ms per call, launches per call)}, dominant name, its (ms per
    call, launches per call) over the timed region)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    gdr.timing_read()            # discard warm-up records
    probe = max(3, min(steps, 10))
    gdr.timing_enable(True)
    for i in range(probe):
        fn(warmup + i)
    torch.cuda.synchronize()
    gdr.timing_enable(False)
    breakdown = {k: (v[0] / probe, v[1] / probe) for k, v in gdr.timing_read().items() if v[1]}
    dominant = max(breakdown, key=lambda k: breakdown[k][0])
    gdr.timing_enable(True, kernels=[dominant])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fn(warmup + probe + i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    gdr.timing_enable(False)
    ms, n = gdr.timing_read()[dominant]
    return dt, breakdown, dominant, (ms / steps, n / steps)


def roofline(name, avg_s, flops=None, nbytes=None):
    if flops is not None:
        a = flops / avg_s
        tr = counter_traffic(name)
        r = {"bound": "mfma", "achieved": a / 1e12, "peak": MFMA_PEAK_FP16 / 1e12, "unit": "TFLOP/s",
             "frac": a / MFMA_PEAK_FP16, "traffic": tr, "kernel": name}
        if tr:   # the same kernel against HBM: its counter-measured bytes over the same duration
            r["traffic_rate_GBps"] = tr / avg_s / 1e9
            r["traffic_hbm_frac"] = tr / avg_s / HBM_PEAK
        return r
    a = nbytes / avg_s
    return {"bound": "hbm", "achieved": a / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s", "frac": a / HBM_PEAK,
            "traffic": counter_traffic(name), "kernel": name}


def bench_prefill(args, gdr, torch, workloads):
    inp = workloads.config_inputs(2)
    dev = "cuda:0"
    base = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    names = ("q", "k", "v", "g", "beta", "state_in")
    sets = [base] + [dict(base, **{n: base[n].clone() for n in names}) for _ in range(args.sets - 1)]
    T, B, Nqk, Nv = inp["T"], inp["B"], inp["Nqk"], inp["Nv"]
    out = torch.empty((T, Nv, D), dtype=torch.bfloat16, device=dev)
    st = torch.empty((B, Nv, D, D), dtype=torch.float32, device=dev)
    ws = torch.empty(gdr.chunk_prefill_workspace_size(T, B, Nqk, Nv), dtype=torch.uint8, device=dev)

    def step(i):
        s = sets[i % len(sets)]
        gdr.chunk_prefill(s["q"], s["k"], s["v"], s["g"], s["beta"], s["cu_seqlens"], s["scale"],
                          state_in=s["state_in"], out=out, state_out=st, workspace=ws)

    dt, per, dominant, live = timed(step, args.steps, args.warmup, gdr, torch)
    seq_lens = [1000, 4096, 300, 2796]
    fl = flops_prefill(seq_lens, Nqk, Nv)
    kernels = {}
    for name in fl:
        ms, n = per.get(name, (0.0, 0))
        per_call = ms / 1e3
        kernels[name] = {"us_per_call": per_call * 1e6, "launches_per_call": n, "alg_gflop": fl[name] / 1e9,
                         "mfma_frac": (fl[name] / per_call / MFMA_PEAK_FP16) if per_call > 0 and fl[name] else None}
    # the dominant kernel's time per call over the timed region itself (one
    # launch per call: its average launch duration)
    dom_avg = live[0] / 1e3
    kernels[dominant]["us_per_call_timed_region"] = dom_avg * 1e6
    step_s = dt / args.steps
    f_total = sum(fl.values())
    b_total = bytes_prefill(T, B, Nqk, Nv)
    return dict(inp=inp, step_s=step_s, tok_s=T / step_s, kernels=kernels,
                roofline=roofline(dominant, dom_avg, flops=fl[dominant]),
                path={"alg_gflop": f_total / 1e9, "mfma_frac": f_total / step_s / MFMA_PEAK_FP16,
                      "alg_bytes_mb": b_total / 1e6, "hbm_frac": b_total / step_s / HBM_PEAK})


def bench_decode(args, gdr, torch, workloads):
    inp = workloads.config_inputs(3)
    dev = "cuda:0"
    base = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    names = ("q", "k", "v", "g", "beta", "pool")
    sets = [base] + [dict(base, **{n: base[n].clone() for n in names}) for _ in range(args.sets - 1)]
    out = torch.empty((inp["B"], inp["Nv"], inp["S"], inp["Dv"]), dtype=torch.bfloat16, device=dev)

    def step(i):
        s = sets[i % len(sets)]
        gdr.recurrent_decode(s["q"], s["k"], s["v"], s["g"], s["gk"], s["beta"], s["pool"], s["idx"],
                             s["lens"], s["scale"], out=out)

    steps = max(args.steps * 4, 20)
    dt, per, _, live = timed(step, steps, args.warmup, gdr, torch)
    # reference: a plain device copy moving the same number of bytes (half read, half written)
    nb_copy = (bytes_decode(inp) // 2 + 255) // 256 * 256
    src = torch.empty(nb_copy, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * nb_copy * 20 / (e0.elapsed_time(e1) / 1e3) / 1e9
    del src, dst
    ms, n = live
    avg = ms / 1e3 / max(n, 1)
    nb = bytes_decode(inp)
    ntok = int(inp["lens"].sum())
    return dict(inp=inp, step_s=dt / steps, steps=steps, tok_s=ntok / (dt / steps), kernel_avg_us=avg * 1e6,
                roofline=roofline("gdr_decode", avg, nbytes=nb), alg_bytes_mb=nb / 1e6, copy_gbs=copy_gbs)


def time_config(n, args, gdr, torch, workloads):
    """Per-call time of one configured workload (inputs resident, one set);
    n is a config number or the name of an extra workload."""
    inp = workloads.config_inputs(n) if isinstance(n, int) else workloads.extra_inputs(n)
    dev = "cuda:0"
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    if "cu_seqlens" in inp:
        ws = torch.empty(gdr.chunk_prefill_workspace_size(inp["T"], inp["B"], inp["Nqk"], inp["Nv"],
                                                          gk=inp.get("gk") is not None),
                         dtype=torch.uint8, device=dev)

        def f(i):
            gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["scale"],
                              state_in=d["state_in"], workspace=ws, gk=d.get("gk"))
        ntok = inp["T"]
    else:
        def f(i):
            gdr.recurrent_decode(d["q"], d["k"], d["v"], d["g"], d["gk"], d["beta"], d["pool"], d["idx"],
                                 d["lens"], d["scale"])
        ntok = int(inp["lens"].sum())
    steps = 20 if ntok < 65536 else 5
    dt, per, _, _ = timed(f, steps, 2, gdr, torch)
    name = workloads.CONFIG_NAMES[n] if isinstance(n, int) else workloads.EXTRA_NAMES[n]
    return {"config": name, "ms_per_call": dt / steps * 1e3, "tok_s": ntok / (dt / steps),
            "kernels_us_per_call": {k: round(v[0] * 1e3, 1) for k, v in per.items()}}


def cpu_baseline_prefill(inp):
    import oracle
    t0 = time.perf_counter()
    oracle.prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["state_in"], inp["cu_seqlens"],
                   inp["scale"])
    dt = time.perf_counter() - t0
    return {"value": inp["T"] / dt, "unit": "tok/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"one fp64 oracle call on the whole workload (T={inp['T']}, all {inp['Nv']} value "
                      f"heads): {dt:.2f} s wall"}


def cpu_baseline_decode(inp):
    import oracle
    t0 = time.perf_counter()
    oracle.decode(inp["q"], inp["k"], inp["v"], inp["g"], inp["gk"], inp["beta"], inp["pool"], inp["idx"],
                  inp["lens"], inp["scale"], round_state_bf16=True)
    dt = time.perf_counter() - t0
    ntok = int(inp["lens"].sum())
    return {"value": ntok / dt, "unit": "tok/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"one fp64 oracle call on the whole workload ({ntok} tokens x {inp['Nv']} heads): "
                      f"{dt:.2f} s wall"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=4, help="rotating device copies of the inputs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "decode"], default="all",
                    help="time one path only (for counter runs)")
    ap.add_argument("--all-configs", action="store_true",
                    help="also time every configured workload (one line per workload, after the main line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (3 launches), the reference for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this operator is measured on one GPU only (got --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import gated_delta_rule_chunk_amd as gdr
    import workloads

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "launches": 3}))
        return
    gdr.lib()
    if args.only != "all":
        res = (bench_prefill if args.only == "prefill" else bench_decode)(args, gdr, torch, workloads)
        print(json.dumps({"only": args.only, "ms_per_step": res["step_s"] * 1e3, "tok_s": res["tok_s"]}))
        return
    pre = bench_prefill(args, gdr, torch, workloads)
    dec = bench_decode(args, gdr, torch, workloads)
    inp = pre["inp"]
    line = {
        "metric": "GDR prefill tok/s (T=8192) + decode tok/s; % MFMA / % HBM peak",
        "value": pre["tok_s"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pre["step_s"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 MFMA operands, fp32 accumulate/state (bf16 I/O)",
        "data": "synthetic",
        "config": {"workload": workloads.CONFIG_NAMES[2], "global_batch": inp["B"], "seq_len": inp["T"],
                   "parallelism": "single GPU", "input_sets_rotated": args.sets},
        "roofline": pre["roofline"],
        "path": pre["path"],
        "kernels": pre["kernels"],
        "decode": {"metric": "GDR decode tok/s", "value": dec["tok_s"], "unit": "tok/s",
                   "workload": workloads.CONFIG_NAMES[3], "steps": dec["steps"],
                   "ms_per_call": dec["step_s"] * 1e3, "kernel_avg_us": dec["kernel_avg_us"],
                   "alg_bytes_mb": dec["alg_bytes_mb"], "roofline": dec["roofline"],
                   "device_copy_reference_GBps": dec["copy_gbs"]},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(inp)
        line["decode"]["cpu_baseline"] = cpu_baseline_decode(dec["inp"])
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line))
    if args.all_configs:
        for n in (1, 2, 3, 4, 5, *workloads.EXTRA_NAMES):
            print(json.dumps(time_config(n, args, gdr, torch, workloads)), flush=True)


if __name__ == "__main__":
    main()

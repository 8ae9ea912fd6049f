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
MFMA_PEAK_FP32 = 157.3e12    # MI355X dense fp32 MFMA, FLOP/s
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


def flops_tile(seq_lens, Nv):
    """F_tile: the flops of the dense 128-token tiles the kernels work on --
    8 dense 128^3 contractions (Gram, u, w, P, v', (q^ e^g) S, P v_new, the
    state update) plus the triangular solve (L^3 / 3) per value head and
    chunk, ragged chunks counted as full."""
    nchunks = sum((n + L - 1) // L for n in seq_lens)
    return nchunks * Nv * (8 * 2 * L * D * D + L ** 3 / 3)


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


def counter_record(kernel):
    """The kernel's record in the committed counter runs
    (profiles/counters.json), or None if its source changed since they
    were taken."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(kernel)
    if not rec or rec.get("source_sha256_16") != source_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec


def counter_traffic(kernel):
    """HBM bytes per launch from the committed counter runs, or None."""
    rec = counter_record(kernel)
    return rec.get("hbm_bytes_per_launch") if rec else None


def counter_mfma(kernel):
    """Executed MFMA flops per launch and the fraction of cycles the matrix
    cores were busy, from the committed counter runs, or (None, None)."""
    rec = counter_record(kernel)
    if not rec:
        return None, None
    return rec.get("mfma_flops_per_launch"), rec.get("mfma_busy_frac")


def timed(fn, steps, warmup, gdr, torch, whole_region=False):
    """Warm up; take the per-kernel breakdown in an untimed pass with every
    kernel's events; then time `steps` steps with events around the dominant
    kernel (the most time per call) only.  Returns (seconds, breakdown
    {name: (ms per call, launches per call)}, dominant name, its (ms per
    call, launches per call) over the timed region).

    whole_region: for a step that is one launch of one kernel (the decode),
    one event pair on the launch stream brackets the whole timed region
    instead of a pair per launch; a pair per launch adds its own few
    microseconds to each launch it brackets, which shows against a kernel of
    about 100 us (rocprofv3's kernel trace agrees with the whole-region
    average, not with the per-launch one)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    gdr.timing_read()            # discard warm-up records
    # The breakdown pass runs 100 steps (at least 20 ms of the T=8192 prefill,
    # whatever `steps` is).  Besides averaging the per-kernel times over more
    # launches, it puts the timed region after the part has settled under the
    # workload's load: a cold process ran its first 50 prefill steps at 257 us
    # each and was at 186-190 us from about the 100th (one box), and 50 steps
    # after a pause of a second ran at 216-220 us.
    probe = 100
    gdr.timing_enable(True)
    for i in range(probe):
        fn(warmup + i)
    torch.cuda.synchronize()
    gdr.timing_enable(False)
    breakdown = {k: (v[0] / probe, v[1] / probe) for k, v in gdr.timing_read().items() if v[1]}
    dominant = max(breakdown, key=lambda k: breakdown[k][0])
    if whole_region:
        if len(breakdown) != 1 or breakdown[dominant][1] != 1:
            raise RuntimeError(f"whole-region timing needs one launch of one kernel per step, got {breakdown}")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record()
        for i in range(steps):
            fn(warmup + probe + i)
        e1.record()
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        return dt, breakdown, dominant, (e0.elapsed_time(e1) / steps, 1.0)
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
    mfma_exec_total = 0.0
    for name in fl:
        ms, n = per.get(name, (0.0, 0))
        if not n:   # not launched for this workload (the chunk map is built inside the intra kernel)
            continue
        per_call = ms / 1e3
        kernels[name] = {"us_per_call": per_call * 1e6, "launches_per_call": n, "alg_gflop": fl[name] / 1e9,
                         "mfma_frac": (fl[name] / per_call / MFMA_PEAK_FP16) if per_call > 0 and fl[name] else None}
        fx, busy = counter_mfma(name)
        if fx is not None and n:
            kernels[name]["mfma_executed_gflop"] = fx * n / 1e9
            kernels[name]["mfma_busy_frac_counter"] = busy
            mfma_exec_total += fx * n
    # the dominant kernel's time per call over the timed region itself (one
    # launch per call: its average launch duration)
    dom_avg = live[0] / 1e3
    kernels[dominant]["us_per_call_timed_region"] = dom_avg * 1e6
    step_s = dt / args.steps
    f_total = sum(fl.values())
    f_tile = flops_tile(seq_lens, Nv)
    b_total = bytes_prefill(T, B, Nqk, Nv)
    path = {"alg_gflop": f_total / 1e9, "mfma_frac": f_total / step_s / MFMA_PEAK_FP16,
            "tile_gflop": f_tile / 1e9, "mfma_frac_tile": f_tile / step_s / MFMA_PEAK_FP16,
            "alg_bytes_mb": b_total / 1e6, "hbm_frac": b_total / step_s / HBM_PEAK,
            # the larger of the two floors (MFMA at peak, HBM at peak) over the time taken
            "attainable_frac": max(f_total / MFMA_PEAK_FP16, b_total / HBM_PEAK) / step_s}
    if mfma_exec_total:
        path["mfma_executed_gflop"] = mfma_exec_total / 1e9
        path["mfma_frac_executed"] = mfma_exec_total / step_s / MFMA_PEAK_FP16
    return dict(inp=inp, step_s=step_s, tok_s=T / step_s, kernels=kernels,
                roofline=roofline(dominant, dom_avg, flops=fl[dominant]), path=path)


def bench_decode(args, gdr, torch, workloads):
    inp = workloads.config_inputs(3)
    if args.decode_contiguous_slots:
        # reference run: the same rows in slots 0 .. B-1 in row order
        inp["idx"] = torch.arange(inp["idx"].numel(), dtype=torch.int32)
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
    dt, per, _, live = timed(step, steps, args.warmup, gdr, torch, whole_region=True)
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
    t = dt / steps
    rec = {"config": name, "ms_per_call": t * 1e3, "tok_s": ntok / t,
           "kernels_us_per_call": {k: round(v[0] * 1e3, 1) for k, v in per.items()}}
    if "cu_seqlens" in inp:
        lens = [int(x) for x in (inp["cu_seqlens"][1:] - inp["cu_seqlens"][:-1]).tolist()]
        fa = sum(flops_prefill(lens, inp["Nqk"], inp["Nv"]).values())
        ab = 4 if inp["act"] == "fp32" else 2
        nb = bytes_prefill(inp["T"], inp["B"], inp["Nqk"], inp["Nv"], ab)
        if inp.get("gk") is not None:
            nb += inp["T"] * inp["Nv"] * D * 4
        rec.update(alg_gflop=fa / 1e9, mfma_frac=fa / t / MFMA_PEAK_FP16, alg_bytes_mb=nb / 1e6,
                   hbm_frac=nb / t / HBM_PEAK,
                   attainable_frac=max(fa / MFMA_PEAK_FP16, nb / HBM_PEAK) / t)
    else:
        nb = bytes_decode(inp)
        rec.update(alg_bytes_mb=nb / 1e6, hbm_frac=nb / t / HBM_PEAK,
                   kernel_hbm_frac=nb / (per["gdr_decode"][0] / 1e3) / HBM_PEAK)
    return rec


def host_cpu():
    """The host's CPU model (first "model name" of /proc/cpuinfo) and the
    logical CPUs this process may run on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": len(os.sched_getaffinity(0))}


def cpu_baseline_prefill(inp):
    """The oracle on the whole workload; inputs are widened to fp64 before
    the clock starts, so only the oracle call is timed."""
    import oracle
    w = {n: oracle._f64(inp[n]) for n in ("q", "k", "v", "g", "beta", "state_in")}
    t0 = time.perf_counter()
    oracle.prefill(w["q"], w["k"], w["v"], w["g"], w["beta"], w["state_in"], inp["cu_seqlens"], inp["scale"])
    dt = time.perf_counter() - t0
    return {"value": inp["T"] / dt, "unit": "tok/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"one fp64 oracle call on the whole workload (T={inp['T']}, all {inp['Nv']} value "
                      f"heads; inputs widened to fp64 before timing): {dt:.2f} s wall", **host_cpu()}


def cpu_baseline_decode(inp):
    """The oracle on the whole workload; inputs (the pool included) are
    widened to fp64 before the clock starts and the pool is updated in
    place, so only the recurrence is timed."""
    import oracle
    w = {n: oracle._f64(inp[n]) for n in ("q", "k", "v", "g", "beta", "pool")}
    t0 = time.perf_counter()
    oracle.decode(w["q"], w["k"], w["v"], w["g"], inp["gk"], w["beta"], w["pool"], inp["idx"], inp["lens"],
                  inp["scale"], round_state_bf16=True, in_place=True)
    dt = time.perf_counter() - t0
    ntok = int(inp["lens"].sum())
    return {"value": ntok / dt, "unit": "tok/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"one fp64 oracle call on the whole workload ({ntok} tokens x {inp['Nv']} heads; inputs "
                      f"widened to fp64 before timing, pool updated in place): {dt:.3f} s wall", **host_cpu()}


# Kernel functions of each timing id (the per-key-gate and two-level variants
# included), for matching rocprofv3 kernel names.
def stream_ceiling(torch):
    """HBM rates of plain streams on this GPU, with torch's elementwise
    kernels: in-place x.mul_(1) (every byte read, then written back to the
    same address: the access pattern of an in-place state update) and an
    out-of-place copy, over four rotating 512 MiB bf16 buffers (2 GiB, so the
    256 MB last-level cache holds none of them between launches).  Bytes
    counted: read + written."""
    n = 256 << 20   # bf16 elements: 512 MiB
    bufs = [torch.ones(n, dtype=torch.bfloat16, device="cuda:0") for _ in range(4)]
    dst = [torch.empty_like(b) for b in bufs]
    res = {}
    for name, fn in (("in_place_update", lambda i: bufs[i % 4].mul_(1.0)),
                     ("out_of_place_copy", lambda i: dst[i % 4].copy_(bufs[(i + 1) % 4]))):
        for i in range(4):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(20):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) / 1e3 / 20
        res[name] = {"GBps": 2 * n * 2 / s / 1e9, "hbm_frac": 2 * n * 2 / s / HBM_PEAK, "us_per_launch": s * 1e6}
    del bufs, dst
    res.update(slab_stream(torch))
    return {"stream_ceiling": res, "bytes_per_launch": 2 * n * 2}


def slab_stream(torch):
    """The one-token decode's memory traffic without its arithmetic
    (gdr_slab_stream_probe) on the B=256 decode workload's pool shape: every
    row's 128 x 128 bf16 slabs read and written back in place, with the
    workload's seeded random slots and with row b in slot b; four pools
    rotated, as the decode bench does."""
    import gated_delta_rule_chunk_amd as gdr
    import workloads
    inp = workloads.config_inputs(3)
    B, Nv, slots = inp["B"], inp["Nv"], inp["num_slots"]
    pools = [inp["pool"].to("cuda:0")] + [inp["pool"].to("cuda:0") for _ in range(3)]
    res = {}
    for name, idx in (("decode_slabs_random_slots", inp["idx"][:B]),
                      ("decode_slabs_slot_order", torch.arange(B, dtype=torch.int32))):
        idx = idx.to(torch.int32).to("cuda:0")
        nbytes = 2 * B * Nv * 128 * 128 * 2
        for i in range(4):
            gdr.slab_stream_probe(pools[i % 4], idx)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(40):
            gdr.slab_stream_probe(pools[i % 4], idx)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3 / 40
        res[name] = {"GBps": nbytes / t / 1e9, "hbm_frac": nbytes / t / HBM_PEAK, "us_per_launch": t * 1e6}
    return res


def mfma_peak(torch, gdr):
    """Dense MFMA issue rates of this GPU from the library's probe
    (gdr_mfma_peak_probe): per instruction kind, two launches to warm up, then
    five timed with hipEvents on the probe's stream; TFLOP/s, the fraction of
    the published dense peak of that dtype, the shader clock the probe ran at
    (median over workgroups, last launch) and the fraction rescaled to the
    published 2.4 GHz."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 8 * 256, dtype=torch.float32, device="cuda:0")
    published = {"f16_16x16x32": MFMA_PEAK_FP16, "bf16_16x16x32": MFMA_PEAK_FP16,
                 "f16_16x16x16": MFMA_PEAK_FP16, "f32_16x16x4": MFMA_PEAK_FP32, "f16_32x32x16": MFMA_PEAK_FP16}
    iters = {"f16_16x16x32": 2000, "bf16_16x16x32": 2000, "f16_16x16x16": 2000, "f32_16x16x4": 1000,
             "f16_32x32x16": 2000}
    res = {}
    for kind in gdr.PROBE_KINDS:
        for _ in range(2):
            gdr.mfma_peak_probe(kind, iters[kind], sink)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        flops = sum(gdr.mfma_peak_probe(kind, iters[kind], sink) for _ in range(5))
        e1.record()
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) / 1e3
        mhz = sink[::256].float().median().item()
        res[kind] = {"TFLOP_s": flops / s / 1e12, "frac_of_published": flops / s / published[kind],
                     "us_per_launch": s / 5 * 1e6, "shader_clock_MHz": mhz,
                     "frac_of_published_at_2400MHz": flops / s / published[kind] * 2400.0 / mhz if mhz else None}
    return res


KERNEL_FUNCTIONS = {"chunkmap_kernel": "gdr_chunkmap", "intra_kernel": "gdr_intra", "intra_gk_kernel": "gdr_intra",
                    "scan_kernel": "gdr_scan", "scan_gk_out_kernel": "gdr_scan", "combine_kernel": "gdr_scan",
                    "output_kernel": "gdr_output", "output_gk_kernel": "gdr_output",
                    "decode_kernel": "gdr_decode", "decode1_kernel": "gdr_decode"}


def _kernel_id(name):
    import re
    m = re.search(r"::(\w+)(?:<|\()", name.replace("(anonymous namespace)", "anon"))
    if m and m.group(1) in KERNEL_FUNCTIONS:
        return KERNEL_FUNCTIONS[m.group(1)]
    return "copy" if "copyBuffer" in name else None


def _csv_means(path):
    """{kernel id: {counter: mean value per dispatch}} from a rocprofv3
    counter_collection.csv."""
    import csv
    import collections
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(path)):
        kid = _kernel_id(r["Kernel_Name"])
        if kid:
            acc[kid][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in acc.items()}


def ingest_counters(fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, mfma_csv):
    """Write profiles/counters.json from rocprofv3 --pmc runs: FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) of bench.py, the same counters of
    `bench.py --copy-calibration` (a plain 1 GiB copy, 3 launches: the
    scale factors), and SQ_INSTS_VALU_MFMA_MOPS_F16 / _F32,
    SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE of bench.py."""
    fetch, write = _csv_means(fetch_csv), _csv_means(write_csv)
    n = 1 << 30
    # the copy's launches are the copyBuffer dispatches with the largest counts
    import csv
    cf = max(float(r["Counter_Value"]) for r in csv.DictReader(open(cal_fetch_csv)) if "copyBuffer" in r["Kernel_Name"])
    cw = max(float(r["Counter_Value"]) for r in csv.DictReader(open(cal_write_csv)) if "copyBuffer" in r["Kernel_Name"])
    ff, fw = n / (cf * 1024), n / (cw * 1024)
    mf = _csv_means(mfma_csv) if mfma_csv else {}
    out = {"_calibration": {"copy_bytes": n, "fetch_counter_KiB": cf, "write_counter_KiB": cw,
                            "fetch_factor": ff, "write_factor": fw},
           "_mfma_busy_note": "busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs)"}
    for kid in sorted(set(KERNEL_FUNCTIONS.values())):
        if kid not in fetch or kid not in write:
            continue
        rb = fetch[kid]["FETCH_SIZE"] * 1024 * ff
        wb = write[kid]["WRITE_SIZE"] * 1024 * fw
        rec = {"source_sha256_16": source_hash(KERNEL_SOURCES[kid]), "source": KERNEL_SOURCES[kid],
               "fetch_KiB": fetch[kid]["FETCH_SIZE"], "write_KiB": write[kid]["WRITE_SIZE"],
               "read_bytes": rb, "write_bytes": wb, "hbm_bytes_per_launch": rb + wb}
        m = mf.get(kid)
        if m and "SQ_INSTS_VALU_MFMA_MOPS_F16" in m:
            mops = m["SQ_INSTS_VALU_MFMA_MOPS_F16"] + m.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0)
            rec["mfma_flops_per_launch"] = mops * 512
            if m.get("GRBM_GUI_ACTIVE"):
                rec["mfma_busy_frac"] = m["SQ_VALU_MFMA_BUSY_CYCLES"] / (m["GRBM_GUI_ACTIVE"] / 8 * 1024)
        out[kid] = rec
    path = os.path.join(ROOT, "profiles", "counters.json")
    json.dump(out, open(path, "w"), indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=4, help="rotating device copies of the inputs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "decode"], default="all",
                    help="time one path only (for counter runs)")
    ap.add_argument("--no-configs", action="store_true",
                    help="leave out the per-workload records (the \"configs\" key of the line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (3 launches), the reference for scaling "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes")
    ap.add_argument("--decode-contiguous-slots", action="store_true",
                    help="reference run: time the decode with its rows in slots 0 .. B-1 in row order instead of "
                         "the workload's seeded random slots (the pool's access order only; same arithmetic)")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="measure plain HBM streams the decode is compared with: an in-place update (read then "
                         "write the same bytes, like the decode's slab update) and an out-of-place copy, each over "
                         "four rotating 512 MiB bf16 buffers; prints one JSON line")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="measure the dense MFMA issue rate of each instruction kind the kernels use with the "
                         "library's probe; prints one JSON line")
    ap.add_argument("--config", metavar="NAME",
                    help="time one workload only (a config number 1-5 or an extra workload's name, e.g. "
                         "long_few_heads) and print its record as one JSON line (for per-workload profiles)")
    ap.add_argument("--ingest-counters", nargs=5, metavar=("FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE", "MFMA"),
                    help="write profiles/counters.json from rocprofv3 counter_collection.csv files and exit")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.gpus != 1:
        print(f"bench.py: this operator is measured on one GPU only (got --gpus {args.gpus}); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import gated_delta_rule_chunk_amd as gdr
    import workloads

    if args.stream_ceiling:
        print(json.dumps(stream_ceiling(torch)))
        return
    if args.mfma_peak:
        print(json.dumps({"mfma_peak": mfma_peak(torch, gdr)}))
        return
    if args.config:
        n = int(args.config) if args.config.isdigit() else args.config
        if n not in workloads.CONFIG_NAMES and n not in workloads.EXTRA_NAMES:
            print(f"bench.py: unknown workload {args.config!r}", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(time_config(n, args, gdr, torch, workloads)))
        return
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
        line = {"only": args.only, "ms_per_step": res["step_s"] * 1e3, "tok_s": res["tok_s"]}
        if args.only == "decode":
            line.update(kernel_avg_us=res["kernel_avg_us"], roofline=res["roofline"],
                        contiguous_slots=bool(args.decode_contiguous_slots))
        print(json.dumps(line))
        return
    # the ceilings measured on this GPU (plain HBM streams, dense MFMA issue
    # rates), taken before the timed workloads
    ceilings = {"hbm": stream_ceiling(torch)["stream_ceiling"], "mfma": mfma_peak(torch, gdr)}
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
    # the ceilings measured on this GPU, beside the published peaks the
    # roofline objects use: dense MFMA issue rates and plain HBM streams
    line["measured_ceilings"] = ceilings
    if not args.no_configs:
        # the other configured workloads (the T=8192 prefill and the B=256
        # decode are the entries above) and the extra ones, each timed on its
        # own with one input set resident
        line["configs"] = {str(n): time_config(n, args, gdr, torch, workloads)
                           for n in (1, 4, 5, *workloads.EXTRA_NAMES)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(inp)
        line["decode"]["cpu_baseline"] = cpu_baseline_decode(dec["inp"])
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line))


if __name__ == "__main__":
    main()

"""Opt-in per-kernel timing (gdr_timing_*) on the GPU, through the C ABI.

A timed launch goes through hipExtLaunchKernelGGL with the timing events; an
untimed one through hipLaunchKernelGGL.  Both must run the same kernel on the
same arguments, so results with timing on are compared bit for bit with
results with timing off, and the timing records are checked for one launch
per kernel per call with a positive duration.
"""
import pytest
import torch

import gated_delta_rule_chunk_amd as gdr
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def to_dev(inp):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


@pytest.mark.parametrize("gk", [None, "strong"])
def test_prefill_with_timing_on_is_bit_identical_and_records_each_kernel(gk):
    print(f"[timing] prefill gk={gk}", flush=True)
    d = to_dev(workloads.prefill_inputs(31, [300, 129, 700], Nqk=2, Nv=4, act="bf16", gk=gk))

    def call():
        return gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["scale"],
                                 state_in=d["state_in"], gk=d["gk"])

    out0, st0 = call()
    torch.cuda.synchronize()
    gdr.timing_read()   # drop anything recorded before
    gdr.timing_enable(True)
    try:
        out1, st1 = call()
        torch.cuda.synchronize()
        rec = gdr.timing_read()
    finally:
        gdr.timing_enable(False)
    assert torch.equal(bits(out0), bits(out1)) and torch.equal(bits(st0), bits(st1))
    # three sequences: the intra kernel builds the chunk map itself; with the
    # per-key gate the scan forms the output and no output kernel runs
    expect = {"gdr_chunkmap": 0, "gdr_intra": 1, "gdr_scan": 1, "gdr_output": 0 if gk else 1, "gdr_decode": 0}
    for name, n in expect.items():
        ms, launches = rec[name]
        assert launches == n, (name, rec)
        assert (ms > 0) == (n > 0), (name, rec)
    # with timing off again nothing is recorded
    call()
    torch.cuda.synchronize()
    assert all(v[1] == 0 for v in gdr.timing_read().values())


def test_decode_with_timing_on_is_bit_identical_and_records_one_launch():
    print("[timing] decode", flush=True)
    d = to_dev(workloads.decode_inputs(32, B=19, S=1, Nk=2, Nv=4, Dk=128, Dv=128, num_slots=40))

    def call():
        pool = d["pool"].clone()
        out, _ = gdr.recurrent_decode(d["q"], d["k"], d["v"], d["g"], d["gk"], d["beta"], pool, d["idx"],
                                      d["lens"], d["scale"])
        return out, pool

    out0, pool0 = call()
    torch.cuda.synchronize()
    gdr.timing_read()
    gdr.timing_enable(True, kernels=["gdr_decode"])
    try:
        out1, pool1 = call()
        torch.cuda.synchronize()
        rec = gdr.timing_read()
    finally:
        gdr.timing_enable(False)
    assert torch.equal(bits(out0), bits(out1)) and torch.equal(bits(pool0), bits(pool1))
    ms, launches = rec["gdr_decode"]
    assert launches == 1 and ms > 0, rec
    assert all(v[1] == 0 for k, v in rec.items() if k != "gdr_decode"), rec

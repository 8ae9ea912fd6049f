"""HIP graph capture of both entry points (through the C ABI).

Both calls issue only kernel launches on the caller's stream -- no
allocation, copy, memset or host synchronisation once the output, state and
workspace buffers are passed in -- so a graph can capture a call and replay
it.  Each replay follows eager work and a synchronisation of the program's
own, and is compared bit for bit with the eager call on the same buffers.
"""
import pytest
import torch

import gated_delta_rule_chunk_amd as gdr
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def capture(call):
    """Warm up on a side stream, then capture one call into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    return graph


def bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


@pytest.mark.parametrize("gk", [None, "strong"])
def test_prefill_replays_in_a_graph(gk):
    print(f"[graph] prefill gk={gk}", flush=True)
    inp = workloads.prefill_inputs(71, [300, 129, 0, 5], Nqk=2, Nv=4, act="bf16", gk=gk)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    T, B, Nv = inp["T"], inp["B"], inp["Nv"]
    out = torch.empty((T, Nv, 128), dtype=torch.bfloat16, device=DEV)
    st = torch.empty((B, Nv, 128, 128), dtype=torch.float32, device=DEV)
    ws = torch.empty(gdr.chunk_prefill_workspace_size(T, B, inp["Nqk"], Nv, gk=gk is not None),
                     dtype=torch.uint8, device=DEV)

    def call():
        gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["scale"],
                          state_in=d["state_in"], out=out, state_out=st, workspace=ws, gk=d.get("gk"))

    call()
    torch.cuda.synchronize()
    ref_out, ref_st = out.clone(), st.clone()
    graph = capture(call)
    for rep in range(3):
        out.fill_(0.0)
        st.fill_(0.0)
        ws.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(ref_out)), f"replay {rep}: out"
        assert torch.equal(bits(st), bits(ref_st)), f"replay {rep}: state"


def test_decode_replays_in_a_graph():
    print("[graph] decode B=64 S=4 gk two-slot routing", flush=True)
    inp = workloads.config_inputs(4)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    pool0 = d["pool"].clone()
    out = torch.empty((inp["B"], inp["Nv"], inp["S"], inp["Dv"]), dtype=torch.bfloat16, device=DEV)

    def call():
        gdr.recurrent_decode(d["q"], d["k"], d["v"], d["g"], d["gk"], d["beta"], d["pool"], d["idx"],
                             d["lens"], d["scale"], out=out)

    call()
    torch.cuda.synchronize()
    ref_out, ref_pool = out.clone(), d["pool"].clone()
    d["pool"].copy_(pool0)
    graph = capture(call)
    for rep in range(3):
        d["pool"].copy_(pool0)   # the pool is updated in place: start every replay from the same pool
        out.fill_(0.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(ref_out)), f"replay {rep}: out"
        assert torch.equal(bits(d["pool"]), bits(ref_pool)), f"replay {rep}: pool"

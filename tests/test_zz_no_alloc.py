"""gdr_chunk_prefill_noalloc (the allocation-free prefill, for callers that
cannot allocate) against gdr_chunk_prefill on the same inputs, through the
C ABI: two calls in a row, the second smaller, each bit-identical to the
workspace entry point and within the parity tolerances of the oracle."""
import pytest
import torch

import gated_delta_rule_chunk_amd as gdr
import oracle
import workloads
from parity import assert_out_close, assert_state_close

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _both(inp, gk=False):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    T, B, Nv = inp["T"], inp["B"], inp["Nv"]
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["scale"])
    o1, s1 = gdr.chunk_prefill(*args, state_in=d["state_in"], gk=d.get("gk"))
    o2 = torch.full((T, Nv, 128), float("nan"), dtype=d["q"].dtype, device=DEV)
    s2 = torch.full((B, Nv, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    gdr.chunk_prefill_noalloc(*args, state_in=d["state_in"], out=o2, state_out=s2, gk=d.get("gk"))
    torch.cuda.synchronize()
    return o1.cpu(), s1.cpu(), o2.cpu(), s2.cpu()


@pytest.mark.parametrize("gk", [None, "strong"])
def test_noalloc_prefill_matches_workspace_prefill_twice(gk):
    cases = [workloads.prefill_inputs(70, [1000, 129, 300], Nqk=4, Nv=8, act="bf16", gk=gk),
             workloads.prefill_inputs(71, [200, 77], Nqk=2, Nv=4, act="bf16", gk=gk)]
    for n, inp in enumerate(cases):
        print(f"[noalloc] call {n}: lens {inp['cu_seqlens'].tolist()} Nv={inp['Nv']} gk={gk}", flush=True)
        o1, s1, o2, s2 = _both(inp)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "out differs from gdr_chunk_prefill"
        assert torch.equal(s1, s2), "state differs from gdr_chunk_prefill"
        o_ref, s_ref = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["state_in"],
                                      inp["cu_seqlens"], inp["scale"], gk=inp.get("gk"))
        assert_out_close(o2, o_ref, True, f"noalloc call {n} out")
        assert_state_close(s2, s_ref, f"noalloc call {n} state")


@pytest.mark.parametrize("case", ["two_level", "many_sequences"])
def test_noalloc_prefill_other_paths(case):
    """The scratch array also carries the two-level scan's segment maps and
    start states (few long streams), and the chunk map built by its own
    launch (more than 168 sequences, no initial state)."""
    if case == "two_level":
        inp = workloads.prefill_inputs(72, [16000, 4000], Nqk=1, Nv=2, act="bf16")
    else:
        lens = [int(x) for x in torch.randint(0, 90, (200,), generator=torch.Generator().manual_seed(73))]
        inp = workloads.prefill_inputs(74, lens, Nqk=1, Nv=2, act="bf16", init_state="zeros")
    print(f"[noalloc] {case}: T={inp['T']} B={inp['B']}", flush=True)
    o1, s1, o2, s2 = _both(inp)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "out differs from gdr_chunk_prefill"
    assert torch.equal(s1, s2), "state differs from gdr_chunk_prefill"


def test_noalloc_prefill_rejects_a_workload_beyond_its_scratch():
    inp = workloads.config_inputs(2)
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    with pytest.raises(RuntimeError, match="scratch"):
        gdr.chunk_prefill_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["scale"],
                                  state_in=d["state_in"])

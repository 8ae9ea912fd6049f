"""GPU parity of gdr_recurrent_decode against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as gdr
import oracle
import workloads
from parity import assert_out_close, assert_state_close, out_kind, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_gpu(inp, pool=None, rule="gated_delta"):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    pool_dev = (inp["pool"] if pool is None else pool).clone().to(DEV)
    g, gk, beta = d["g"], d["gk"], d["beta"]
    if rule in ("delta", "linear"):   # NULL where the rule ignores the input
        g = gk = None
    if rule in ("gated", "linear"):
        beta = None
    out, _ = gdr.recurrent_decode(d["q"], d["k"], d["v"], g, gk, beta, pool_dev,
                                  d["idx"], d["lens"], d["scale"], num_accepted_tokens=d.get("nacc"), rule=rule)
    torch.cuda.synchronize()
    return out.cpu(), pool_dev.cpu()


def run_oracle(inp, pool=None, rule="gated_delta"):
    pool = inp["pool"] if pool is None else pool
    rnd = {torch.bfloat16: "bf16", torch.float16: "fp16"}.get(pool.dtype)
    return oracle.decode(inp["q"], inp["k"], inp["v"], inp["g"], inp["gk"], inp["beta"], pool,
                         inp["idx"], inp["lens"], inp["scale"], round_state=rnd,
                         num_accepted=inp.get("nacc"), rule=rule)


def written_slots(inp):
    idx = inp["idx"].numpy().reshape(inp["B"], inp["S"])
    lens = inp["lens"].numpy()
    return sorted({int(idx[b, t]) for b in range(inp["B"]) for t in range(lens[b])})


def check_parity(inp, tag, rule="gated_delta"):
    print(f"[decode parity] {tag}", flush=True)
    out, pool = run_gpu(inp, rule=rule)
    out_ref, pool_ref = run_oracle(inp, rule=rule)
    lens = inp["lens"].numpy()
    valid = np.zeros(out.shape, bool)
    for b in range(inp["B"]):
        valid[b, :, :lens[b]] = True
    exc, lit = assert_out_close(to_f64(out)[valid], out_ref[valid], out_kind(out), f"{tag} out")
    # padded token rows are zeros
    assert not torch.any(out[torch.from_numpy(~valid)] != 0)
    ws = written_slots(inp)
    es = assert_state_close(to_f64(pool)[ws], pool_ref[ws], f"{tag} state")
    # every slot no token writes keeps its exact bits
    untouched = sorted(set(range(inp["num_slots"])) - set(ws))
    two_byte = pool.element_size() == 2
    assert torch.equal(pool[untouched].view(torch.int16) if two_byte else pool[untouched],
                       inp["pool"][untouched].view(torch.int16) if two_byte else inp["pool"][untouched])
    print(f"    out err beyond rounding {exc:.2e} (literal {lit:.2e}) x RMS; state relFro {es:.2e}", flush=True)


def test_decode_b256_nk16_nv32_dk128_bf16_pool():
    check_parity(workloads.config_inputs(3), "B=256 Nk=16 Nv=32 Dk=Dv=128 bf16 pool")


def test_decode_b64_s4_gk_dk64_dv512_two_slot_routing():
    check_parity(workloads.config_inputs(4), "B=64 S=4 gk Dk=64 Dv=512 two-slot routing")


@pytest.mark.parametrize("Dk,Dv", [(64, 64), (128, 64), (64, 256), (128, 512)])
def test_decode_shapes_fp32_pool(Dk, Dv):
    inp = workloads.decode_inputs(30 + Dk + Dv, B=5, S=3, Nk=2, Nv=4, Dk=Dk, Dv=Dv, num_slots=12,
                                  with_gk=True, lens="random", routing="two_slots", state="fp32")
    check_parity(inp, f"Dk={Dk} Dv={Dv} fp32 pool")


def test_decode_fp32_activations_bf16_pool():
    inp = workloads.decode_inputs(41, B=6, S=2, Nk=1, Nv=3, Dk=128, Dv=128, num_slots=13,
                                  lens="random", routing="two_slots", act="fp32")
    check_parity(inp, "fp32 act")


def test_decode_unit_key_read_back_is_bit_exact():
    """k = q = e_i, beta = 1, g = 0, zero slot, scale 1: out == v and row i == v, exactly."""
    B, Nv, Dk, Dv = 4, 2, 128, 128
    inp = workloads.decode_inputs(42, B=B, S=1, Nk=1, Nv=Nv, Dk=Dk, Dv=Dv, num_slots=8)
    q = torch.zeros(B, 1, 1, Dk, dtype=torch.bfloat16)
    rows = [3, 0, 127, 64]
    for b, i in enumerate(rows):
        q[b, 0, 0, i] = 1.0
    inp.update(q=q, k=q.clone(), beta=torch.ones(B, Nv, 1, dtype=torch.bfloat16),
               g=torch.zeros(B, Nv, 1), scale=1.0, pool=torch.zeros(8, Nv, Dk, Dv, dtype=torch.bfloat16))
    out, pool = run_gpu(inp)
    idx = inp["idx"].numpy()
    for b, i in enumerate(rows):
        for h in range(Nv):
            assert torch.equal(out[b, h, 0], inp["v"][b, h, 0])
            slab = pool[idx[b], h]
            assert torch.equal(slab[i], inp["v"][b, h, 0])
            assert not torch.any(torch.cat([slab[:i], slab[i + 1:]]) != 0)


def test_decode_beta_zero_gate_zero_keeps_pool_bits():
    inp = workloads.decode_inputs(43, B=8, S=2, Nk=2, Nv=4, Dk=128, Dv=128, num_slots=20)
    inp.update(beta=torch.zeros_like(inp["beta"]), g=torch.zeros_like(inp["g"]))
    out, pool = run_gpu(inp)
    assert torch.equal(pool.view(torch.int16), inp["pool"].view(torch.int16))
    out_ref, _ = run_oracle(inp)
    assert_out_close(out, out_ref, True, "beta=0 out")


def test_decode_repeated_slots_last_write_wins_and_len0_rows():
    inp = workloads.decode_inputs(44, B=3, S=4, Nk=1, Nv=2, Dk=64, Dv=128, num_slots=10, with_gk=True)
    idx = torch.tensor([[5, 1, 5, 2], [0, 0, 7, 7], [3, 4, 6, 8]], dtype=torch.int32).reshape(-1)
    lens = torch.tensor([4, 3, 0], dtype=torch.int32)
    inp.update(idx=idx, lens=lens)
    check_parity(inp, "repeated slots / len 0")


def test_decode_out_of_range_indices_stay_in_bounds():
    """A token naming a slot outside the pool stores nothing; a chain whose
    first slot is outside starts from zeros.  No other slot changes."""
    inp = workloads.decode_inputs(45, B=2, S=2, Nk=1, Nv=1, Dk=64, Dv=64, num_slots=4, state="fp32")
    inp.update(idx=torch.tensor([9, 1, 2, -3], dtype=torch.int32), lens=torch.tensor([2, 2], dtype=torch.int32))
    out, pool = run_gpu(inp)
    assert torch.equal(pool[0], inp["pool"][0]) and torch.equal(pool[3], inp["pool"][3])
    ref = dict(inp)
    ref_pool = inp["pool"].clone()
    ref_pool[0] = 0   # row 0 starts from zeros: emulate with a zero slot 0 and index 0
    ref.update(pool=ref_pool, idx=torch.tensor([0, 1, 2, 2], dtype=torch.int32))
    out_ref, pool_ref = run_oracle(ref)
    assert_out_close(out, out_ref, True, "oob out")
    assert_state_close(pool[1], pool_ref[1], "oob state slot 1", tol=1e-5)


def test_decode_is_deterministic():
    inp = workloads.config_inputs(4)
    o1, p1 = run_gpu(inp)
    o2, p2 = run_gpu(inp)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(p1.view(torch.int16), p2.view(torch.int16))


@pytest.mark.parametrize("Dk,Dv,with_gk", [(128, 128, False), (64, 512, True)])
def test_decode_speculative_rounds_resume_after_accepted_tokens(Dk, Dv, with_gk):
    """Speculative decoding: call 1 drafts S = 4 tokens per row, leaving the
    state after each in a slot of its own; call 2 (same index positions,
    num_accepted_tokens ~ U{1..4}) resumes each row from the state after its
    last accepted draft.  Both calls run on the GPU and in the oracle."""
    B, S, slots = 24, 4, 100
    r1 = workloads.decode_inputs(70 + Dv, B=B, S=S, Nk=2, Nv=4, Dk=Dk, Dv=Dv, num_slots=slots,
                                 with_gk=with_gk, routing="per_token")
    r2 = workloads.decode_inputs(71 + Dv, B=B, S=S, Nk=2, Nv=4, Dk=Dk, Dv=Dv, num_slots=slots,
                                 with_gk=with_gk, lens="random", routing="per_token", accepted=True)
    r2["idx"] = r1["idx"].clone()
    print(f"[decode parity] speculative rounds Dk={Dk} Dv={Dv} nacc={r2['nacc'].tolist()[:8]}...", flush=True)
    _, pool1 = run_gpu(r1)
    out2, pool2 = run_gpu(r2, pool=pool1)
    _, pool1_ref = run_oracle(r1)
    out2_ref, pool2_ref = run_oracle(r2, pool=torch.from_numpy(pool1_ref).to(torch.bfloat16))
    lens = r2["lens"].numpy()
    valid = np.zeros(out2.shape, bool)
    for b in range(B):
        valid[b, :, :lens[b]] = True
    exc, lit = assert_out_close(to_f64(out2)[valid], out2_ref[valid], True, "speculative out")
    ws = written_slots(r2)
    es = assert_state_close(to_f64(pool2)[ws], pool2_ref[ws], "speculative state")
    print(f"    out err beyond rounding {exc:.2e} (literal {lit:.2e}) x RMS; state relFro {es:.2e}", flush=True)


@pytest.mark.parametrize("rule", ["delta", "gated", "linear"])
def test_decode_update_rules(rule):
    """Update rules ("LinearAttention" page, update_rule) with NULL g, gk or
    beta where the rule ignores them."""
    inp = workloads.decode_inputs(90, B=12, S=3, Nk=2, Nv=4, Dk=128, Dv=128, num_slots=30, with_gk=True,
                                  lens="random", routing="two_slots")
    check_parity(inp, f"rule {rule}", rule=rule)


@pytest.mark.parametrize("act,state", [("fp16", "fp16"), ("fp16", "fp32"), ("bf16", "fp16")])
def test_decode_fp16_activations_and_state(act, state):
    """IEEE half activations and/or state pool (the LinearAttention page
    allows float16 for both)."""
    inp = workloads.decode_inputs(95, B=10, S=3, Nk=2, Nv=4, Dk=128, Dv=128, num_slots=25, with_gk=True,
                                  lens="random", routing="two_slots", act=act, state=state)
    check_parity(inp, f"act {act} state {state}")


# One token per row (S = 1, the ordinary decode step) runs a kernel of its own
# that keeps each slab packed in its 16-bit form; its variants:
@pytest.mark.parametrize("rule,state,Dk,Dv", [("gated_delta", "fp16", 128, 128), ("delta", "bf16", 128, 128),
                                              ("gated", "bf16", 64, 512), ("linear", "bf16", 64, 64),
                                              ("gated_delta", "bf16", 128, 256)])
def test_decode_one_token_per_row(rule, state, Dk, Dv):
    inp = workloads.decode_inputs(100 + Dk + Dv, B=9, S=1, Nk=2, Nv=4, Dk=Dk, Dv=Dv, num_slots=20,
                                  with_gk=True, state=state)
    # rows 2 and 7 have no token: not read, not written, out rows zero
    lens = inp["lens"].clone()
    idx = inp["idx"].clone()
    lens[2] = 0
    lens[7] = 0
    idx[2] = -1
    idx[7] = -1
    inp.update(lens=lens, idx=idx)
    check_parity(inp, f"S=1 rule {rule} {state} pool Dk={Dk} Dv={Dv}", rule=rule)


def test_decode_one_token_rows_in_groups_of_eight_with_a_short_last_group():
    """S = 1 with a 16-bit pool: the kernel takes its rows in groups of eight
    (one row per XCD) and each head's slab in two 64-column halves.  1001
    rows are 125 whole groups and a last group of one; every row's slot is a
    distinct random one of 1200, and a few rows carry no token."""
    inp = workloads.decode_inputs(121, B=1001, S=1, Nk=2, Nv=4, Dk=128, Dv=128, num_slots=1200)
    lens = inp["lens"].clone()
    idx = inp["idx"].clone()
    for b in (0, 7, 8, 999, 1000):
        lens[b] = 0
        idx[b] = -1
    inp.update(lens=lens, idx=idx)
    check_parity(inp, "S=1 bf16 pool B=1001 Nv=4 Dk=Dv=128")


def test_decode_one_token_out_of_range_slot():
    """S = 1: a row whose slot lies outside the pool starts from zeros and
    stores nothing."""
    inp = workloads.decode_inputs(120, B=3, S=1, Nk=1, Nv=2, Dk=128, Dv=128, num_slots=4)
    inp.update(idx=torch.tensor([7, 1, -2], dtype=torch.int32))
    out, pool = run_gpu(inp)
    assert torch.equal(pool[[0, 2, 3]].view(torch.int16), inp["pool"][[0, 2, 3]].view(torch.int16))
    ref_pool = inp["pool"].clone()
    ref_pool[0] = 0
    ref_pool[2] = 0
    ref = dict(inp, pool=ref_pool, idx=torch.tensor([0, 1, 2], dtype=torch.int32))
    out_ref, pool_ref = run_oracle(ref)
    assert_out_close(out, out_ref, True, "S=1 oob out")
    assert_state_close(to_f64(pool[1]), pool_ref[1], "S=1 oob state slot 1")


def _random_decode_case(seed):
    """A seeded draw of the decode's shape and option space: 1-16 rows of
    1-8 tokens, GQA groups of 1 or 2, both key sizes and every value size,
    every activation and pool dtype and rule, the per-key gate with the
    rules that decay, every slot routing, ragged lengths and accepted-token
    counts; the pool kept under 8 M elements so that the fp64 oracle stays
    quick."""
    rng = np.random.default_rng(3000 + seed)
    S = 1 if rng.random() < 0.3 else int(rng.integers(2, 9))   # one token per row has its own kernel
    Nk = int(rng.choice([1, 2, 4]))
    Nv = Nk * int(rng.choice([1, 2]))
    Dk = int(rng.choice([64, 128]))
    Dv = int(rng.choice([64, 128, 256, 512]))
    act = str(rng.choice(["bf16", "fp16", "fp32"]))
    state = str(rng.choice(["bf16", "fp16", "fp32"]))
    rule = str(rng.choice(["gated_delta", "gated_delta", "delta", "gated", "linear"]))
    with_gk = rule in ("gated_delta", "gated") and bool(rng.random() < 0.5)
    lens = str(rng.choice(["full", "random"]))
    routing = str(rng.choice(["one_slot", "two_slots", "per_token"]))
    accepted = routing == "per_token" and bool(rng.random() < 0.5)
    B = int(rng.integers(1, 17))
    per_row = {"one_slot": 1, "two_slots": 2, "per_token": S}[routing]
    while B > 1 and (B * per_row + 4) * Nv * Dk * Dv > 8 << 20:
        B -= 1
    num_slots = B * per_row + int(rng.integers(0, 5))
    return dict(B=B, S=S, Nk=Nk, Nv=Nv, Dk=Dk, Dv=Dv, num_slots=num_slots, with_gk=with_gk, lens=lens,
                routing=routing, act=act, state=state, accepted=accepted), rule


@pytest.mark.parametrize("seed", range(16))
def test_decode_random_cases(seed):
    kw, rule = _random_decode_case(seed)
    inp = workloads.decode_inputs(4000 + seed, **kw)
    check_parity(inp, f"random case {seed}: {kw} rule {rule}", rule=rule)

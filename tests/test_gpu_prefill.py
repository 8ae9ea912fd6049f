"""GPU parity of gdr_chunk_prefill against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_chunk_amd as gdr
import oracle
import workloads
from parity import assert_out_close, assert_state_close, out_kind, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_gpu(inp, state_in="from_inputs", rule="gated_delta", drop_unused=True):
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    s_in = d["state_in"] if isinstance(state_in, str) else (None if state_in is None else state_in.to(DEV))
    g, beta = d["g"], d["beta"]
    if drop_unused:   # the rules without a gate / delta term take NULL there
        g = None if rule in ("delta", "linear") else g
        beta = None if rule in ("gated", "linear") else beta
    out, st = gdr.chunk_prefill(d["q"], d["k"], d["v"], g, beta, d["cu_seqlens"], d["scale"],
                                state_in=s_in, rule=rule, gk=d.get("gk"))
    torch.cuda.synchronize()
    return out.cpu(), st.cpu()


def run_oracle(inp, rule="gated_delta"):
    return oracle.prefill(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["state_in"],
                          inp["cu_seqlens"], inp["scale"], rule=rule, gk=inp.get("gk"))


def check_parity(inp, tag, rule="gated_delta"):
    print(f"[prefill parity] {tag}", flush=True)
    out, st = run_gpu(inp, rule=rule)
    out_ref, st_ref = run_oracle(inp, rule=rule)
    exc, lit = assert_out_close(out, out_ref, out_kind(out), f"{tag} out")
    es = assert_state_close(st, st_ref, f"{tag} state")
    print(f"    out err beyond rounding {exc:.2e} (literal {lit:.2e}) x RMS; state relFro {es:.2e}", flush=True)
    return out, st


def test_prefill_t256_nqk2_nv4_fp32():
    check_parity(workloads.config_inputs(1), "T=256 Nqk=2 Nv=4 fp32")


@pytest.mark.parametrize("act", ["bf16", "fp32"])
def test_prefill_ragged_varlen_small(act):
    lens = [1, 127, 128, 129, 300, 0, 77]
    inp = workloads.prefill_inputs(50, lens, Nqk=2, Nv=4, act=act)
    check_parity(inp, f"ragged varlen {lens} {act}")


def test_prefill_gqa_group_of_four():
    inp = workloads.prefill_inputs(51, [260, 45], Nqk=1, Nv=4, act="bf16")
    check_parity(inp, "Nqk=1 Nv=4")


def test_prefill_varlen_b4_t8192_nqk16_nv32_bf16():
    check_parity(workloads.config_inputs(2), "B=4 T=8192 Nqk=16 Nv=32 bf16")


def test_prefill_long_context_t131072_all_heads():
    """Full-size long-context workload (B=1, T=131072, Nqk=16, Nv=32): every
    value head over all 131072 tokens against the oracle."""
    check_parity(workloads.config_inputs(5), "T=131072 Nqk=16 Nv=32 bf16, all heads")


def test_prefill_element_offsets_past_2_31():
    """Token offsets past 2^31 elements of v and out ([T, 32, 128] at
    T = 540672) and workspace tiles past 2^31 elements: two sequences,
    532480 + 8192 tokens.  The oracle checks the second sequence on every
    value head (its tokens all lie past element 2^31) and the first sequence
    on its first and last value heads over all its tokens."""
    lens = [532480, 8192]
    inp = workloads.large_prefill_inputs(12, lens, Nqk=16, Nv=32)
    assert inp["T"] * inp["Nv"] * 128 > 2 ** 31 and lens[0] * inp["Nv"] * 128 > 2 ** 31
    print(f"[prefill parity] offsets past 2^31: lens {lens}", flush=True)
    out, st = run_gpu(inp)
    t1 = lens[0]
    second = dict(inp, q=inp["q"][t1:], k=inp["k"][t1:], v=inp["v"][t1:], g=inp["g"][t1:],
                  beta=inp["beta"][t1:], state_in=inp["state_in"][1:],
                  cu_seqlens=torch.tensor([0, lens[1]], dtype=torch.int32))
    o_ref, s_ref = run_oracle(second)
    exc, lit = assert_out_close(out[t1:], o_ref, True, "second sequence out")
    es = assert_state_close(st[1:], s_ref, "second sequence state")
    print(f"    second sequence, all heads: out {exc:.2e} (literal {lit:.2e}); state {es:.2e}", flush=True)
    G = inp["Nv"] // inp["Nqk"]
    for h in (0, inp["Nv"] - 1):
        hq = h // G
        sub = dict(q=inp["q"][:t1, hq:hq + 1], k=inp["k"][:t1, hq:hq + 1], v=inp["v"][:t1, h:h + 1],
                   g=inp["g"][:t1, h:h + 1], beta=inp["beta"][:t1, h:h + 1],
                   state_in=inp["state_in"][:1, h:h + 1], cu_seqlens=torch.tensor([0, t1], dtype=torch.int32),
                   scale=inp["scale"])
        o_ref, s_ref = run_oracle(sub)
        exc, lit = assert_out_close(out[:t1, h:h + 1], o_ref, True, f"first sequence head {h} out")
        es = assert_state_close(st[:1, h:h + 1], s_ref, f"first sequence head {h} state")
        print(f"    first sequence head {h}: out {exc:.2e} (literal {lit:.2e}); state {es:.2e}", flush=True)


def test_prefill_strong_gate_without_per_key_gate():
    """The decode page's gate range g = -U(0.01, 1.01) in the prefill: the
    chunk-local decays reach e^-128, so k^ beta e^{g_cum} underflows fp16 in
    the stored w tile and most intra-chunk terms vanish."""
    inp = workloads.prefill_inputs(63, [1000, 4096, 300, 2796], Nqk=16, Nv=32, act="bf16", g_range=(0.01, 1.01))
    check_parity(inp, "T=8192 varlen, g = -U(0.01, 1.01)")


def test_prefill_repeated_keys_beta_one():
    """Three keys written in turn with beta = 1, so every write replaces the
    value stored under its key: the strictly lower L then holds entries near
    one (exactly one without decay), the largest the block substitution for w
    and u meets ("Qwen3Next Samples", Matrix Inversion)."""
    inp = workloads.prefill_inputs(90, [300, 130, 1], Nqk=1, Nv=2, act="bf16", g_range=(1e-6, 1e-5))
    T = inp["k"].shape[0]
    k = inp["k"][:3].clone()[torch.arange(T) % 3]
    inp = dict(inp, k=k, beta=torch.ones_like(inp["beta"]))
    check_parity(inp, "three repeated keys, beta = 1")


def test_prefill_large_values_inside_fp16_range():
    """v and the initial state scaled by 512 (bf16, entries up to a few
    thousand): the fp16 intermediates (u, v_new, the chunk-start states) hold
    them, and the errors scale with the values."""
    inp = workloads.prefill_inputs(91, [700, 300], Nqk=2, Nv=4, act="bf16")
    inp = dict(inp, v=(inp["v"].float() * 512).to(torch.bfloat16), state_in=inp["state_in"] * 512)
    check_parity(inp, "v and state x 512")


@pytest.mark.parametrize("rule,g_range", [("linear", (0.001, 0.1)), ("gated_delta", (1e-6, 1e-5))])
def test_prefill_long_sequence_without_forgetting(rule, g_range):
    """32768 tokens with no decay (the linear rule, whose state only grows)
    and with a gate of about 1e-5 per token: the state carried across 256
    chunks stays large, which the fp16 copy of S inside the scan must
    hold."""
    inp = workloads.prefill_inputs(64, [32768], Nqk=1, Nv=2, act="bf16", g_range=g_range)
    check_parity(inp, f"T=32768 rule {rule} g=-U{g_range}", rule=rule)


def test_prefill_empty_sequences_pass_state_through():
    inp = workloads.prefill_inputs(52, [0, 130, 0], Nqk=2, Nv=2, act="bf16")
    out, st = run_gpu(inp)
    assert torch.equal(st[0], inp["state_in"][0]) and torch.equal(st[2], inp["state_in"][2])
    out_ref, st_ref = run_oracle(inp)
    assert_out_close(out, out_ref, True)
    assert_state_close(st[1], st_ref[1])


def test_prefill_all_empty_t0():
    inp = workloads.prefill_inputs(53, [0, 0], Nqk=1, Nv=2, act="bf16")
    out, st = run_gpu(inp)
    assert out.shape[0] == 0 and torch.equal(st, inp["state_in"])


def test_prefill_zero_initial_state_default():
    inp = workloads.prefill_inputs(54, [200], Nqk=1, Nv=2, act="bf16", init_state="zeros")
    check_parity(inp, "state_in NULL")


def test_prefill_beta_zero_gate_zero_keeps_state_bits():
    inp = workloads.prefill_inputs(55, [300, 20], Nqk=2, Nv=4, act="bf16")
    inp.update(beta=torch.zeros_like(inp["beta"]), g=torch.zeros_like(inp["g"]))
    out, st = run_gpu(inp)
    assert torch.equal(st, inp["state_in"])
    out_ref, _ = run_oracle(inp)
    assert_out_close(out, out_ref, True, "beta=0 out")


def test_prefill_split_and_resume_matches_one_call():
    inp = workloads.prefill_inputs(56, [700], Nqk=2, Nv=4, act="bf16")
    out, st = run_gpu(inp)
    t1 = 333
    a = dict(inp, q=inp["q"][:t1], k=inp["k"][:t1], v=inp["v"][:t1], g=inp["g"][:t1], beta=inp["beta"][:t1],
             cu_seqlens=torch.tensor([0, t1], dtype=torch.int32))
    oa, sa = run_gpu(a)
    b = dict(inp, q=inp["q"][t1:], k=inp["k"][t1:], v=inp["v"][t1:], g=inp["g"][t1:], beta=inp["beta"][t1:],
             cu_seqlens=torch.tensor([0, 700 - t1], dtype=torch.int32), state_in=sa)
    ob, sb = run_gpu(b)
    out_ref, st_ref = run_oracle(inp)
    assert_out_close(torch.cat([oa, ob]), out_ref, True, "resumed out")
    assert_state_close(sb, st_ref, "resumed state")


def test_prefill_state_out_may_alias_state_in():
    inp = workloads.prefill_inputs(57, [150, 260], Nqk=2, Nv=4, act="bf16")
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    s = d["state_in"].clone()
    gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["scale"], state_in=s,
                      state_out=s)
    torch.cuda.synchronize()
    _, st_ref = run_oracle(inp)
    assert_state_close(s.cpu(), st_ref, "aliased state")


def test_prefill_is_deterministic():
    inp = workloads.prefill_inputs(58, [1000, 300], Nqk=2, Nv=4, act="bf16")
    o1, s1 = run_gpu(inp)
    o2, s2 = run_gpu(inp)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(s1, s2)


@pytest.mark.parametrize("B,Nqk,Nv", [(1, 1, 4), (2, 16, 32), (4, 8, 32), (8, 16, 32)])
def test_prefill_every_scan_slice_width(B, Nqk, Nv):
    """B * Nv value-head streams pick the scan's column split (16, 32, 64 or
    128 state columns per workgroup); each split is checked."""
    lens = [150 + 37 * i for i in range(B)]
    inp = workloads.prefill_inputs(60 + B, lens, Nqk=Nqk, Nv=Nv, act="bf16")
    check_parity(inp, f"B={B} Nv={Nv} ({B * Nv} streams)")


@pytest.mark.parametrize("rule", ["delta", "gated", "linear"])
def test_prefill_update_rules(rule):
    """Update rules ("LinearAttention" page, update_rule) against the oracle,
    with NULL gates / beta where the rule ignores them; passing them instead
    must not change a bit."""
    inp = workloads.prefill_inputs(80, [300, 129, 5, 0, 260], Nqk=2, Nv=4, act="bf16")
    print(f"[prefill parity] rule {rule}", flush=True)
    out, st = run_gpu(inp, rule=rule)
    out_ref, st_ref = run_oracle(inp, rule=rule)
    exc, lit = assert_out_close(out, out_ref, True, f"{rule} out")
    es = assert_state_close(st, st_ref, f"{rule} state")
    print(f"    out err beyond rounding {exc:.2e} (literal {lit:.2e}) x RMS; state relFro {es:.2e}", flush=True)
    out2, st2 = run_gpu(inp, rule=rule, drop_unused=False)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16)) and torch.equal(st, st2)


def test_prefill_fp16_activations():
    """IEEE half activations (the LinearAttention page allows float16)."""
    inp = workloads.prefill_inputs(85, [300, 129, 77], Nqk=2, Nv=4, act="fp16")
    check_parity(inp, "fp16 activations")


@pytest.mark.parametrize("Nqk,Nv", [(2, 16), (4, 4), (1, 8)])
def test_prefill_gqa_group_sizes(Nqk, Nv):
    """Group sizes G = Nv / Nqk of 8, 1 and 8 with one qk head: the
    XCD-grouped launch grids round up to multiples of 8 G."""
    inp = workloads.prefill_inputs(90 + Nv, [333, 129, 64, 1], Nqk=Nqk, Nv=Nv, act="bf16")
    check_parity(inp, f"Nqk={Nqk} Nv={Nv}")


@pytest.mark.parametrize("gk", [None, "strong"])
def test_prefill_many_short_sequences(gk):
    """300 sequences (more than one 256-wide pass of the chunk-map prefix),
    lengths 0..200 including empty ones; with gk, 600 one- or two-chunk
    streams through the scan that forms the output itself."""
    rng = np.random.default_rng(99)
    lens = rng.integers(0, 201, 300).tolist()
    lens[5] = 0
    lens[299] = 0
    inp = workloads.prefill_inputs(98, lens, Nqk=1, Nv=2, act="bf16", gk=gk)
    check_parity(inp, f"B=300 T={sum(lens)} gk={gk}")


def test_prefill_chunk_map_built_in_the_intra_kernel_at_its_limit():
    """Up to 168 sequences the intra kernel builds the chunk map itself; with
    more, a separate launch builds it.  168 sequences (empty ones at both
    ends, chunk-edge lengths) are checked against the oracle; appending an
    empty 169th sequence switches to the separate launch and must leave
    every output bit and the first 168 states unchanged, the new sequence's
    state passed through."""
    rng = np.random.default_rng(124)
    lens = rng.integers(0, 300, 168).tolist()
    lens[0] = lens[167] = lens[90] = 0
    lens[7], lens[8], lens[9] = 128, 129, 256
    inp = workloads.prefill_inputs(125, lens, Nqk=1, Nv=2, act="bf16")
    out, st = check_parity(inp, f"B=168 T={sum(lens)}")
    extra = torch.randn((1, 2, 128, 128), generator=torch.Generator().manual_seed(126)) * 0.02
    inp2 = dict(inp, B=169, cu_seqlens=torch.cat([inp["cu_seqlens"], inp["cu_seqlens"][-1:]]),
                state_in=torch.cat([inp["state_in"], extra]))
    print("[prefill] B=169 (separate chunk-map launch)", flush=True)
    out2, st2 = run_gpu(inp2)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(st, st2[:168]) and torch.equal(st2[168], extra[0])


# Two-level scan: with few (sequence, value head) streams and long sequences
# the library cuts each sequence into segments, finds every segment's affine
# map (S_end = M S_start + B) first, then each segment's start state, then
# scans the segments side by side (the workspace size shows the extra maps;
# tests/test_abi.py checks that these shapes select it).
def _weak_forgetting(inp):
    """Gates near zero and small beta, so that a segment's map M stays far
    from zero and an error in it would show in the outputs."""
    dt = inp["beta"].dtype
    inp = dict(inp)
    inp["g"] = inp["g"] * 0.01
    inp["beta"] = (inp["beta"].float() * 0.1).to(dt)
    return inp


def test_prefill_two_level_scan_one_long_sequence():
    inp = workloads.prefill_inputs(60, [32768], Nqk=1, Nv=2, act="bf16")
    check_parity(inp, "two-level T=32768 Nqk=1 Nv=2 bf16")


def test_prefill_two_level_scan_mixed_lengths_weak_forgetting():
    inp = _weak_forgetting(workloads.prefill_inputs(61, [20000, 0, 5003], Nqk=1, Nv=4, act="bf16"))
    check_parity(inp, "two-level lens [20000, 0, 5003] Nqk=1 Nv=4 bf16, weak forgetting")


def test_prefill_two_level_scan_fp32_weak_forgetting():
    inp = _weak_forgetting(workloads.prefill_inputs(62, [9000], Nqk=1, Nv=1, act="fp32"))
    check_parity(inp, "two-level T=9000 Nqk=1 Nv=1 fp32, weak forgetting")


@pytest.mark.parametrize("rule", ["gated_delta", "delta"])
def test_prefill_two_level_scan_zero_initial_state(rule):
    """Two-level scan without an initial state: the first segment of each
    stream starts from the zeros the combine writes; with and without the
    gate (the delta rule's segment maps carry no decay)."""
    inp = workloads.prefill_inputs(66, [16000, 700], Nqk=1, Nv=2, act="bf16", init_state="zeros")
    check_parity(inp, f"two-level lens [16000, 700] Nqk=1 Nv=2, no initial state, rule {rule}", rule=rule)


def test_prefill_two_level_scan_long_few_heads_all_heads():
    """Full-size few-head long-context workload (two-level scan): every value
    head over all 131072 tokens against the oracle."""
    check_parity(workloads.extra_inputs("long_few_heads"), "two-level T=131072 Nqk=1 Nv=4, all heads")


def test_prefill_two_level_scan_state_out_may_alias_state_in():
    """On the two-level path the last segment writes state_out in the same
    launch in which the first segment starts; with state_out aliasing
    state_in the result must not change."""
    inp = workloads.prefill_inputs(65, [20000, 3000], Nqk=1, Nv=2, act="bf16")
    d = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    s = d["state_in"].clone()
    out, _ = gdr.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["cu_seqlens"], d["scale"],
                               state_in=s, state_out=s)
    torch.cuda.synchronize()
    out_ref, st_ref = run_oracle(inp)
    assert_out_close(out.cpu(), out_ref, True, "two-level aliased out")
    assert_state_close(s.cpu(), st_ref, "two-level aliased state")


# Per-key gate gk [T, Nv, D]: the decay between tokens differs per key, so the
# intra-chunk products are formed per 16-token block pair (the library's
# per-key-gate path); "strong" is the decode page's example range, "weak"
# keeps the state alive across chunks so that the scan's per-row decay shows.
@pytest.mark.parametrize("act,strength", [("bf16", "strong"), ("bf16", "weak"), ("fp32", "weak"),
                                          ("fp16", "strong")])
def test_prefill_per_key_gate_ragged(act, strength):
    lens = [1, 127, 128, 129, 300, 0, 77]
    inp = workloads.prefill_inputs(80, lens, Nqk=2, Nv=4, act=act, gk=strength)
    check_parity(inp, f"gk {strength} ragged varlen {lens} {act}")


def test_prefill_per_key_gate_gated_rule():
    inp = workloads.prefill_inputs(81, [260, 45], Nqk=1, Nv=2, act="bf16", gk="weak")
    check_parity(inp, "gk weak, gated rule", rule="gated")


def test_prefill_per_key_gate_rules_without_decay_ignore_it():
    inp = workloads.prefill_inputs(82, [200, 77], Nqk=2, Nv=4, act="bf16", gk="strong")
    plain = dict(inp, gk=None)
    for rule in ("delta", "linear"):
        o1, s1 = run_gpu(inp, rule=rule)
        o2, s2 = run_gpu(plain, rule=rule)
        assert torch.equal(o1, o2) and torch.equal(s1, s2), rule


@pytest.mark.parametrize("name", ["varlen_gk", "varlen_gk_small"])
def test_prefill_per_key_gate_varlen_t8192(name):
    # the timed per-key-gate workloads, in full: the decode page's gk range
    # (mostly fp32 diagonal tiles) and a small gate (all fp16)
    check_parity(workloads.extra_inputs(name), workloads.EXTRA_NAMES[name])


@pytest.mark.parametrize("B,Nqk,Nv", [(2, 16, 32), (8, 16, 32), (16, 8, 32)])
def test_prefill_per_key_gate_every_scan_slice_width(B, Nqk, Nv):
    """With the per-key gate the one-level scan forms the output itself; its
    column split (16, 32 or 64 state columns per workgroup, 64 also standing
    in for a whole-row split) follows the B * Nv streams, and each is checked
    (16 by the ragged cases above)."""
    lens = [150 + 37 * i for i in range(B)]
    inp = workloads.prefill_inputs(86 + B, lens, Nqk=Nqk, Nv=Nv, act="bf16", gk="weak")
    check_parity(inp, f"gk weak B={B} Nv={Nv} ({B * Nv} streams)")


def test_prefill_per_key_gate_two_level_scan():
    inp = workloads.prefill_inputs(84, [20000], Nqk=1, Nv=2, act="bf16", gk="weak")
    check_parity(inp, "gk weak two-level T=20000 Nqk=1 Nv=2 bf16")



@pytest.mark.parametrize("strength", ["extreme", "reset"])
def test_prefill_per_key_gate_any_magnitude(strength):
    """Per-key gates far outside the decode page's example range: g + gk down
    to about -40 per token ("extreme"), and a reset gk = -1e4 on about one
    (token, head, key) in a hundred ("reset"), which wipes that key row of
    the state.  The diagonal 16-token blocks then need the element-by-element
    tier (and the others the fp32 and fp16 ones)."""
    lens = [1, 127, 128, 129, 300, 0, 77, 1000]
    inp = workloads.prefill_inputs(66, lens, Nqk=2, Nv=4, act="bf16", gk=strength)
    check_parity(inp, f"gk {strength} ragged varlen {lens}")


def test_prefill_per_key_gate_reset_t8192():
    inp = workloads.prefill_inputs(67, [1000, 4096, 300, 2796], Nqk=16, Nv=32, act="bf16", gk="reset")
    check_parity(inp, "gk reset T=8192 varlen Nqk=16 Nv=32")


def _random_case(seed):
    """A seeded draw of the prefill's shape and option space: 1-6 sequences
    whose lengths mix the chunk edges (0, 1, 127-129, 255-257) with random
    ones, GQA groups of 1, 2 or 4, every activation dtype and rule, the
    per-key gate in its ranges (with the rules that decay), with and without
    an initial state, gates from nearly none to strong."""
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 7))
    edges = [0, 1, 2, 63, 64, 127, 128, 129, 255, 256, 257]
    lens = [int(rng.choice(edges)) if rng.random() < 0.5 else int(rng.integers(1, 700)) for _ in range(B)]
    if sum(lens) == 0:
        lens[0] = 1
    Nqk = int(rng.choice([1, 2, 4]))
    Nv = Nqk * int(rng.choice([1, 2, 4]))
    act = str(rng.choice(["bf16", "fp16", "fp32"]))
    rule = str(rng.choice(["gated_delta", "gated_delta", "delta", "gated", "linear"]))
    gk = None if rule in ("delta", "linear") else [None, None, "weak", "strong", "reset"][int(rng.integers(0, 5))]
    init = str(rng.choice(["randn", "zeros"]))
    g_lo = float(rng.choice([1e-6, 0.001, 0.01]))
    g_range = (g_lo, g_lo * float(rng.choice([10.0, 100.0])))
    return lens, Nqk, Nv, act, rule, gk, init, g_range


@pytest.mark.parametrize("seed", range(16))
def test_prefill_random_cases(seed):
    lens, Nqk, Nv, act, rule, gk, init, g_range = _random_case(seed)
    inp = workloads.prefill_inputs(2000 + seed, lens, Nqk=Nqk, Nv=Nv, act=act, init_state=init, gk=gk,
                                   g_range=g_range)
    check_parity(inp, f"random case {seed}: lens {lens} Nqk={Nqk} Nv={Nv} {act} rule {rule} gk {gk} "
                      f"init {init} g=-U{g_range}", rule=rule)

"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test ties the oracle to what the pages and the mathematics fix:
  * brute-force agreement of the per-token recurrence (decode page,
    algorithm flow) with an independent statement of the chunked formulas
    ("Qwen3Next Samples" page, Mathematical Formulas), for several chunk
    lengths -- this pins signs, masks and gate indices of both, and the tests
    show that each alternative reading of the garbled passages disagrees;
  * a hand-derived worked example (tests/golden/decode_hand_2x2.json);
  * closed forms: unit-key read-back, beta = 0 identity, pure decay,
    orthonormal keys = causal linear attention, per-key reset, the eps
    inside the L2 norm;
  * invariants: GQA = replicated heads, varlen packing = separate calls,
    split-and-resume = one call, multi-token decode = chained single tokens,
    decode = prefill on unit-norm inputs, linearity in scale.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
from oracle import chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_prefill(rng, lens, Nqk, Nv, Dk, Dv, with_state=True):
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q = rng.standard_normal((T, Nqk, Dk))
    k = rng.standard_normal((T, Nqk, Dk))
    v = rng.standard_normal((T, Nv, Dv))
    g = -rng.uniform(0.01, 0.6, (T, Nv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, Nv))))
    s0 = rng.standard_normal((len(lens), Nv, Dk, Dv)) * 0.5 if with_state else None
    return q, k, v, g, beta, s0, cu


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("L", [1, 2, 3, 4, 8, 128])
def test_chunked_formulas_equal_recurrence(L):
    rng = np.random.default_rng(100 + L)
    for trial in range(6):
        nseq = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(0, 23, nseq)]
        Nqk = int(rng.integers(1, 3))
        Nv = Nqk * int(rng.integers(1, 3))
        Dk, Dv = int(rng.integers(2, 6)), int(rng.integers(2, 6))
        args = rand_prefill(rng, lens, Nqk, Nv, Dk, Dv, with_state=trial % 2 == 0)
        scale = float(rng.uniform(0.2, 1.5))
        o_ref, s_ref = oracle.prefill(*args, scale)
        o_chk, s_chk = chunked.prefill(*args, scale, L=L)
        np.testing.assert_allclose(o_chk, o_ref, rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(s_chk, s_ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("L", [1, 3, 8, 128])
@pytest.mark.parametrize("rule", ["gated_delta", "gated"])
def test_chunked_per_key_gate_equals_recurrence(L, rule):
    """Prefill with the per-key gate gk: the chunked per-key form (decays
    exp(G_i[d] - G_j[d]) per key) equals the recurrence, which applies
    exp(g) exp(gk[d]) to state row d at every token."""
    rng = np.random.default_rng(200 + L)
    for trial in range(4):
        nseq = int(rng.integers(1, 4))
        lens = [int(x) for x in rng.integers(0, 23, nseq)]
        Nqk = int(rng.integers(1, 3))
        Nv = Nqk * int(rng.integers(1, 3))
        Dk, Dv = int(rng.integers(2, 6)), int(rng.integers(2, 6))
        q, k, v, g, beta, s0, cu = rand_prefill(rng, lens, Nqk, Nv, Dk, Dv, with_state=trial % 2 == 0)
        gk = -rng.uniform(0.0, 1.5, (sum(lens), Nv, Dk))
        scale = float(rng.uniform(0.2, 1.5))
        o_ref, s_ref = oracle.prefill(q, k, v, g, beta, s0, cu, scale, rule=rule, gk=gk)
        o_chk, s_chk = chunked.prefill(q, k, v, g, beta, s0, cu, scale, L=L, rule=rule, gk=gk)
        np.testing.assert_allclose(o_chk, o_ref, rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(s_chk, s_ref, rtol=1e-10, atol=1e-11)


@settings(max_examples=60, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(seed=st.integers(0, 2 ** 31 - 1), L=st.integers(1, 20),
       rule=st.sampled_from(["gated_delta", "delta", "gated", "linear"]),
       gate=st.sampled_from(["weak", "strong", "per_key", "per_key_reset"]))
def test_property_chunked_equals_recurrence(seed, L, rule, gate):
    """Generated cases: any chunk length from 1 to 20, every update rule,
    gates from weak to the decode page's strong range, and per-key gates up
    to a reset of single key rows (gk = -40).  Sequence lengths straddle the
    chunk length (empty, shorter, exact multiples, ragged tails), so a
    mistake at a chunk boundary in either statement shows."""
    rng = np.random.default_rng(seed)
    nseq = int(rng.integers(1, 4))
    lens = [int(rng.choice([0, 1, L - 1, L, L + 1, 2 * L, 3 * L + 2, int(rng.integers(0, 45))])) for _ in range(nseq)]
    lens = [max(x, 0) for x in lens]
    Nqk = int(rng.integers(1, 3))
    Nv = Nqk * int(rng.integers(1, 3))
    Dk, Dv = int(rng.integers(1, 6)), int(rng.integers(1, 6))
    q, k, v, g, beta, s0, cu = rand_prefill(rng, lens, Nqk, Nv, Dk, Dv, with_state=bool(rng.integers(0, 2)))
    T = sum(lens)
    gk = None
    if gate == "strong":
        g = -rng.uniform(0.01, 1.01, (T, Nv))
    elif gate == "weak":
        g = -rng.uniform(0.0, 0.05, (T, Nv))
    else:
        gk = -rng.uniform(0.0, 1.0, (T, Nv, Dk))
        if gate == "per_key_reset":
            gk[rng.random((T, Nv, Dk)) < 0.1] = -40.0
    scale = float(rng.uniform(0.2, 1.5))
    o_ref, s_ref = oracle.prefill(q, k, v, g, beta, s0, cu, scale, rule=rule, gk=gk)
    o_chk, s_chk = chunked.prefill(q, k, v, g, beta, s0, cu, scale, L=L, rule=rule, gk=gk)
    np.testing.assert_allclose(o_chk, o_ref, rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(s_chk, s_ref, rtol=1e-9, atol=1e-10)


def test_per_key_gate_zero_is_no_gate_and_rules_without_decay_ignore_it():
    rng = np.random.default_rng(201)
    q, k, v, g, beta, s0, cu = rand_prefill(rng, [7, 5], 1, 2, 4, 3)
    o0, s_0 = oracle.prefill(q, k, v, g, beta, s0, cu, 0.7)
    o1, s_1 = oracle.prefill(q, k, v, g, beta, s0, cu, 0.7, gk=np.zeros((12, 2, 4)))
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(s_0, s_1)
    gk = -rng.uniform(0.1, 1.0, (12, 2, 4))
    for rule in ("delta", "linear"):
        o2, s2 = oracle.prefill(q, k, v, g, beta, s0, cu, 0.7, rule=rule)
        o3, s3 = oracle.prefill(q, k, v, g, beta, s0, cu, 0.7, rule=rule, gk=gk)
        np.testing.assert_array_equal(o2, o3)
        np.testing.assert_array_equal(s2, s3)


def test_per_key_gate_reset_of_one_key_row():
    """A very negative gk on key row d wipes that row of the state before the
    token's update, in prefill as in decode: with a key that is zero on rows
    0 and 2, row 0 of the final state is exactly zero and row 2 is unchanged."""
    Dk, Dv = 3, 2
    q = np.array([[[1.0, 0.0, 0.0]]])
    k = np.array([[[0.0, 1.0, 0.0]]])
    v = np.array([[[0.5, -0.25]]])
    s0 = np.arange(Dk * Dv, dtype=float).reshape(1, 1, Dk, Dv) + 1.0
    gk = np.zeros((1, 1, Dk))
    gk[0, 0, 0] = -1e4
    _, s = oracle.prefill(q, k, v, np.zeros((1, 1)), np.full((1, 1), 0.5), s0, [0, 1], 1.0, gk=gk)
    np.testing.assert_array_equal(s[0, 0, 0], np.zeros(Dv))          # row 0: reset
    np.testing.assert_allclose(s[0, 0, 2], s0[0, 0, 2], rtol=1e-12)  # row 2: untouched (k_2 = 0)


@pytest.mark.parametrize("reading", [dict(mask_sign=+1.0), dict(strict_out_tril=True),
                                     dict(raw_g_last=True), dict(raw_g_in_kgexp=True)])
def test_alternative_readings_disagree(reading):
    """The readings of the garbled passages are the only ones that agree with
    the recurrence; each alternative is off by a wide margin."""
    rng = np.random.default_rng(7)
    args = rand_prefill(rng, [13], 1, 1, 4, 4)
    o_ref, s_ref = oracle.prefill(*args, 1.0)
    o_alt, s_alt = chunked.prefill(*args, 1.0, L=4, **reading)
    dev = max(np.abs(o_alt - o_ref).max(), np.abs(s_alt - s_ref).max())
    assert dev > 1e-2, reading


def test_matrix_inversion_forms_agree():
    """Neumann series == row recurrence, and (I - A) T == I ("Matrix Inversion")."""
    rng = np.random.default_rng(3)
    for n in (1, 2, 5, 16, 40):
        A = np.tril(rng.standard_normal((n, n)) * 0.3, -1)
        T1 = chunked.inverse_neumann(A)
        T2 = chunked.inverse_rows(A)
        np.testing.assert_allclose(T1, T2, atol=1e-10)
        np.testing.assert_allclose((np.eye(n) - A) @ T2, np.eye(n), atol=1e-10)
        np.testing.assert_allclose(T2, np.linalg.inv(np.eye(n) - A), atol=1e-9)


# ---------------------------------------------------------------- golden

def test_decode_hand_derived_example():
    d = json.load(open(os.path.join(GOLDEN, "decode_hand_2x2.json")))
    q = np.array(d["q"], float)
    k = np.array(d["k"], float)
    v = np.array(d["v"], float)
    g = np.log(np.array(d["g_is_ln"], float))
    gk = np.log(np.array(d["gk_is_ln"], float))
    beta = np.array(d["beta"], float)
    pool = np.array(d["pool"], float)
    out, pool_out = oracle.decode(q, k, v, g, gk, beta, pool, d["idx"], d["lens"], d["scale"])
    np.testing.assert_allclose(out, np.array(d["expected_out"], float), rtol=0, atol=1e-14)
    np.testing.assert_allclose(pool_out, np.array(d["expected_pool"], float), rtol=0, atol=1e-14)


# ---------------------------------------------------------------- closed forms

def _decode_one(q, k, v, g, beta, S0, scale=1.0, gk=None):
    """Single row, single head decode of a token chain over one slot."""
    n = q.shape[0]
    Dk, Dv = S0.shape
    out, pool = oracle.decode(q.reshape(1, 1, n, Dk), k.reshape(1, 1, n, Dk), v.reshape(1, 1, n, Dv),
                              np.asarray(g, float).reshape(1, 1, n),
                              None if gk is None else gk.reshape(1, 1, n, Dk),
                              np.asarray(beta, float).reshape(1, 1, n), S0.reshape(1, 1, Dk, Dv),
                              np.zeros(n, np.int32), [n], scale)
    return out.reshape(n, Dv), pool.reshape(Dk, Dv)


def test_unit_key_read_back_is_exact():
    """beta=1, g=0, zero state and a unit key: the stored association reads back exactly."""
    rng = np.random.default_rng(11)
    Dk, Dv = 8, 6
    for i in range(Dk):
        e = np.zeros(Dk)
        e[i] = 1.0
        v = rng.standard_normal(Dv)
        out, S = _decode_one(e[None], e[None], v[None], [0.0], [1.0], np.zeros((Dk, Dv)))
        assert np.array_equal(out[0], v)
        assert np.array_equal(S[i], v)
        assert not np.any(np.delete(S, i, axis=0))


def test_prefill_read_back_carries_eps():
    """Through prefill the key is normalised with eps under the root, so a unit
    key reads back v * |k|^2 / (|k|^2 + eps) ("L2 Normalization")."""
    rng = np.random.default_rng(12)
    D = 4
    e = np.zeros((1, 1, D))
    e[0, 0, 0] = 1.0
    v = rng.standard_normal((1, 1, D))
    out, S = oracle.prefill(e, e, v, np.zeros((1, 1)), np.ones((1, 1)), None, [0, 1], 1.0)
    c = 1.0 / math.sqrt(1.0 + 1e-6)
    np.testing.assert_allclose(out[0, 0], v[0, 0] * c * c, rtol=1e-15)
    np.testing.assert_allclose(S[0, 0, 0], v[0, 0] * c, rtol=1e-15)


def test_beta_zero_gate_zero_is_identity():
    rng = np.random.default_rng(13)
    q, k, v, g, beta, s0, cu = rand_prefill(rng, [9, 4], 2, 4, 5, 3)
    g[:] = 0.0
    beta[:] = 0.0
    out, s1 = oracle.prefill(q, k, v, g, beta, s0, cu, 0.7)
    assert np.array_equal(s1, s0)
    qn = q / np.sqrt((q * q).sum(-1, keepdims=True) + 1e-6) * 0.7
    for t in range(13):
        b = 0 if t < 9 else 1
        for h in range(4):
            np.testing.assert_allclose(out[t, h], s0[b, h].T @ qn[t, h // 2], rtol=1e-13, atol=1e-14)


def test_pure_decay():
    rng = np.random.default_rng(14)
    q, k, v, g, beta, s0, cu = rand_prefill(rng, [7], 1, 2, 3, 4)
    beta[:] = 0.0
    _, s1 = oracle.prefill(q, k, v, g, beta, s0, cu, 1.0)
    for h in range(2):
        np.testing.assert_allclose(s1[0, h], np.exp(g[:, h].sum()) * s0[0, h], rtol=1e-13)


def test_orthonormal_keys_equal_causal_linear_attention():
    """k_t = e_t, beta=1, g=0, S0=0: the delta rule reduces to causal linear
    attention o_t = sum_{s<=t} (q_t . k_s) v_s (textbook form)."""
    rng = np.random.default_rng(15)
    D, T = 8, 8
    k = np.eye(D)[:T].reshape(T, 1, D)
    q = rng.standard_normal((T, 1, D))
    v = rng.standard_normal((T, 1, D))
    out, _ = oracle.prefill(q, k, v, np.zeros((T, 1)), np.ones((T, 1)), None, [0, T], 1.0)
    qn = q[:, 0] / np.sqrt((q[:, 0] ** 2).sum(-1, keepdims=True) + 1e-6)
    kn = k[:, 0] / math.sqrt(1 + 1e-6)
    for t in range(T):
        expect = sum((qn[t] @ kn[s]) * v[s, 0] for s in range(t + 1))
        np.testing.assert_allclose(out[t, 0], expect, rtol=1e-12, atol=1e-13)


def test_per_key_gate_reset():
    """gk_i = -1e4 zeroes key row i of the state before the update."""
    rng = np.random.default_rng(16)
    Dk, Dv = 5, 3
    S0 = rng.standard_normal((Dk, Dv))
    gk = np.zeros((1, Dk))
    gk[0, 2] = -1e4
    q = rng.standard_normal((1, Dk))
    k = rng.standard_normal((1, Dk))
    _, S1 = _decode_one(q, k, rng.standard_normal((1, Dv)), [-0.3], [0.0], S0, gk=gk)
    expect = S0 * math.exp(-0.3)
    expect[2] = 0.0
    np.testing.assert_allclose(S1, expect, rtol=1e-14, atol=0)


def test_round_bf16_matches_torch_on_fp32_values():
    """On fp32-exact inputs torch's fp32 -> bf16 cast is a single RNE rounding."""
    rng = np.random.default_rng(17)
    x = rng.standard_normal(20000).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0]   # exact ties, both parities
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), ref)


def test_round_fp16_matches_numpy_half():
    """numpy's float64 -> float16 cast is a single RNE rounding (normals,
    subnormals, overflow to infinity)."""
    rng = np.random.default_rng(18)
    x = np.concatenate([rng.standard_normal(20000), rng.standard_normal(2000) * 1e-5,
                        rng.standard_normal(2000) * 3e4, [65504.0, 65519.0, 65520.0, 1e-8, 2.0 ** -25,
                                                          3 * 2.0 ** -25, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11]])
    x = np.concatenate([x, -x])
    with np.errstate(over="ignore"):   # the overflow to infinity is part of the check
        ref = x.astype(np.float16).astype(np.float64)
    assert np.isinf(ref).any() and np.array_equal(oracle.round_fp16(x), ref)


# ---------------------------------------------------------------- invariants

def test_gqa_equals_replicated_heads():
    rng = np.random.default_rng(18)
    q, k, v, g, beta, s0, cu = rand_prefill(rng, [11, 6], 2, 6, 4, 3)
    o1, s1 = oracle.prefill(q, k, v, g, beta, s0, cu, 0.9)
    rep = np.repeat(np.arange(2), 3)
    o2, s2 = oracle.prefill(q[:, rep], k[:, rep], v, g, beta, s0, cu, 0.9)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_varlen_packing_equals_separate_calls():
    rng = np.random.default_rng(19)
    lens = [5, 0, 12, 3]
    q, k, v, g, beta, s0, cu = rand_prefill(rng, lens, 1, 2, 4, 4)
    o, s = oracle.prefill(q, k, v, g, beta, s0, cu, 1.0)
    for b in range(len(lens)):
        a, e = cu[b], cu[b + 1]
        ob, sb = oracle.prefill(q[a:e], k[a:e], v[a:e], g[a:e], beta[a:e], s0[b:b + 1], [0, e - a], 1.0)
        np.testing.assert_array_equal(o[a:e], ob)
        np.testing.assert_array_equal(s[b], sb[0])
    assert np.array_equal(s[1], s0[1])   # an empty sequence passes its state through


def test_split_and_resume_equals_one_call():
    rng = np.random.default_rng(20)
    q, k, v, g, beta, s0, cu = rand_prefill(rng, [30], 1, 1, 4, 5)
    o, s = oracle.prefill(q, k, v, g, beta, s0, cu, 1.0)
    for t1 in (1, 13, 29):
        oa, sa = oracle.prefill(q[:t1], k[:t1], v[:t1], g[:t1], beta[:t1], s0, [0, t1], 1.0)
        ob, sb = oracle.prefill(q[t1:], k[t1:], v[t1:], g[t1:], beta[t1:], sa, [0, 30 - t1], 1.0)
        np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(sb, s, rtol=1e-13, atol=1e-13)


def test_state_independent_of_q_and_output_linear_in_scale():
    rng = np.random.default_rng(21)
    q, k, v, g, beta, s0, cu = rand_prefill(rng, [10], 1, 1, 4, 4)
    o1, s1 = oracle.prefill(q, k, v, g, beta, s0, cu, 0.5)
    o2, s2 = oracle.prefill(-3 * q + 1, k, v, g, beta, s0, cu, 2.0)
    np.testing.assert_array_equal(s1, s2)
    o3, _ = oracle.prefill(q, k, v, g, beta, s0, cu, 2.0)
    np.testing.assert_allclose(o3, 4 * o1, rtol=1e-13, atol=1e-14)


def test_multi_token_decode_equals_chained_single_tokens():
    """Routing reading: the chain starts at idx[b*S+0]; the state after token
    t lands in idx[b*S+t]; later writes to one slot win."""
    rng = np.random.default_rng(22)
    B, S, Nk, Nv, Dk, Dv, slots = 3, 4, 1, 2, 4, 3, 8
    q = rng.standard_normal((B, Nk, S, Dk))
    k = rng.standard_normal((B, Nk, S, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, Nv, S, Dv))
    g = -rng.uniform(0.01, 1, (B, Nv, S))
    gk = -rng.uniform(0.01, 1, (B, Nv, S, Dk))
    beta = rng.uniform(0.05, 0.95, (B, Nv, S))
    pool = rng.standard_normal((slots, Nv, Dk, Dv))
    idx = np.array([[5, 1, 5, 2], [0, 0, -1, -1], [3, 4, 6, 7]], np.int32)
    lens = np.array([4, 2, 0], np.int32)
    out, pool_out = oracle.decode(q, k, v, g, gk, beta, pool, idx.reshape(-1), lens, 0.8)
    expect = pool.copy()
    for b in range(B):
        for h in range(Nv):
            if lens[b] == 0:
                assert not np.any(out[b, h])
                continue
            Sm = pool[idx[b, 0], h]
            for t in range(lens[b]):
                o1, Sm = _decode_one(q[b, 0, t][None], k[b, 0, t][None], v[b, h, t][None], [g[b, h, t]],
                                     [beta[b, h, t]], Sm, scale=0.8, gk=gk[b, h, t][None])
                np.testing.assert_allclose(out[b, h, t], o1[0], rtol=1e-14, atol=1e-15)
                expect[idx[b, t], h] = Sm
            assert not np.any(out[b, h, lens[b]:])
    np.testing.assert_allclose(pool_out, expect, rtol=1e-14, atol=1e-15)
    # slot 2 receives the state after token 3, slot 5 the one after token 2
    assert not np.array_equal(pool_out[5], pool[5]) and not np.array_equal(pool_out[2], pool[2])


# ---------------------------------------------------------------- update rules

@pytest.mark.parametrize("rule", ["gated_delta", "delta", "gated", "linear"])
@pytest.mark.parametrize("L", [1, 3, 8])
def test_update_rules_chunked_equal_recurrence(rule, L):
    """Each update rule ("LinearAttention" page, update_rule): the chunked
    statement (no pre-attention matrix without the delta term, g = 0
    without the gate) equals the per-token recurrence."""
    rng = np.random.default_rng(60 + L)
    q, k, v, g, beta, s0, cu = rand_prefill(rng, [11, 5], 1, 2, 4, 3)
    o_r, s_r = oracle.prefill(q, k, v, g, beta, s0, cu, 0.8, rule=rule)
    o_c, s_c = chunked.prefill(q, k, v, g, beta, s0, cu, 0.8, L=L, rule=rule)
    np.testing.assert_allclose(o_c, o_r, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s_c, s_r, rtol=1e-11, atol=1e-12)


def test_linear_and_gated_rules_closed_form():
    """Without the delta term the state is a (decayed) sum of outer products:
    o_t = e^{G_t} S0^T q_t + sum_{s<=t} e^{G_t - G_s} (q_t . k_s) v_s with
    G_t = sum_{r<=t} g_r (G = 0 for the linear rule); beta plays no part."""
    rng = np.random.default_rng(64)
    T, Dk, Dv = 9, 5, 4
    q, k, v, g, beta, s0, cu = rand_prefill(rng, [T], 1, 1, Dk, Dv)
    qn = q[:, 0] / np.sqrt(np.sum(q[:, 0] ** 2, -1, keepdims=True) + 1e-6) * 0.7
    kn = k[:, 0] / np.sqrt(np.sum(k[:, 0] ** 2, -1, keepdims=True) + 1e-6)
    for rule, G in (("linear", np.zeros(T)), ("gated", np.cumsum(g[:, 0]))):
        o, st = oracle.prefill(q, k, v, g, beta, s0, cu, 0.7, rule=rule)
        o2, _ = oracle.prefill(q, k, v, g, np.ones_like(beta), s0, cu, 0.7, rule=rule)
        assert np.array_equal(o, o2)
        for t in range(T):
            ref = np.exp(G[t]) * s0[0, 0].T @ qn[t]
            for s_ in range(t + 1):
                ref += np.exp(G[t] - G[s_]) * (qn[t] @ kn[s_]) * v[s_, 0]
            np.testing.assert_allclose(o[t, 0], ref, rtol=1e-12, atol=1e-13)
        Sref = np.exp(G[-1]) * s0[0, 0] + sum(np.exp(G[-1] - G[s_]) * np.outer(kn[s_], v[s_, 0]) for s_ in range(T))
        np.testing.assert_allclose(st[0, 0], Sref, rtol=1e-12, atol=1e-13)


def test_delta_rule_is_gated_delta_without_gates():
    rng = np.random.default_rng(65)
    q, k, v, g, beta, s0, cu = rand_prefill(rng, [7, 4], 1, 2, 4, 3)
    a = oracle.prefill(q, k, v, g, beta, s0, cu, 0.5, rule="delta")
    b = oracle.prefill(q, k, v, np.zeros_like(g), beta, s0, cu, 0.5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # decode: g and gk are ignored by the delta and linear rules
    _, r, _ = _spec_case(66)
    pool = rng.standard_normal((4, 2, 4, 3))
    idx = np.repeat(np.array([0, 1, 2], np.int32), 4)
    lens = np.array([4, 3, 1], np.int32)
    d1 = oracle.decode(*r[:4], r[4], r[5], pool, idx, lens, 0.9, rule="delta")
    d2 = oracle.decode(r[0], r[1], r[2], np.zeros_like(r[3]), None, r[5], pool, idx, lens, 0.9)
    for x, y in zip(d1, d2):
        assert np.array_equal(x, y)
    l1 = oracle.decode(*r[:4], r[4], r[5], pool, idx, lens, 0.9, rule="linear")
    l2 = oracle.decode(*r[:4], None, np.ones_like(r[5]), pool, idx, lens, 0.9, rule="gated")
    l3 = oracle.decode(r[0], r[1], r[2], np.zeros_like(r[3]), None, r[5], pool, idx, lens, 0.9, rule="gated")
    for x, y in zip(l1, l3):
        assert np.array_equal(x, y)
    assert not np.array_equal(l1[0], l2[0])


def _spec_case(seed, B=3, S=4, Nk=1, Nv=2, Dk=4, Dv=3):
    rng = np.random.default_rng(seed)
    def toks():
        q = rng.standard_normal((B, Nk, S, Dk))
        k = rng.standard_normal((B, Nk, S, Dk))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        return (q, k, rng.standard_normal((B, Nv, S, Dv)), -rng.uniform(0.01, 1, (B, Nv, S)),
                -rng.uniform(0.01, 1, (B, Nv, S, Dk)), rng.uniform(0.05, 0.95, (B, Nv, S)))
    return rng, toks(), toks()


def test_speculative_continuation_starts_after_the_accepted_prefix():
    """num_accepted_tokens (decode page, parameters): a call that drafted S
    tokens stores the state after each token t in slot idx[b*S+t]; the next
    call, told that n_b tokens were accepted, must continue from the state
    after exactly n_b tokens of the first chain -- the same result as feeding
    only the accepted tokens through one slot and then the new ones."""
    B, S, Nv, Dk, Dv = 3, 4, 2, 4, 3
    rng, r1, r2 = _spec_case(40, B, S, 1, Nv, Dk, Dv)
    slots = B * S + B
    pool = rng.standard_normal((slots, Nv, Dk, Dv))
    # row b starts from its own slot b, which also receives the state after
    # its token 0; each later drafted token has a slot of its own
    idx = (np.arange(B * S, dtype=np.int32) + B).reshape(B, S)
    start = np.arange(B, dtype=np.int32)
    idx[:, 0] = start
    idx = idx.reshape(-1)
    lens = np.full(B, S, np.int32)
    _, pool1 = oracle.decode(*r1[:4], r1[4], r1[5], pool, idx, lens, 0.7)
    nacc = np.array([1, 3, 4], np.int32)
    out2, _ = oracle.decode(*r2[:4], r2[4], r2[5], pool1, idx, lens, 0.7, num_accepted=nacc)
    for b in range(B):
        for h in range(Nv):
            n = int(nacc[b])
            cat = lambda a, c: np.concatenate([a[b, 0 if a.shape[1] == 1 else h, :n], c[b, 0 if c.shape[1] == 1 else h]])
            q = cat(r1[0], r2[0]); k = cat(r1[1], r2[1]); v = cat(r1[2], r2[2])
            g = cat(r1[3], r2[3]); gk = cat(r1[4], r2[4]); beta = cat(r1[5], r2[5])
            o_ref, _ = _decode_one(q, k, v, g, beta, pool[start[b], h], scale=0.7, gk=gk)
            np.testing.assert_allclose(out2[b, h], o_ref[n:], rtol=1e-12, atol=1e-13)


def test_num_accepted_equal_to_length_is_ordinary_inference():
    """With every index of a row naming one slot (ordinary inference),
    num_accepted_tokens = actual_seq_lengths changes nothing."""
    B, S = 3, 4
    rng, r, _ = _spec_case(41, B, S)
    pool = rng.standard_normal((5, 2, 4, 3))
    idx = np.repeat(np.array([3, 0, 4], np.int32), S)
    lens = np.array([4, 2, 3], np.int32)
    a = oracle.decode(*r[:4], r[4], r[5], pool, idx, lens, 0.9)
    b = oracle.decode(*r[:4], r[4], r[5], pool, idx, lens, 0.9, num_accepted=lens)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_num_accepted_clamps_and_empty_initial_slot_is_zero():
    """n is clamped to 1..S; an initial index outside the pool (a padded
    position) starts the chain from a zero state."""
    B, S = 2, 4
    rng, r, _ = _spec_case(42, B, S)
    pool = rng.standard_normal((6, 2, 4, 3))
    idx = np.array([1, 2, -1, -1, 3, 4, 5, 0], np.int32)
    lens = np.array([2, 4], np.int32)
    o_hi, _ = oracle.decode(*r[:4], r[4], r[5], pool, idx, lens, 1.0, num_accepted=np.array([9, 9], np.int32))
    o_s, _ = oracle.decode(*r[:4], r[4], r[5], pool, idx, lens, 1.0, num_accepted=np.array([4, 4], np.int32))
    assert np.array_equal(o_hi, o_s)
    o_lo, _ = oracle.decode(*r[:4], r[4], r[5], pool, idx, lens, 1.0, num_accepted=np.array([0, -3], np.int32))
    o_1, _ = oracle.decode(*r[:4], r[4], r[5], pool, idx, lens, 1.0)
    assert np.array_equal(o_lo, o_1)
    # row 0 with n = 4 reads idx[3] = -1: same as a chain from a zero slot
    zpool = pool.copy()
    zpool[1] = 0.0
    o_z, _ = oracle.decode(*r[:4], r[4], r[5], zpool, idx, lens, 1.0)
    np.testing.assert_array_equal(o_s[0], o_z[0])


def test_decode_equals_prefill_on_unit_inputs():
    """Cross-path: decode token by token == prefill of the same sequence when
    q, k are already unit (prefill then only adds the eps of its norm)."""
    rng = np.random.default_rng(23)
    T, Dk, Dv = 9, 6, 5
    q = rng.standard_normal((T, 1, Dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, 1, Dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, 1, Dv))
    g = -rng.uniform(0.01, 0.5, (T, 1))
    beta = rng.uniform(0.05, 0.95, (T, 1))
    s0 = rng.standard_normal((1, 1, Dk, Dv))
    o_p, s_p = oracle.prefill(q, k, v, g, beta, s0, [0, T], 0.6)
    Sm = s0[0, 0]
    for t in range(T):
        o1, Sm = _decode_one(q[t], k[t], v[t], g[t], beta[t], Sm, scale=0.6)
        np.testing.assert_allclose(o1[0], o_p[t, 0], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(Sm, s_p[0, 0], rtol=1e-5, atol=1e-5)
    # and with the per-key gate: prefill's gk [T, Nv, Dk] is decode's [B, Nv, S, Dk]
    gk = -rng.uniform(0.01, 1.0, (T, 1, Dk))
    o_p, s_p = oracle.prefill(q, k, v, g, beta, s0, [0, T], 0.6, gk=gk)
    Sm = s0[0, 0]
    for t in range(T):
        o1, Sm = _decode_one(q[t], k[t], v[t], g[t], beta[t], Sm, scale=0.6, gk=gk[t])
        np.testing.assert_allclose(o1[0], o_p[t, 0], rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(Sm, s_p[0, 0], rtol=1e-5, atol=1e-5)


def test_oracle_rejects_bad_sizes():
    with pytest.raises(ValueError):
        oracle.prefill(np.zeros((2, 3, 4)), np.zeros((2, 3, 4)), np.zeros((2, 4, 4)),
                       np.zeros((2, 4)), np.zeros((2, 4)), None, [0, 2], 1.0)   # Nv % Nqk != 0
    with pytest.raises(ValueError):   # index out of range
        _ = oracle.decode(np.zeros((1, 1, 1, 2)), np.zeros((1, 1, 1, 2)), np.zeros((1, 1, 1, 2)),
                          np.zeros((1, 1, 1)), None, np.zeros((1, 1, 1)), np.zeros((1, 1, 2, 2)),
                          [3], [1], 1.0)

"""Seeded synthetic inputs for the Gated Delta Rule (shared by tests and bench).

This module draws inputs only; it contains none of the operator's arithmetic.
Both the fp64 oracle and the GPU path receive the *same* host tensors (the
GPU side copies them to the device), so parity compares like with like.

Recipe (numpy PCG64, seeded): values are drawn in fp64 and cast once to the
storage dtype (bf16 or fp32) with torch's round-to-nearest-even conversion.
Distributions follow the pages' workloads:
  * prefill ("Qwen3Next Samples" page, Parameter Description / Supported
    Configurations): q, k, v ~ N(0,1); beta = sigmoid(N(0,1)); gate
    g = -U(0.001, 0.1) per token and value head; initial state zeros or
    N(0, 0.02^2); D = 128.
  * decode ("lite_boost.ops.recurrent_gated_delta_rule" page, example):
    q, k drawn N(0,1) and L2-normalised in fp64 before the bf16 cast (the
    operator requires unit-norm q and k from its caller); v ~ N(0,1);
    beta = U(0.05, 0.95); g = -U(0.01, 1.01); gk = -U(0.01, 1.01);
    state pool ~ N(0, 0.02^2).
"""
from __future__ import annotations

import math

import numpy as np
import torch

SCALE_128 = 1.0 / math.sqrt(128.0)

_TORCH_DTYPE = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(_TORCH_DTYPE[dtype]).contiguous()


def _normal_blocks(rng, shape, std=1.0, dtype="bf16", block_rows=8192):
    """N(0, std^2) of `shape`, drawn in fp64 block by block along axis 0 (to
    bound host memory for the long-context workload), cast per block."""
    out = torch.empty(shape, dtype=_TORCH_DTYPE[dtype])
    for r0 in range(0, shape[0], block_rows):
        r1 = min(shape[0], r0 + block_rows)
        out[r0:r1] = _cast(rng.standard_normal((r1 - r0,) + tuple(shape[1:])) * std, dtype)
    return out


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def prefill_inputs(seed: int, seq_lens, Nqk: int, Nv: int, D: int = 128, act: str = "bf16",
                   init_state: str = "randn", scale: float | None = None, gk: str | None = None,
                   g_range=(0.001, 0.1)):
    """Packed varlen prefill inputs.

    Returns a dict of CPU tensors: q, k [T,Nqk,D]; v [T,Nv,D]; beta [T,Nv]
    (act dtype); g [T,Nv] fp32; state_in [B,Nv,D,D] fp32 or None;
    cu_seqlens [B+1] int32; gk [T,Nv,D] fp32 or None; plus scale, T, B, Nqk,
    Nv, D, act.  g = -U(g_range).  gk: None; "strong", the decode page's
    example range -U(0.01, 1.01); "weak", -U(0.001, 0.05), under which the
    state carries across chunks; "extreme", -U(0.01, 40); or "reset", weak
    everywhere except about one (token, value head, key) entry in a hundred,
    where it is -1e4 (that key row of the state is wiped before the token's
    update).  gk is drawn last, so the other inputs do not depend on it.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    seq_lens = [int(x) for x in seq_lens]
    B = len(seq_lens)
    T = int(sum(seq_lens))
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(seq_lens)
    q = _normal_blocks(rng, (T, Nqk, D), dtype=act)
    k = _normal_blocks(rng, (T, Nqk, D), dtype=act)
    v = _normal_blocks(rng, (T, Nv, D), dtype=act)
    beta = _cast(_sigmoid(rng.standard_normal((T, Nv))), act)
    g = _cast(-rng.uniform(g_range[0], g_range[1], (T, Nv)), "fp32")
    if init_state == "zeros":
        state_in = None
    elif init_state == "randn":
        state_in = _normal_blocks(rng, (B, Nv, D, D), std=0.02, dtype="fp32", block_rows=1)
    else:
        raise ValueError(init_state)
    if gk is None:
        gkt = None
    elif gk in ("strong", "weak", "extreme"):
        lo, hi = {"strong": (0.01, 1.01), "weak": (0.001, 0.05), "extreme": (0.01, 40.0)}[gk]
        gkt = _cast(-rng.uniform(lo, hi, (T, Nv, D)), "fp32")
    elif gk == "reset":
        x = -rng.uniform(0.001, 0.05, (T, Nv, D))
        x[rng.random((T, Nv, D)) < 0.01] = -1e4
        gkt = _cast(x, "fp32")
    else:
        raise ValueError(gk)
    return dict(q=q, k=k, v=v, g=g, beta=beta, state_in=state_in,
                cu_seqlens=torch.from_numpy(cu), scale=SCALE_128 if scale is None else scale,
                T=T, B=B, Nqk=Nqk, Nv=Nv, D=D, act=act, gk=gkt)


def large_prefill_inputs(seed: int, seq_lens, Nqk: int, Nv: int, D: int = 128):
    """Packed varlen bf16 prefill inputs too large to draw in fp64 in
    reasonable time (hundreds of thousands of tokens): the same
    distributions as prefill_inputs (q, k, v ~ N(0,1); beta =
    sigmoid(N(0,1)); g = -U(0.001, 0.1); state_in ~ N(0, 0.02^2)), drawn in
    fp32 from torch's seeded CPU generator and cast to bf16.  Same dict
    layout as prefill_inputs (gk None)."""
    gen = torch.Generator().manual_seed(seed)
    seq_lens = [int(x) for x in seq_lens]
    B, T = len(seq_lens), int(sum(seq_lens))
    cu = torch.zeros(B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(seq_lens, dtype=torch.int64), 0).to(torch.int32)

    def normal(shape, std=1.0, dtype=torch.bfloat16, rows=65536):
        out = torch.empty(shape, dtype=dtype)
        for r0 in range(0, shape[0], rows):
            r1 = min(shape[0], r0 + rows)
            out[r0:r1] = (torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen) * std).to(dtype)
        return out

    q = normal((T, Nqk, D))
    k = normal((T, Nqk, D))
    v = normal((T, Nv, D))
    beta = torch.sigmoid(torch.randn((T, Nv), generator=gen)).to(torch.bfloat16)
    g = -(0.001 + 0.099 * torch.rand((T, Nv), generator=gen))
    state_in = normal((B, Nv, D, D), std=0.02, dtype=torch.float32, rows=1)
    return dict(q=q, k=k, v=v, g=g.contiguous(), beta=beta.contiguous(), state_in=state_in, cu_seqlens=cu,
                scale=SCALE_128, T=T, B=B, Nqk=Nqk, Nv=Nv, D=D, act="bf16", gk=None)


def _unit_rows(rng, shape):
    x = rng.standard_normal(shape)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def decode_inputs(seed: int, B: int, S: int, Nk: int, Nv: int, Dk: int, Dv: int, num_slots: int,
                  with_gk: bool = False, lens: str = "full", routing: str = "one_slot",
                  act: str = "bf16", state: str = "bf16", scale: float | None = None,
                  accepted: bool = False):
    """Recurrent-decode inputs over a slot pool.

    lens:    "full" (every row has S valid tokens) or "random" (U{1..S}).
    routing: "one_slot"  -- row b uses one slot for all its tokens, the first
                            B entries of a seeded permutation of the slots;
             "two_slots" -- row b owns slots {pi[2b], pi[2b+1]} of a seeded
                            permutation and each valid token picks one of the
                            two at random (collision-free across rows);
             "per_token" -- speculative decoding: row b owns S slots
                            pi[S b .. S b + S - 1], one per token position,
                            padded positions included.
    accepted: also draw num_accepted_tokens nacc [B] ~ U{1..S}.
    Padded token positions (t >= len_b) get zero-valued inputs and, except
    under per_token routing, index -1.
    Returns a dict of CPU tensors: q, k [B,Nk,S,Dk]; v [B,Nv,S,Dv];
    beta [B,Nv,S]; g [B,Nv,S] fp32; gk [B,Nv,S,Dk] fp32 or None;
    pool [slots,Nv,Dk,Dv]; idx [B*S] int32; lens [B] int32; scale.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _cast(_unit_rows(rng, (B, Nk, S, Dk)), act)
    k = _cast(_unit_rows(rng, (B, Nk, S, Dk)), act)
    v = _cast(rng.standard_normal((B, Nv, S, Dv)), act)
    beta = _cast(rng.uniform(0.05, 0.95, (B, Nv, S)), act)
    g = _cast(-rng.uniform(0.01, 1.01, (B, Nv, S)), "fp32")
    gk = _cast(-rng.uniform(0.01, 1.01, (B, Nv, S, Dk)), "fp32") if with_gk else None
    pool = _normal_blocks(rng, (num_slots, Nv, Dk, Dv), std=0.02, dtype=state, block_rows=1)
    if lens == "full":
        ln = np.full(B, S, np.int32)
    elif lens == "random":
        ln = rng.integers(1, S + 1, B).astype(np.int32)
    else:
        raise ValueError(lens)
    perm = rng.permutation(num_slots).astype(np.int32)
    idx = np.full((B, S), -1, np.int32)
    if routing == "one_slot":
        if num_slots < B:
            raise ValueError("one_slot routing needs num_slots >= B")
        for b in range(B):
            idx[b, :ln[b]] = perm[b]
    elif routing == "two_slots":
        if num_slots < 2 * B:
            raise ValueError("two_slots routing needs num_slots >= 2B")
        pick = rng.integers(0, 2, (B, S))
        for b in range(B):
            idx[b, :ln[b]] = perm[2 * b + pick[b, :ln[b]]]
    elif routing == "per_token":
        if num_slots < S * B:
            raise ValueError("per_token routing needs num_slots >= S*B")
        idx[:] = perm[:S * B].reshape(B, S)
    else:
        raise ValueError(routing)
    nacc = rng.integers(1, S + 1, B).astype(np.int32) if accepted else None
    # padded tokens carry zero-valued inputs (they are never read)
    for b in range(B):
        if ln[b] < S:
            q[b, :, ln[b]:] = 0
            k[b, :, ln[b]:] = 0
            v[b, :, ln[b]:] = 0
            beta[b, :, ln[b]:] = 0
            g[b, :, ln[b]:] = 0
            if gk is not None:
                gk[b, :, ln[b]:] = 0
    return dict(q=q, k=k, v=v, g=g, gk=gk, beta=beta, pool=pool,
                idx=torch.from_numpy(idx.reshape(-1).copy()), lens=torch.from_numpy(ln),
                nacc=None if nacc is None else torch.from_numpy(nacc),
                scale=SCALE_128 if scale is None else scale,
                B=B, S=S, Nk=Nk, Nv=Nv, Dk=Dk, Dv=Dv, num_slots=num_slots, act=act, state=state)


# The five workloads the operator is measured on.  The T=256 and T=8192
# prefills and both decode workloads are small enough for full parity; the
# T=131072 long-context prefill is parity-checked on sampled heads.
def config_inputs(n: int):
    if n == 1:
        return prefill_inputs(1, [256], Nqk=2, Nv=4, act="fp32", init_state="zeros")
    if n == 2:
        return prefill_inputs(2, [1000, 4096, 300, 2796], Nqk=16, Nv=32, act="bf16")
    if n == 3:
        return decode_inputs(3, B=256, S=1, Nk=16, Nv=32, Dk=128, Dv=128, num_slots=512)
    if n == 4:
        return decode_inputs(4, B=64, S=4, Nk=64, Nv=64, Dk=64, Dv=512, num_slots=128,
                             with_gk=True, lens="random", routing="two_slots")
    if n == 5:
        return prefill_inputs(5, [131072], Nqk=16, Nv=32, act="bf16")
    raise ValueError(n)


CONFIG_NAMES = {
    1: "prefill T=256 Nqk=2 Nv=4 D=128 fp32",
    2: "prefill varlen B=4 lens=[1000,4096,300,2796] T=8192 Nqk=16 Nv=32 D=128 bf16",
    3: "decode B=256 S=1 Nk=16 Nv=32 Dk=Dv=128 bf16 pool 512 slots",
    4: "decode B=64 S=4 (lens U{1..4}) Nk=Nv=64 Dk=64 Dv=512 gk, bf16 pool 128 slots",
    5: "prefill long-context B=1 T=131072 Nqk=16 Nv=32 D=128 bf16",
}


# Extra workloads beyond the five configured ones.  "long few heads" has too
# few (sequence, value head) streams to fill the GPU with the one-level scan,
# so the library scans it in two levels.  The two "varlen gk" ones are the
# T=8192 prefill with a per-key gate: in the decode page's example range,
# and small (under which every 16-token block's diagonal tiles take the fp16
# path).
EXTRA_NAMES = {
    "long_few_heads": "prefill long-context few heads B=1 T=131072 Nqk=1 Nv=4 D=128 bf16",
    "varlen_gk": "prefill varlen B=4 lens=[1000,4096,300,2796] T=8192 Nqk=16 Nv=32 D=128 bf16, "
                 "per-key gate gk=-U(0.01,1.01)",
    "varlen_gk_small": "prefill varlen B=4 lens=[1000,4096,300,2796] T=8192 Nqk=16 Nv=32 D=128 bf16, "
                       "per-key gate gk=-U(0.001,0.05)",
}


def extra_inputs(name: str):
    if name == "long_few_heads":
        return prefill_inputs(6, [131072], Nqk=1, Nv=4, act="bf16")
    if name == "varlen_gk":
        return prefill_inputs(7, [1000, 4096, 300, 2796], Nqk=16, Nv=32, act="bf16", gk="strong")
    if name == "varlen_gk_small":
        return prefill_inputs(8, [1000, 4096, 300, 2796], Nqk=16, Nv=32, act="bf16", gk="weak")
    raise ValueError(name)


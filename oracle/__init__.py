"""fp64 CPU oracle for the Gated Delta Rule (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU product path
(``gated_delta_rule_chunk_amd``) never imports it and shares no code with it.

Contents
--------
``gdr_oracle.c``   the per-token recurrence in fp64 (decode page
                   "lite_boost.ops.recurrent_gated_delta_rule", algorithm
                   flow), OpenMP over independent (sequence, value head)
                   streams; prefill adds the in-op L2 normalisation of the
                   "Qwen3Next Samples" page (L2 Normalization formula).
``chunked.py``     an independent fp64 numpy statement of the chunked formulas
                   of the "Qwen3Next Samples" page (Mathematical Formulas);
                   it exists to pin the recurrence and is used only by tests.

Inputs are widened exactly to float64 (bf16 and fp32 values are exactly
representable), so the oracle's only rounding is fp64 arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_PLAIN_LIB = os.path.join(_HERE, "liboracle.so")
# A build instrumented with AddressSanitizer and UndefinedBehaviorSanitizer
# (every finding aborts); selected with GDR_ORACLE_SANITIZED=1, in a process
# that preloads the sanitizer runtimes.
_SAN_LIB = os.path.join(_HERE, "liboracle_san.so")
SANITIZED = os.environ.get("GDR_ORACLE_SANITIZED") == "1"
_LIB_PATH = _SAN_LIB if SANITIZED else _PLAIN_LIB
_lib = None


def build(force: bool = True, sanitized: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, IEEE fp64 semantics); with
    `sanitized`, the ASan + UBSan build instead."""
    path = _SAN_LIB if sanitized else _PLAIN_LIB
    if force or not os.path.exists(path):
        tmp = path + ".tmp"
        san = ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all"] if sanitized else []
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", *san, "-shared", "-fPIC",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, path)
    return path


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True, sanitized=SANITIZED)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        i = ctypes.c_int
        lib.gdr_oracle_prefill.argtypes = [dp, dp, dp, dp, dp, dp, dp, ip, i, i, i, i, i, i,
                                           ctypes.c_double, i, dp, dp]
        lib.gdr_oracle_prefill.restype = i
        lib.gdr_oracle_decode.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, i, ip, ip, ip,
                                          i, i, i, i, i, i, ctypes.c_double, i, i, dp]
        lib.gdr_oracle_decode.restype = i
        lib.gdr_oracle_round_bf16.argtypes = [ctypes.c_double]
        lib.gdr_oracle_round_bf16.restype = ctypes.c_double
        lib.gdr_oracle_round_fp16.argtypes = [ctypes.c_double]
        lib.gdr_oracle_round_fp16.restype = ctypes.c_double
        lib.gdr_oracle_num_threads.argtypes = []
        lib.gdr_oracle_num_threads.restype = i
        _lib = lib
    return _lib


def _f64(x):
    """Widen a numpy array or CPU torch tensor exactly to contiguous float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (bf16 -> fp64 is exact)
        import torch
        x = x.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _i32(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=np.int32)


def _dp(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _ip(a):
    if a is None:
        return ctypes.POINTER(ctypes.c_int32)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def num_threads() -> int:
    return int(_load().gdr_oracle_num_threads())


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even), as float64."""
    f = _load().gdr_oracle_round_bf16
    x = np.asarray(x, dtype=np.float64)
    return np.vectorize(f, otypes=[np.float64])(x) if x.size else x.copy()


def round_fp16(x):
    """Round float64 values to the nearest IEEE half (ties to even), as float64."""
    f = _load().gdr_oracle_round_fp16
    x = np.asarray(x, dtype=np.float64)
    return np.vectorize(f, otypes=[np.float64])(x) if x.size else x.copy()


RULES = {"gated_delta": 0, "delta": 1, "gated": 2, "linear": 3}


def prefill(q, k, v, g, beta, state_in, cu_seqlens, scale, rule="gated_delta", gk=None):
    """Chunked-prefill semantics by the per-token recurrence.

    q, k [T,Nqk,Dk]; v [T,Nv,Dv]; g, beta [T,Nv]; state_in [B,Nv,Dk,Dv] or
    None (zeros); cu_seqlens [B+1]; rule one of RULES; gk [T,Nv,Dk] or None
    (the per-key gate: state row i also decays by exp(gk[t,h,i])).  Returns
    (out [T,Nv,Dv], state_out [B,Nv,Dk,Dv]) in float64.
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    gk = _f64(gk)
    state_in = _f64(state_in)
    cu = _i32(cu_seqlens)
    T, Nqk, Dk = q.shape
    Nv, Dv = v.shape[1], v.shape[2]
    B = cu.shape[0] - 1
    assert k.shape == q.shape and v.shape[0] == T and g.shape == (T, Nv) and beta.shape == (T, Nv)
    if state_in is not None:
        assert state_in.shape == (B, Nv, Dk, Dv)
    if gk is not None:
        assert gk.shape == (T, Nv, Dk)
    out = np.zeros((T, Nv, Dv), np.float64)
    state_out = np.zeros((B, Nv, Dk, Dv), np.float64)
    rc = _load().gdr_oracle_prefill(_dp(q), _dp(k), _dp(v), _dp(g), _dp(gk), _dp(beta), _dp(state_in),
                                    _ip(cu), T, B, Nqk, Nv, Dk, Dv, float(scale), RULES[rule],
                                    _dp(out), _dp(state_out))
    if rc != 0:
        raise ValueError(f"oracle prefill rejected its arguments (rc={rc})")
    return out, state_out


def decode(q, k, v, g, gk, beta, pool, idx, lens, scale, round_state_bf16=False, num_accepted=None,
           rule="gated_delta", round_state=None, in_place=False):
    """Recurrent decode over a slot pool.

    q, k [B,Nk,S,Dk] (caller-normalised); v [B,Nv,S,Dv]; g, beta [B,Nv,S];
    gk [B,Nv,S,Dk] or None; pool [slots,Nv,Dk,Dv]; idx [B*S]; lens [B];
    num_accepted [B] or None (row b starts from slot idx[b*S + n_b - 1]).
    Returns (out [B,Nv,S,Dv], pool_out [slots,Nv,Dk,Dv]) in float64; pool_out
    equals the input pool except for the slots the call writes.  With
    `in_place` (for timing; rows must not share slots) the written states go
    into the float64 widening of `pool` itself, which is returned, instead of
    into a copy; a float64 numpy `pool` is then updated in place.
    """
    q, k, v, g, beta, pool = map(_f64, (q, k, v, g, beta, pool))
    gk = _f64(gk)
    idx = _i32(idx).reshape(-1)
    lens = _i32(lens).reshape(-1)
    B, Nk, S, Dk = q.shape
    Nv, Dv = v.shape[1], v.shape[3]
    slots = pool.shape[0]
    assert pool.shape == (slots, Nv, Dk, Dv) and idx.shape[0] == B * S and lens.shape[0] == B
    nacc = None if num_accepted is None else _i32(num_accepted).reshape(-1)
    assert nacc is None or nacc.shape[0] == B
    out = np.zeros((B, Nv, S, Dv), np.float64)
    pool_out = pool if in_place else pool.copy()
    rc = _load().gdr_oracle_decode(_dp(q), _dp(k), _dp(v), _dp(g), _dp(gk), _dp(beta),
                                   _dp(pool), _dp(pool_out), slots, _ip(idx), _ip(lens), _ip(nacc),
                                   B, S, Nk, Nv, Dk, Dv, float(scale),
                                   {None: 0, "bf16": 1, "fp16": 2}["bf16" if round_state_bf16 else round_state],
                                   RULES[rule], _dp(out))
    if rc != 0:
        raise ValueError(f"oracle decode rejected its arguments (rc={rc})")
    return out, pool_out

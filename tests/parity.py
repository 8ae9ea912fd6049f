"""Comparison helpers for GPU-vs-oracle parity.

Tolerances (written here and used by every parity test):
  * outputs:  max_i (|y_i - y_ref_i| - h_i) <= 2e-2 * RMS(y_ref), where
    y_ref is the fp64 oracle, RMS runs over all compared elements and h_i is
    half a unit in the last place of y_ref_i in the output dtype (bf16 or
    fp16; 0 for fp32 outputs).  A bf16 output cannot be closer to the exact value than its own
    rounding, and that rounding alone reaches 2.4e-2 to 4.8e-2 of RMS on
    these workloads, so the bound applies to the error beyond it.
  * states:   ||S - S_ref||_F / ||S_ref||_F <= 1e-3, with S_ref the oracle's
    fp32-exact state for fp32 states and its bf16 / fp16 rounding for such
    pools.
  * routing and untouched slots: bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

OUT_TOL = 2e-2
STATE_TOL = 1e-3


def to_f64(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu", torch.float64).numpy()


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at |x| (8 significant bits): 2^(floor(log2|x|) - 8)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(e - 8), 0.0)


def half_ulp_fp16(x: np.ndarray) -> np.ndarray:
    """Half an IEEE-half ulp at |x| (11 significant bits; subnormal step 2^-24)."""
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    return np.where(ax > 0, np.exp2(np.maximum(e, -14) - 11), 0.0)


def out_error(y, y_ref, bf16):
    """(excess error / RMS, literal max error / RMS) of an output tensor.
    `bf16`: True or "bf16" for bf16 outputs, "fp16" for half outputs, False
    or "fp32" for fp32 outputs."""
    y = to_f64(y)
    y_ref = to_f64(y_ref)
    rms = float(np.sqrt(np.mean(y_ref * y_ref))) if y_ref.size else 0.0
    if rms == 0.0:
        rms = 1.0
    d = np.abs(y - y_ref)
    lit = float(d.max()) / rms if d.size else 0.0
    if bf16 == "fp16":
        ex = d - half_ulp_fp16(y_ref)
    elif bf16 is True or bf16 == "bf16":
        ex = d - half_ulp_bf16(y_ref)
    else:
        ex = d
    exc = float(max(ex.max(), 0.0)) / rms if d.size else 0.0
    return exc, lit


def state_error(s, s_ref) -> float:
    s = to_f64(s)
    s_ref = to_f64(s_ref)
    den = float(np.linalg.norm(s_ref))
    num = float(np.linalg.norm(s - s_ref))
    return num / den if den > 0 else num


def out_kind(t) -> str:
    """Rounding kind of an output tensor's dtype for out_error."""
    return {torch.bfloat16: "bf16", torch.float16: "fp16"}.get(t.dtype, "fp32")


def assert_out_close(y, y_ref, bf16, what: str = "out", tol: float = OUT_TOL):
    exc, lit = out_error(y, y_ref, bf16)
    assert exc <= tol, f"{what}: error beyond output rounding {exc:.3e} x RMS > {tol} (literal {lit:.3e})"
    return exc, lit


def assert_state_close(s, s_ref, what: str = "state", tol: float = STATE_TOL):
    e = state_error(s, s_ref)
    assert e <= tol, f"{what}: relative Frobenius error {e:.3e} > {tol}"
    return e

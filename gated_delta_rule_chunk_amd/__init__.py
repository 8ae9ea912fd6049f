"""Python binding of libgdr.so, the gfx950 Gated Delta Rule library.

Argument marshalling only: every step of the operator runs in the HIP
kernels behind the C ABI of include/gdr.h.  PyTorch supplies device memory
(tensors) and the current HIP stream; nothing here computes.  If the
library is not built this module raises on first use -- there is no CPU
fallback.

Functions mirror the C entry points:
  chunk_prefill(...)                 gdr_chunk_prefill
  chunk_prefill_noalloc(...)         gdr_chunk_prefill_noalloc
  chunk_prefill_workspace_size(...)  gdr_chunk_prefill_workspace_size
  recurrent_decode(...)              gdr_recurrent_decode
Errors follow the decode page's exceptions section: shape and grouping
errors raise ValueError; dtype/device errors and backend failures raise
RuntimeError.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# GDR_LIBRARY may name another build of the same C ABI (the tests use it for
# a host-side sanitizer build of the validation layer); unset, the in-tree
# library is loaded.
LIB_PATH = os.environ.get("GDR_LIBRARY") or os.path.join(_HERE, "libgdr.so")

GDR_OK = 0
GDR_ERR_INVALID_ARGUMENT = 1
GDR_ERR_UNSUPPORTED = 2
GDR_ERR_DTYPE = 3
GDR_ERR_WORKSPACE = 4
GDR_ERR_HIP = 5
GDR_FP32 = 0
GDR_BF16 = 1
GDR_FP16 = 2

# Every symbol include/gdr.h declares, with its ctypes signature.
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
SIGNATURES = {
    "gdr_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "gdr_last_error": (ctypes.c_char_p, []),
    "gdr_version": (ctypes.c_int, []),
    "gdr_chunk_prefill_workspace_size": (ctypes.c_int, [_i64, _i32, _i32, _i32, _i32, _i32,
                                                        ctypes.POINTER(ctypes.c_size_t)]),
    "gdr_chunk_prefill": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                                         _i32, ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp, _vp, _vp,
                                         ctypes.c_size_t, _vp]),
    "gdr_chunk_prefill_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32,
                                                 _i32, _i32, ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp,
                                                 _vp, _vp]),
    "gdr_recurrent_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i32,
                                            _i32, _i32, _i32, _i32, _i32, ctypes.c_float,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp, _vp]),
    "gdr_timing_enable": (ctypes.c_int, [ctypes.c_int]),
    "gdr_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int32),
                                       _i32]),
    "gdr_timing_kernel_name": (ctypes.c_char_p, [_i32]),
    "gdr_mfma_peak_probe": (ctypes.c_int, [_i32, _i64, _vp, _i64, ctypes.POINTER(ctypes.c_double), _vp]),
    "gdr_slab_stream_probe": (ctypes.c_int, [_vp, _i32, _vp, _i32, _i32, _vp]),
}
# MFMA instruction of each probe kind (gdr_mfma_peak_probe)
PROBE_KINDS = ("f16_16x16x32", "bf16_16x16x32", "f16_16x16x16", "f32_16x16x4", "f16_32x32x16")
TIMING_KERNELS = 5

_lib = None


def lib():
    """The loaded libgdr.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run gated_delta_rule_chunk_amd.build.build()")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def check(status: int, what: str) -> None:
    """Map a gdr_status to the exception classes of the decode page."""
    if status == GDR_OK:
        return
    name = lib().gdr_status_string(status).decode()
    detail = lib().gdr_last_error().decode()
    msg = f"{what}: {name}: {detail}"
    if status == GDR_ERR_INVALID_ARGUMENT:
        raise ValueError(msg)
    raise RuntimeError(msg)


_DT = {torch.bfloat16: GDR_BF16, torch.float32: GDR_FP32, torch.float16: GDR_FP16}


def _act(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DT:
        raise RuntimeError(f"{name}: dtype {t.dtype} not supported (bfloat16, float16 or float32)")
    return _DT[t.dtype]


def _dev(tensors, device):
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda or t.device != device:
            raise RuntimeError(f"{name} must be on {device} (got {t.device})")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


RULES = {"gated_delta": 0, "delta": 1, "gated": 2, "linear": 3}


def _rule(rule, g, beta) -> int:
    if rule not in RULES:
        raise ValueError(f"rule must be one of {sorted(RULES)} (got {rule!r})")
    if rule in ("gated_delta", "gated") and g is None:
        raise ValueError(f"rule {rule} needs g")
    if rule in ("gated_delta", "delta") and beta is None:
        raise ValueError(f"rule {rule} needs beta")
    return RULES[rule]


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def timing_enable(on: bool = True, kernels=None) -> None:
    """Record hipEvents around the named kernels (every kernel if None; see gdr.h)."""
    if not on:
        mask = 0
    elif kernels is None:
        mask = -1
    else:
        names = [lib().gdr_timing_kernel_name(i).decode() for i in range(TIMING_KERNELS)]
        mask = 0
        for k in kernels:
            mask |= 1 << names.index(k)
    check(lib().gdr_timing_enable(mask), "gdr_timing_enable")


def timing_read() -> dict:
    """{kernel name: (summed ms, launches)} since the previous read."""
    ms = (ctypes.c_double * TIMING_KERNELS)()
    n = (ctypes.c_int32 * TIMING_KERNELS)()
    check(lib().gdr_timing_read(ms, n, TIMING_KERNELS), "gdr_timing_read")
    return {lib().gdr_timing_kernel_name(i).decode(): (ms[i], n[i]) for i in range(TIMING_KERNELS)}


def mfma_peak_probe(kind: str, iters: int, sink) -> float:
    """Enqueue one launch of the MFMA issue-rate probe (see gdr.h) on the
    current stream of sink's device; returns the launch's flop count.  sink
    is a float32 device tensor of at least CUs * 8 * 256 elements."""
    flops = ctypes.c_double(0.0)
    check(lib().gdr_mfma_peak_probe(PROBE_KINDS.index(kind), int(iters), sink.data_ptr(), sink.numel(),
                                    ctypes.byref(flops), _stream(sink.device)), "gdr_mfma_peak_probe")
    return float(flops.value)


def slab_stream_probe(pool, idx) -> None:
    """Enqueue the slab-stream probe (see gdr.h) on pool's current stream: the
    one-token decode's reads and in-place writes of pool[idx[b], h] for every
    row b and head h, without its arithmetic (2 * 32 KiB per in-range row and
    head).  pool is a bf16 or fp16 [slots, Nv, 128, 128] device tensor, idx
    int32 [B] on the same device."""
    if pool.dim() != 4 or tuple(pool.shape[2:]) != (128, 128) or pool.element_size() != 2:
        raise ValueError(f"pool must be a 16-bit [slots, Nv, 128, 128] tensor (got {tuple(pool.shape)}, {pool.dtype})")
    if idx.dtype != torch.int32 or idx.dim() != 1 or idx.device != pool.device:
        raise ValueError("idx must be an int32 [B] tensor on the pool's device")
    slots, Nv = pool.shape[0], pool.shape[1]
    check(lib().gdr_slab_stream_probe(pool.data_ptr(), slots, idx.data_ptr(), idx.numel(), Nv,
                                      _stream(pool.device)), "gdr_slab_stream_probe")


def chunk_prefill_workspace_size(T: int, B: int, Nqk: int, Nv: int, D: int = 128, gk: bool = False) -> int:
    n = ctypes.c_size_t(0)
    check(lib().gdr_chunk_prefill_workspace_size(T, B, Nqk, Nv, D, int(bool(gk)), ctypes.byref(n)),
          "gdr_chunk_prefill_workspace_size")
    return int(n.value)


def _prefill_checked(q, k, v, g, beta, cu_seqlens, state_in, out, state_out, rule, gk):
    """Shape, dtype and device checks shared by the prefill entry points;
    returns (sizes, rule code, act code, gk used, out, state_out)."""
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[0] != q.shape[0]:
        raise ValueError(f"q, k must be [T,Nqk,D] and v [T,Nv,D] (got {tuple(q.shape)}, "
                         f"{tuple(k.shape)}, {tuple(v.shape)})")
    T, Nqk, D = q.shape
    Nv = v.shape[1]
    if v.shape[2] != D:
        raise ValueError("v must have the head dimension of q")
    code = _rule(rule, g, beta)
    if (g is not None and g.shape != (T, Nv)) or (beta is not None and beta.shape != (T, Nv)):
        raise ValueError(f"g and beta must be [T, Nv] = [{T}, {Nv}]")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [B+1] with B >= 1")
    B = cu_seqlens.numel() - 1
    act = _act(q, "q")
    for name, t in (("k", k), ("v", v), ("beta", beta)):
        if t is not None and t.dtype != q.dtype:
            raise RuntimeError(f"{name} must have the dtype of q ({q.dtype}), got {t.dtype}")
    if g is not None and g.dtype != torch.float32:
        raise RuntimeError("g must be float32")
    if cu_seqlens.dtype != torch.int32:
        raise RuntimeError("cu_seqlens must be int32")
    if gk is not None:
        if gk.shape != (T, Nv, D) or gk.dtype != torch.float32:
            raise ValueError(f"gk must be [T,Nv,D] = [{T},{Nv},{D}] float32")
        if rule not in ("gated_delta", "gated"):
            gk = None
    if state_in is not None:
        if state_in.shape != (B, Nv, D, D):
            raise ValueError(f"state_in must be [B,Nv,D,D] = [{B},{Nv},{D},{D}]")
        if state_in.dtype != torch.float32:
            raise RuntimeError("state_in must be float32")
    device = q.device
    if out is None:
        out = torch.empty((T, Nv, D), dtype=q.dtype, device=device)
    if state_out is None:
        state_out = torch.empty((B, Nv, D, D), dtype=torch.float32, device=device)
    if out.shape != (T, Nv, D) or out.dtype != q.dtype:
        raise ValueError("out must be [T,Nv,D] of q's dtype")
    if state_out.shape != (B, Nv, D, D) or state_out.dtype != torch.float32:
        raise ValueError("state_out must be [B,Nv,D,D] float32")
    _dev(dict(q=q, k=k, v=v, g=g, gk=gk, beta=beta, cu_seqlens=cu_seqlens, state_in=state_in, out=out,
              state_out=state_out), device)
    return (T, B, Nqk, Nv, D), code, act, gk, out, state_out


def chunk_prefill(q, k, v, g, beta, cu_seqlens, scale, state_in=None, out=None, state_out=None,
                  workspace=None, rule="gated_delta", gk=None):
    """Chunked Gated Delta Rule prefill ("Qwen3Next Samples" page).

    q, k [T,Nqk,D]; v [T,Nv,D]; beta [T,Nv] (act dtype: bf16, fp16 or fp32);
    g [T,Nv] fp32; cu_seqlens [B+1] int32; state_in [B,Nv,D,D] fp32 or None;
    rule one of RULES (g may be None without a gate, beta without the delta
    term); gk [T,Nv,D] fp32 or None: the per-key gate (ignored by the rules
    without decay).
    Returns (out [T,Nv,D] act dtype, state_out [B,Nv,D,D] fp32).  `out`,
    `state_out` and `workspace` (uint8, >= chunk_prefill_workspace_size
    bytes) may be passed in to avoid allocations.
    """
    (T, B, Nqk, Nv, D), code, act, gk, out, state_out = _prefill_checked(
        q, k, v, g, beta, cu_seqlens, state_in, out, state_out, rule, gk)
    device = q.device
    nbytes = chunk_prefill_workspace_size(T, B, Nqk, Nv, D, gk is not None)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _dev(dict(workspace=workspace), device)
    check(lib().gdr_chunk_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gk), _ptr(beta), _ptr(state_in),
                                  _ptr(cu_seqlens), T, B, Nqk, Nv, D, float(scale), code, act, _ptr(out),
                                  _ptr(state_out), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(device)),
          "gdr_chunk_prefill")
    return out, state_out


def chunk_prefill_noalloc(q, k, v, g, beta, cu_seqlens, scale, state_in=None, out=None, state_out=None,
                          rule="gated_delta", gk=None):
    """gdr_chunk_prefill_noalloc: the prefill of chunk_prefill in the
    library's per-GPU scratch array, with no workspace (for callers that
    cannot allocate; sizes whose workspace exceeds the scratch raise
    RuntimeError).  Pass `out` and `state_out` to allocate nothing here
    either."""
    (T, B, Nqk, Nv, D), code, act, gk, out, state_out = _prefill_checked(
        q, k, v, g, beta, cu_seqlens, state_in, out, state_out, rule, gk)
    check(lib().gdr_chunk_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gk), _ptr(beta),
                                          _ptr(state_in), _ptr(cu_seqlens), T, B, Nqk, Nv, D, float(scale),
                                          code, act, _ptr(out), _ptr(state_out), _stream(q.device)),
          "gdr_chunk_prefill_noalloc")
    return out, state_out


def recurrent_decode(q, k, v, g, gk, beta, state_pool, ssm_state_indices, actual_seq_lengths,
                     scale=1.0, out=None, num_accepted_tokens=None, rule="gated_delta"):
    """Recurrent Gated Delta Rule decode over a slot pool
    ("lite_boost.ops.recurrent_gated_delta_rule" page).

    q, k [B,Nk,S,Dk]; v [B,Nv,S,Dv]; beta [B,Nv,S] (act dtype); g [B,Nv,S]
    fp32; gk [B,Nv,S,Dk] fp32 or None; state_pool [slots,Nv,Dk,Dv] (bf16 or
    fp32, updated in place); ssm_state_indices [B*S] int32;
    actual_seq_lengths [B] int32; num_accepted_tokens [B] int32 or None
    (speculative decoding: row b resumes from slot
    ssm_state_indices[b*S + n_b - 1]); rule one of RULES (g and gk may be
    None without a gate, beta without the delta term).  Returns
    (out [B,Nv,S,Dv], state_pool).
    """
    if q.dim() != 4 or k.shape != q.shape:
        raise ValueError(f"q and k must be [B,Nk,S,Dk] (got {tuple(q.shape)}, {tuple(k.shape)})")
    B, Nk, S, Dk = q.shape
    if v.dim() != 4 or v.shape[0] != B or v.shape[2] != S:
        raise ValueError(f"v must be [B,Nv,S,Dv] (got {tuple(v.shape)})")
    Nv, Dv = v.shape[1], v.shape[3]
    code = _rule(rule, g, beta)
    if (g is not None and g.shape != (B, Nv, S)) or (beta is not None and beta.shape != (B, Nv, S)):
        raise ValueError("g and beta must be [B, Nv, S]")
    if gk is not None and gk.shape != (B, Nv, S, Dk):
        raise ValueError("gk must be [B, Nv, S, Dk]")
    if state_pool.dim() != 4 or state_pool.shape[1:] != (Nv, Dk, Dv):
        raise ValueError(f"state_pool must be [slots,{Nv},{Dk},{Dv}] (got {tuple(state_pool.shape)})")
    if ssm_state_indices.numel() != B * S:
        raise ValueError(f"ssm_state_indices must hold B*S = {B * S} entries "
                         f"(got {ssm_state_indices.numel()})")
    if actual_seq_lengths.numel() != B:
        raise ValueError(f"actual_seq_lengths must hold B = {B} entries")
    if num_accepted_tokens is not None and num_accepted_tokens.numel() != B:
        raise ValueError(f"num_accepted_tokens must hold B = {B} entries")
    act = _act(q, "q")
    for name, t in (("k", k), ("v", v), ("beta", beta)):
        if t is not None and t.dtype != q.dtype:
            raise RuntimeError(f"{name} must have the dtype of q ({q.dtype}), got {t.dtype}")
    st = _act(state_pool, "state_pool")
    if (g is not None and g.dtype != torch.float32) or (gk is not None and gk.dtype != torch.float32):
        raise RuntimeError("g and gk must be float32")
    if ssm_state_indices.dtype != torch.int32 or actual_seq_lengths.dtype != torch.int32 or (
            num_accepted_tokens is not None and num_accepted_tokens.dtype != torch.int32):
        raise RuntimeError("ssm_state_indices, actual_seq_lengths and num_accepted_tokens must be int32")
    device = q.device
    if out is None:
        out = torch.empty((B, Nv, S, Dv), dtype=q.dtype, device=device)
    if out.shape != (B, Nv, S, Dv) or out.dtype != q.dtype:
        raise ValueError("out must be [B,Nv,S,Dv] of q's dtype")
    _dev(dict(q=q, k=k, v=v, g=g, gk=gk, beta=beta, state_pool=state_pool,
              ssm_state_indices=ssm_state_indices, actual_seq_lengths=actual_seq_lengths,
              num_accepted_tokens=num_accepted_tokens, out=out),
         device)
    check(lib().gdr_recurrent_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(gk), _ptr(beta),
                                     _ptr(state_pool), state_pool.shape[0], _ptr(ssm_state_indices),
                                     _ptr(actual_seq_lengths), _ptr(num_accepted_tokens), B, S, Nk, Nv,
                                     Dk, Dv, float(scale), code,
                                     act, st, _ptr(out), _stream(device)),
          "gdr_recurrent_decode")
    return out, state_pool

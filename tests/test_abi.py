"""C ABI checks that need no GPU: the library loads, exports every symbol
include/gdr.h declares, and rejects bad arguments on the host before any
HIP call (status codes mapped to ValueError / RuntimeError as the decode
page's exceptions section assigns them)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_chunk_amd as gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000   # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(os.path.join(ROOT, "include", "gdr.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(gdr.SIGNATURES), names
    lib = gdr.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    lib = gdr.lib()
    assert lib.gdr_status_string(0) == b"GDR_OK"
    assert lib.gdr_status_string(1) == b"GDR_ERR_INVALID_ARGUMENT"
    assert lib.gdr_status_string(5) == b"GDR_ERR_HIP"
    assert lib.gdr_status_string(99) == b"unknown status"
    assert lib.gdr_version() >= 200


def ws_size(T, B, Nqk, Nv, D, gk=0):
    n = ctypes.c_size_t(0)
    return gdr.lib().gdr_chunk_prefill_workspace_size(T, B, Nqk, Nv, D, gk, ctypes.byref(n)), n.value


def _one_level_workspace(T, B, Nqk, Nv):
    """Workspace bytes of the one-level scan: chunk map, k^T per qk head;
    w, u, g_cum and the (S_c, v_new) pair per value head; regions 256-aligned."""
    al = lambda x: (x + 255) // 256 * 256
    nc = (T + B * 127) // 128
    tile = 128 * 128 * 2
    return (al(4 * (B + 2)) + al(16 * nc) + al(tile * nc * Nqk) + 2 * al(tile * nc * Nv)
            + al(4 * 128 * nc * Nv) + al(2 * tile * nc * Nv))


def test_workspace_two_level_scan_only_for_few_long_streams():
    # many streams, or short sequences: one-level
    assert ws_size(8192, 4, 16, 32, 128)[1] == _one_level_workspace(8192, 4, 16, 32)
    assert ws_size(4096, 1, 1, 2, 128)[1] == _one_level_workspace(4096, 1, 1, 2)
    # 2 streams of 256 chunks: 32 segments of 8 chunks, each with a 128x256 fp32
    # map and a 128x128 fp32 start state per value head
    extra = ws_size(32768, 1, 1, 2, 128)[1] - _one_level_workspace(32768, 1, 1, 2)
    assert extra == 32 * 2 * 4 * 128 * (256 + 128)
    # 12 streams: segments of at least 8 chunks, at most 256 / (2 * 12) = 10 per sequence
    T = 25003
    extra = ws_size(T, 3, 1, 4, 128)[1] - _one_level_workspace(T, 3, 1, 4)
    assert extra == 3 * 10 * 4 * 4 * 128 * (256 + 128)
    # the shape of the GPU test of the two-level scan without an initial state
    assert ws_size(16700, 2, 1, 2, 128)[1] > _one_level_workspace(16700, 2, 1, 2)


def test_workspace_size_validation_and_monotonicity():
    assert ws_size(256, 1, 2, 4, 128)[0] == gdr.GDR_OK
    assert ws_size(256, 1, 3, 4, 128)[0] == gdr.GDR_ERR_INVALID_ARGUMENT   # Nv % Nqk
    assert ws_size(256, 1, 2, 4, 64)[0] == gdr.GDR_ERR_UNSUPPORTED         # D != 128
    assert ws_size(-1, 1, 2, 4, 128)[0] == gdr.GDR_ERR_INVALID_ARGUMENT
    assert ws_size(256, 0, 2, 4, 128)[0] == gdr.GDR_ERR_INVALID_ARGUMENT
    assert ws_size(2 ** 31, 1, 2, 4, 128)[0] == gdr.GDR_ERR_INVALID_ARGUMENT
    a = ws_size(8192, 4, 16, 32, 128)[1]
    b = ws_size(8192 + 128, 4, 16, 32, 128)[1]
    assert 0 < a < b
    # one 32 KiB tile per (chunk, head) and per intermediate (k^T per qk head;
    # w, u, v_new, S_c per value head), chunks <= (T + B*127) / 128
    nc = (8192 + 4 * 127) // 128
    assert a >= nc * 32768 * (16 + 4 * 32)
    with pytest.raises(ValueError):
        gdr.chunk_prefill_workspace_size(10, 1, 3, 4)


def prefill_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, gk=None, beta=FAKE, state_in=None, cu=FAKE, T=256, B=1, Nqk=2,
             Nv=4, D=128, scale=0.1, rule=0, act=gdr.GDR_BF16, out=FAKE, state_out=FAKE, ws=FAKE,
             ws_bytes=1 << 40, stream=None)
    a.update(over)
    return gdr.lib().gdr_chunk_prefill(a["q"], a["k"], a["v"], a["g"], a["gk"], a["beta"], a["state_in"], a["cu"],
                                       a["T"], a["B"], a["Nqk"], a["Nv"], a["D"], a["scale"], a["rule"],
                                       a["act"], a["out"], a["state_out"], a["ws"], a["ws_bytes"],
                                       a["stream"])


def test_prefill_host_validation():
    E = gdr
    assert prefill_call(Nqk=3) == E.GDR_ERR_INVALID_ARGUMENT
    assert prefill_call(B=0) == E.GDR_ERR_INVALID_ARGUMENT
    assert prefill_call(T=-5) == E.GDR_ERR_INVALID_ARGUMENT
    assert prefill_call(D=64) == E.GDR_ERR_UNSUPPORTED
    assert prefill_call(act=7) == E.GDR_ERR_DTYPE
    assert prefill_call(q=None) == E.GDR_ERR_INVALID_ARGUMENT
    assert prefill_call(cu=None) == E.GDR_ERR_INVALID_ARGUMENT
    assert prefill_call(state_out=None) == E.GDR_ERR_INVALID_ARGUMENT
    assert prefill_call(ws=None) == E.GDR_ERR_WORKSPACE
    assert prefill_call(ws_bytes=100) == E.GDR_ERR_WORKSPACE
    assert b"workspace" in gdr.lib().gdr_last_error()
    # update rules: unknown codes fail; g / beta may be NULL only where the rule ignores them
    assert prefill_call(rule=7) == E.GDR_ERR_INVALID_ARGUMENT
    assert prefill_call(g=None) == E.GDR_ERR_INVALID_ARGUMENT
    assert prefill_call(g=None, rule=1, ws=None) == E.GDR_ERR_WORKSPACE      # passes the pointer checks
    assert prefill_call(beta=None, rule=2, ws=None) == E.GDR_ERR_WORKSPACE
    assert prefill_call(g=None, beta=None, rule=3, ws=None) == E.GDR_ERR_WORKSPACE
    assert prefill_call(beta=None, rule=1) == E.GDR_ERR_INVALID_ARGUMENT
    assert prefill_call(g=None, rule=2) == E.GDR_ERR_INVALID_ARGUMENT
    # a per-key gate needs the larger workspace (queried with with_gk = 1); the
    # rules without decay ignore it
    plain = ws_size(256, 1, 2, 4, 128)[1]
    with_gk = ws_size(256, 1, 2, 4, 128, 1)[1]
    assert with_gk > plain
    assert prefill_call(gk=FAKE, ws_bytes=plain) == E.GDR_ERR_WORKSPACE
    assert b"per-key gate" in gdr.lib().gdr_last_error()
    assert prefill_call(gk=FAKE, ws=None) == E.GDR_ERR_WORKSPACE
    assert prefill_call(gk=FAKE, g=None, rule=1, ws_bytes=plain, ws=None) == E.GDR_ERR_WORKSPACE
    assert b"per-key gate" not in gdr.lib().gdr_last_error()


def decode_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, gk=None, beta=FAKE, pool=FAKE, slots=8, idx=FAKE,
             lens=FAKE, nacc=None, B=2, S=1, Nk=2, Nv=4, Dk=128, Dv=128, scale=0.1, rule=0, act=gdr.GDR_BF16,
             st=gdr.GDR_BF16, out=FAKE, stream=None)
    a.update(over)
    return gdr.lib().gdr_recurrent_decode(a["q"], a["k"], a["v"], a["g"], a["gk"], a["beta"], a["pool"],
                                          a["slots"], a["idx"], a["lens"], a["nacc"], a["B"], a["S"], a["Nk"],
                                          a["Nv"],
                                          a["Dk"], a["Dv"], a["scale"], a["rule"], a["act"], a["st"], a["out"],
                                          a["stream"])


def test_decode_host_validation():
    E = gdr
    assert decode_call(Nk=3) == E.GDR_ERR_INVALID_ARGUMENT       # Nv % Nk
    assert b"multiple of Nk" in gdr.lib().gdr_last_error()
    assert decode_call(S=0) == E.GDR_ERR_INVALID_ARGUMENT
    assert decode_call(S=9) == E.GDR_ERR_INVALID_ARGUMENT        # decode only, S <= 8
    assert decode_call(B=0) == E.GDR_ERR_INVALID_ARGUMENT
    assert decode_call(slots=0) == E.GDR_ERR_INVALID_ARGUMENT
    assert decode_call(Dk=96) == E.GDR_ERR_UNSUPPORTED
    assert decode_call(Dv=100) == E.GDR_ERR_UNSUPPORTED
    assert decode_call(act=3) == E.GDR_ERR_DTYPE
    assert decode_call(st=5) == E.GDR_ERR_DTYPE
    assert decode_call(idx=None) == E.GDR_ERR_INVALID_ARGUMENT
    assert decode_call(pool=None) == E.GDR_ERR_INVALID_ARGUMENT
    assert decode_call(rule=9) == E.GDR_ERR_INVALID_ARGUMENT
    assert decode_call(g=None) == E.GDR_ERR_INVALID_ARGUMENT
    assert decode_call(beta=None, rule=1) == E.GDR_ERR_INVALID_ARGUMENT
    assert decode_call(g=None, rule=2) == E.GDR_ERR_INVALID_ARGUMENT
    assert b"may be NULL" in gdr.lib().gdr_last_error()


def test_binding_maps_errors_to_exception_classes():
    with pytest.raises(ValueError):
        gdr.check(gdr.GDR_ERR_INVALID_ARGUMENT, "x")
    for s in (gdr.GDR_ERR_UNSUPPORTED, gdr.GDR_ERR_DTYPE, gdr.GDR_ERR_WORKSPACE, gdr.GDR_ERR_HIP):
        with pytest.raises(RuntimeError):
            gdr.check(s, "x")
    gdr.check(gdr.GDR_OK, "x")


def test_binding_shape_checks_precede_device_work():
    import torch
    q = torch.zeros(4, 2, 128, dtype=torch.bfloat16)
    v = torch.zeros(4, 3, 128, dtype=torch.bfloat16)
    g = torch.zeros(4, 3)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):   # g of the wrong shape
        gdr.chunk_prefill(q, q, v, torch.zeros(4, 2), g, cu, 0.1)
    with pytest.raises(ValueError):   # decode index count != B*S
        qd = torch.zeros(2, 1, 3, 64, dtype=torch.bfloat16)
        vd = torch.zeros(2, 1, 3, 64, dtype=torch.bfloat16)
        gd = torch.zeros(2, 1, 3)
        gdr.recurrent_decode(qd, qd, vd, gd, None, gd.bfloat16(), torch.zeros(4, 1, 64, 64),
                             torch.zeros(5, dtype=torch.int32), torch.ones(2, dtype=torch.int32))


def noalloc_call(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, gk=None, beta=FAKE, state_in=None, cu=FAKE, T=8192, B=4, Nqk=16,
             Nv=32, D=128, scale=0.1, rule=0, act=gdr.GDR_BF16, out=FAKE, state_out=FAKE, stream=None)
    a.update(over)
    return gdr.lib().gdr_chunk_prefill_noalloc(a["q"], a["k"], a["v"], a["g"], a["gk"], a["beta"],
                                               a["state_in"], a["cu"], a["T"], a["B"], a["Nqk"], a["Nv"],
                                               a["D"], a["scale"], a["rule"], a["act"], a["out"],
                                               a["state_out"], a["stream"])


def test_noalloc_prefill_rejects_sizes_beyond_its_scratch():
    """The allocation-free prefill checks every argument as gdr_chunk_prefill
    does, then the workspace these sizes need against its fixed scratch, all
    before any HIP call (none of these calls reaches a launch)."""
    E = gdr
    scratch = 128 << 20
    assert ws_size(8192, 4, 16, 32, 128)[1] > scratch
    assert noalloc_call() == E.GDR_ERR_WORKSPACE
    msg = gdr.lib().gdr_last_error()
    assert b"scratch" in msg and str(scratch).encode() in msg
    assert noalloc_call(Nqk=3) == E.GDR_ERR_INVALID_ARGUMENT
    assert noalloc_call(q=None) == E.GDR_ERR_INVALID_ARGUMENT
    assert noalloc_call(act=7) == E.GDR_ERR_DTYPE
    assert noalloc_call(D=64) == E.GDR_ERR_UNSUPPORTED
    # a workload that fits without a per-key gate can exceed it with one
    T = 3000
    assert ws_size(T, 1, 16, 32, 128)[1] <= scratch < ws_size(T, 1, 16, 32, 128, 1)[1]
    assert noalloc_call(T=T, B=1, gk=FAKE) == E.GDR_ERR_WORKSPACE
    assert b"per-key gate" in gdr.lib().gdr_last_error()


def test_mfma_probe_rejects_bad_arguments_before_any_hip_call():
    """The MFMA issue-rate probe checks its kind, iteration count and
    pointers on the host first (none of these calls reaches the device)."""
    lib = gdr.lib()
    flops = ctypes.c_double(0.0)
    E = gdr
    assert lib.gdr_mfma_peak_probe(5, 100, FAKE, 1 << 30, ctypes.byref(flops), None) == E.GDR_ERR_INVALID_ARGUMENT
    assert b"kind" in lib.gdr_last_error()
    assert lib.gdr_mfma_peak_probe(-1, 100, FAKE, 1 << 30, ctypes.byref(flops), None) == E.GDR_ERR_INVALID_ARGUMENT
    assert lib.gdr_mfma_peak_probe(0, 0, FAKE, 1 << 30, ctypes.byref(flops), None) == E.GDR_ERR_INVALID_ARGUMENT
    assert lib.gdr_mfma_peak_probe(0, (1 << 24) + 1, FAKE, 1 << 30, ctypes.byref(flops), None) == E.GDR_ERR_INVALID_ARGUMENT
    assert b"iterations" in lib.gdr_last_error()
    assert lib.gdr_mfma_peak_probe(0, 100, None, 1 << 30, ctypes.byref(flops), None) == E.GDR_ERR_INVALID_ARGUMENT
    assert lib.gdr_mfma_peak_probe(0, 100, FAKE, 1 << 30, None, None) == E.GDR_ERR_INVALID_ARGUMENT
    assert len(gdr.PROBE_KINDS) == 5


def test_slab_stream_probe_rejects_bad_arguments_before_any_hip_call():
    lib = gdr.lib()
    E = gdr
    assert lib.gdr_slab_stream_probe(None, 4, FAKE, 2, 2, None) == E.GDR_ERR_INVALID_ARGUMENT
    assert lib.gdr_slab_stream_probe(FAKE, 4, None, 2, 2, None) == E.GDR_ERR_INVALID_ARGUMENT
    assert lib.gdr_slab_stream_probe(FAKE, 4, FAKE, 0, 2, None) == E.GDR_ERR_INVALID_ARGUMENT
    assert lib.gdr_slab_stream_probe(FAKE, 0, FAKE, 2, 2, None) == E.GDR_ERR_INVALID_ARGUMENT
    assert b"num_slots" in lib.gdr_last_error()

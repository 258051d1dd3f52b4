"""The C-ABI library: it loads, exports every function the headers under
include/ declare, and rejects bad arguments before anything reaches a device (these
calls return from host-side validation, so they run without a GPU)."""
import ctypes
import os

import pytest

from quantized_moe_decode_route_amd import ops


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIB_PATH):
        from quantized_moe_decode_route_amd import build
        build.build()
    return ops.lib()


def test_exports_every_declared_function(lib):
    names = ops.header_functions()
    assert len(names) == 40
    for n in names:
        assert hasattr(lib, n), n


def test_stream_read_validation(lib):
    """moe_bench_stream_read rejects bad sizes and launch shapes on the host."""
    fake = ctypes.c_void_p(1 << 20)            # never dereferenced: validation fails first
    sink = ctypes.c_void_p(1 << 21)
    f = lib.moe_bench_stream_read
    assert f(None, 1024, sink, 1, 256, 8, None) == 1
    assert f(fake, 1000, sink, 1, 256, 8, None) == 1           # not a multiple of 16
    assert f(fake, 0, sink, 1, 256, 8, None) == 1
    assert f(ctypes.c_void_p((1 << 20) + 4), 1024, sink, 1, 256, 8, None) == 1   # misaligned
    assert f(fake, 1024, sink, 0, 256, 8, None) == 1
    assert f(fake, 1024, sink, 1, 384, 8, None) == 1
    assert f(fake, 1024, sink, 1, 256, 3, None) == 1
    assert f(fake, 1024, None, 1, 256, 8, None) == 1


def test_struct_layouts():
    assert ctypes.sizeof(ops._Experts) == 72
    assert ops._Experts.w_gate.offset == 24
    assert ctypes.sizeof(ops._Worklist) == 32


def test_status_strings(lib):
    assert lib.moedec_status_string(0) == b"ok"
    assert lib.moedec_status_string(1) == b"invalid argument"
    assert lib.moedec_status_string(99) == b"unknown status"
    assert lib.moedec_abi_version() == 2


FAKE = 1 << 20       # an aligned, never-dereferenced address


def _route(lib, **kw):
    a = dict(x=FAKE, w=FAKE, b=FAKE, T=1, H=256, E=16, G=4, TG=2, K=4, S=1, rsf=2.5,
             scores=FAKE, idx=FAKE, wts=FAKE, wl=None)
    a.update(kw)
    return lib.moe_route_topk(a["x"], a["w"], a["b"], a["T"], a["H"], a["E"], a["G"], a["TG"], a["K"], a["S"],
                              a["rsf"], a["scores"], a["idx"], a["wts"], a["wl"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(scores=None), 1), (dict(T=0), 1), (dict(H=250), 1), (dict(E=15), 1),
    (dict(G=16), 1),                       # one expert per group
    (dict(TG=5), 1), (dict(K=9), 1),       # more experts than two kept groups hold
    (dict(K=0), 1), (dict(S=-1), 1), (dict(rsf=float("nan")), 1), (dict(x=FAKE + 4), 1),
    (dict(T=65), 2), (dict(E=2048, G=8, TG=4), 2), (dict(K=33, E=256, G=1, TG=1), 2),
])
def test_route_rejects(lib, kw, status):
    assert _route(lib, **kw) == status


def _experts(**kw):
    d = dict(hidden=256, inter=128, n_experts=16, n_shared=1, bits=4,
             w_gate=FAKE, w_up=FAKE, w_down=FAKE, s_gate=FAKE, s_up=FAKE, s_down=FAKE)
    d.update(kw)
    return ops._Experts(**d)


def _wl(**kw):
    d = dict(n_active=FAKE, expert_id=FAKE, seg=FAKE, assign=FAKE)
    d.update(kw)
    return ops._Worklist(**d)


@pytest.mark.parametrize("suffix,bits", [("q4", 4), ("q8", 8), ("q2", 2)])
@pytest.mark.parametrize("kw,wkw,call,status", [
    (dict(bits=0), {}, {}, 1),                     # bits do not match the suffix
    (dict(w_up=None), {}, {}, 1),
    ({}, dict(seg=None), {}, 1),
    (dict(hidden=250), {}, {}, 1),                 # not a whole 16-byte group
    (dict(inter=100), {}, {}, 1),
    ({}, {}, dict(T=0), 1), ({}, {}, dict(K=0), 1), ({}, {}, dict(K=17), 1),
    (dict(w_down=FAKE + 8), {}, {}, 1),            # misaligned codes
    ({}, {}, dict(T=65), 2), (dict(hidden=32768), {}, {}, 2), (dict(n_shared=9), {}, {}, 2),
])
def test_expert_calls_reject(lib, suffix, bits, kw, wkw, call, status):
    if "bits" not in kw:
        kw = dict(kw, bits=bits)
    else:
        kw = dict(kw, bits=(bits + 1) if bits != 8 else 4)
    ex, wl = _experts(**kw), _wl(**wkw)
    T, K = call.get("T", 1), call.get("K", 4)
    gu = getattr(lib, f"moe_expert_gate_up_silu_{suffix}")
    dn = getattr(lib, f"moe_expert_down_combine_{suffix}")
    em = getattr(lib, f"moe_expert_down_combine_em_{suffix}")
    assert gu(FAKE, ctypes.byref(ex), ctypes.byref(wl), T, K, FAKE, None) == status
    assert dn(FAKE, ctypes.byref(ex), ctypes.byref(wl), FAKE, T, K, FAKE, None) == status
    assert em(FAKE, ctypes.byref(ex), ctypes.byref(wl), FAKE, FAKE, T, K, FAKE, FAKE, None) == status


def test_expert_calls_reject_null_structs(lib):
    assert lib.moe_expert_gate_up_silu_q4(FAKE, None, ctypes.byref(_wl()), 1, 4, FAKE, None) == 1
    assert lib.moe_expert_down_combine_q4(FAKE, ctypes.byref(_experts()), None, FAKE, 1, 4, FAKE, None) == 1
    assert lib.moe_expert_gate_up_silu_q4(None, ctypes.byref(_experts()), ctypes.byref(_wl()), 1, 4, FAKE, None) == 1
    em = lib.moe_expert_down_combine_em_q4
    ex, wl = ctypes.byref(_experts()), ctypes.byref(_wl())
    assert em(FAKE, ex, wl, FAKE, FAKE, 1, 4, None, FAKE, None) == 1        # no partial-output buffer
    assert em(FAKE, ex, wl, FAKE, FAKE, 1, 4, FAKE, None, None) == 1        # no y
    assert em(FAKE, None, wl, FAKE, FAKE, 1, 4, FAKE, FAKE, None) == 1
    assert em(FAKE + 4, ex, wl, FAKE, FAKE, 1, 4, FAKE, FAKE, None) == 1    # h not 16-byte aligned


def _fused(lib, suffix, ex, wl, **kw):
    a = dict(x=FAKE, w=FAKE, b=FAKE, T=1, G=4, TG=2, K=4, rsf=2.5, scores=FAKE, idx=FAKE, wts=FAKE,
             h=FAKE, y=FAKE, ws=FAKE)
    a.update(kw)
    fn = getattr(lib, f"moe_layer_fused_{suffix}")
    return fn(a["x"], a["w"], a["b"], ctypes.byref(ex) if ex else None, a["T"], a["G"], a["TG"], a["K"], a["rsf"],
              a["scores"], a["idx"], a["wts"], ctypes.byref(wl) if wl else None, a["h"], a["y"], a["ws"], None)


@pytest.mark.parametrize("suffix,bits", [("q4", 4), ("q8", 8), ("q2", 2)])
@pytest.mark.parametrize("ekw,kw,status", [
    ({}, dict(ws=None), 1), ({}, dict(ws=FAKE + 2), 1),          # workspace missing or misaligned
    ({}, dict(h=None), 1), ({}, dict(y=None), 1), ({}, dict(x=FAKE + 4), 1),
    ({}, dict(K=9), 1), ({}, dict(G=16), 1), ({}, dict(rsf=float("inf")), 1),
    (dict(bits=0), {}, 1),
    ({}, dict(T=17), 2),                                          # past the fused token limit
    (dict(n_experts=1024), dict(G=8, TG=4), 2),                   # past the fused expert limit
    ({}, dict(T=65), 2),
])
def test_fused_call_rejects(lib, suffix, bits, ekw, kw, status):
    ekw = dict(ekw, bits=ekw.get("bits", bits))
    assert _fused(lib, suffix, _experts(**ekw), _wl(), **kw) == status


@pytest.mark.parametrize("suffix", ["q4", "q8", "q2"])
def test_fused_resid_and_topp_reject(lib, suffix):
    import math
    ex, wl = _experts(bits=int(suffix[1:])), _wl()
    resid = getattr(lib, f"moe_layer_fused_resid_{suffix}")
    topp = getattr(lib, f"moe_layer_fused_topp_{suffix}")
    head = (FAKE, FAKE, FAKE, ctypes.byref(ex), 1, 4, 2, 4, 2.5)
    tail = (FAKE, FAKE, FAKE, ctypes.byref(wl), FAKE, FAKE, FAKE, None)
    assert resid(*head, 1.0, 1e-6, None, *tail) == 1                 # no x_out
    assert resid(*head, 1.0, -1.0, FAKE, *tail) == 1                 # negative eps
    assert resid(*head, 1.0, math.inf, FAKE, *tail) == 1
    assert resid(*head, math.nan, 1e-6, FAKE, *tail) == 1            # NaN top_p
    assert topp(*head, math.nan, *tail) == 1
    act8 = getattr(lib, f"moe_layer_fused_act8_{suffix}")
    assert act8(*head, math.nan, *tail) == 1                          # NaN top_p
    assert act8(FAKE, FAKE, FAKE, None, 1, 4, 2, 4, 2.5, 1.0, *tail) == 1   # no experts


def test_fused_call_requires_structs(lib):
    assert _fused(lib, "q4", None, _wl()) == 1
    assert _fused(lib, "q4", _experts(), None) == 1


@pytest.mark.parametrize("bits", [4, 8, 2])
def test_pack_validation(lib, bits):
    pk = getattr(lib, f"moe_pack_q{bits}")
    up = getattr(lib, f"moe_unpack_q{bits}")
    assert pk(FAKE, FAKE, -1, 8, None) == 1
    assert up(FAKE, FAKE, 2, -8, None) == 1
    assert pk(None, FAKE, 2, 8, None) == 1
    assert pk(None, None, 0, 8, None) == 0        # empty: nothing to do
    assert up(None, None, 4, 0, None) == 0
    if bits != 8:
        assert pk(FAKE, FAKE, 2, 8 // bits + 1, None) == 1   # row of a partial byte


@pytest.mark.parametrize("bits", [4, 8, 2])
@pytest.mark.parametrize("pack", [False, True])
def test_quantize_validation(lib, bits, pack):
    fn = getattr(lib, f"moe_quantize_pack_rows_q{bits}" if pack else f"moe_quantize_rows_q{bits}")
    assert fn(FAKE, FAKE, FAKE, -1, 8, None) == 1                 # negative sizes
    assert fn(FAKE, FAKE, FAKE, 2, -8, None) == 1
    assert fn(FAKE, FAKE, FAKE, 2, 6, None) == 1                  # row_len % 4
    assert fn(None, FAKE, FAKE, 2, 8, None) == 1                  # null pointers
    assert fn(FAKE, None, FAKE, 2, 8, None) == 1
    assert fn(FAKE, FAKE, None, 2, 8, None) == 1
    assert fn(FAKE + 4, FAKE, FAKE, 2, 8, None) == 1              # w not 16-byte aligned
    assert fn(FAKE, FAKE, FAKE + 2, 2, 8, None) == 1              # scales not 4-byte aligned
    if not pack or bits != 2:
        assert fn(FAKE, FAKE + 1, FAKE, 2, 8, None) == 1          # codes / packed words misaligned
    assert fn(None, None, None, 0, 8, None) == 0                  # no rows: nothing to do


def test_topp_rejects_nan(lib):
    import math
    args = (FAKE, FAKE, FAKE, 1, 256, 16, 4, 2, 4, 1, 2.5, math.nan, FAKE, FAKE, FAKE, None, None)
    assert lib.moe_route_topp(*args) == 1


def test_rmsnorm_validation(lib):
    assert lib.moe_residual_rmsnorm(None, None, FAKE, 1, 8, 1e-6, None) == 1
    assert lib.moe_residual_rmsnorm(FAKE, None, FAKE, 0, 8, 1e-6, None) == 1
    assert lib.moe_residual_rmsnorm(FAKE, None, FAKE, 1, 8, -1.0, None) == 1


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 256)
    with pytest.raises(ValueError):
        ops._dev(x, torch.float32, "x")


def test_binding_constants_match_the_header():
    """The binding's copies of the header's limits and workspace layout."""
    import re
    src = open(os.path.join(os.path.dirname(ops.__file__), "..", "include", "moedec.h")).read()
    defs = {m.group(1): int(m.group(2)) for m in re.finditer(r"#define\s+(MOEDEC_\w+)\s+(\d+)", src)}
    assert defs["MOEDEC_FUSED_WORKSPACE_INTS"] == ops.FUSED_WORKSPACE_INTS
    assert defs["MOEDEC_FUSED_WS_ERROR"] == ops.FUSED_WS_ERROR
    assert defs["MOEDEC_FUSED_MAX_TOKENS"] == ops.FUSED_MAX_TOKENS
    assert defs["MOEDEC_FUSED_MAX_EXPERTS"] == ops.FUSED_MAX_EXPERTS
    assert ops.FUSED_WS_GATES * ops.FUSED_WS_GATE_STRIDE <= ops.FUSED_WS_ERROR
    end = ops.PIPE_WS_BASE + ops.FUSED_WS_GATES * ops.PIPE_WS_STRIDE
    assert ops.FUSED_WS_ERROR < ops.PIPE_WS_BASE and end <= ops.FUSED_WORKSPACE_INTS

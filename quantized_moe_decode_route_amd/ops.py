"""Python binding of libmoedec: argument marshalling only.

Every function here checks that its torch tensors live on the GPU with the
dtype and layout the C ABI (include/moedec.h) expects, passes their device
pointers and the current HIP stream to the library, and raises MoedecError on
a non-zero status.  All arithmetic runs in the library's kernels; there is no
fallback: if libmoedec.so is missing, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoedec.so")
INCLUDE_DIR = os.path.join(os.path.dirname(_HERE), "include")
HEADER_PATH = os.path.join(INCLUDE_DIR, "moedec.h")

MAX_TOKENS = 64
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "device error"}


class MoedecError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


class _Experts(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p), ("s_down", ctypes.c_void_p)]


class _Worklist(ctypes.Structure):
    _fields_ = [("n_active", ctypes.c_void_p), ("expert_id", ctypes.c_void_p),
                ("seg", ctypes.c_void_p), ("assign", ctypes.c_void_p)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float

_SIGS = {
    "moedec_status_string": ([_I], ctypes.c_char_p),
    "moedec_abi_version": ([], _I),
    "moe_route_topk": ([_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P], _I),
    "moe_route_topp": ([_P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _P], _I),
    "moe_residual_rmsnorm": ([_P, _P, _P, _I, _I, _F, _P], _I),
    "moe_bench_stream_read": ([_P, _I64, _P, _I, _I, _I, _P], _I),
}
for _b in ("q4", "q8", "q2"):
    _SIGS[f"moe_expert_gate_up_silu_{_b}"] = ([_P, _P, _P, _I, _I, _P, _P], _I)
    _SIGS[f"moe_expert_down_combine_{_b}"] = ([_P, _P, _P, _P, _I, _I, _P, _P], _I)
    _SIGS[f"moe_expert_down_combine_em_{_b}"] = ([_P, _P, _P, _P, _P, _I, _I, _P, _P, _P], _I)
    _SIGS[f"moe_pack_{_b}"] = ([_P, _P, _I64, _I64, _P], _I)
    _SIGS[f"moe_unpack_{_b}"] = ([_P, _P, _I64, _I64, _P], _I)
    _SIGS[f"moe_quantize_rows_{_b}"] = ([_P, _P, _P, _I64, _I64, _P], _I)
    _SIGS[f"moe_quantize_pack_rows_{_b}"] = ([_P, _P, _P, _I64, _I64, _P], _I)
    _SIGS[f"moe_layer_fused_{_b}"] = ([_P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _P, _P, _P, _P, _P, _P, _P], _I)
    _SIGS[f"moe_layer_fused_topp_{_b}"] = ([_P, _P, _P, _P, _I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _P, _P, _P, _P],
                                           _I)
    _SIGS[f"moe_layer_fused_act8_{_b}"] = ([_P, _P, _P, _P, _I, _I, _I, _I, _F, _F, _P, _P, _P, _P, _P, _P, _P, _P],
                                           _I)
    _SIGS[f"moe_layer_fused_resid_{_b}"] = ([_P, _P, _P, _P, _I, _I, _I, _I, _F, _F, _F, _P, _P, _P, _P, _P, _P, _P,
                                             _P, _P], _I)
_SIGS["moe_expert_down_combine_em_noalloc_q4"] = ([_P, _P, _P, _P, _P, _I, _I, _P, _P], _I)

MOEDEC_ERR_UNSUPPORTED = 2
MOEDEC_ERR_DEVICE = 3

# batches from which the separate calls use the expert-major down (each
# workgroup stages only the h of the experts it streams)
DOWN_EM_MIN_TOKENS = 8

# limits of the fused layer call (include/moedec.h)
FUSED_MAX_TOKENS = 16
FUSED_MAX_EXPERTS = 512
FUSED_WORKSPACE_INTS = 4096
FUSED_WS_ERROR = 512            # workspace word: a wait timed out
FUSED_WS_GATES, FUSED_WS_GATE_STRIDE = 8, 64   # arrival counters (int64) every 64 int32 words
# the plain / top-p / residual fused calls: the scores exchange's counters
# (int64) at words PIPE_WS_BASE + i * PIPE_WS_STRIDE, i < FUSED_WS_GATES
PIPE_WS_BASE = 1024
PIPE_WS_STRIDE = 32            # words between a gate's counters


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m quantized_moe_decode_route_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def header_functions() -> list[str]:
    """Names of the functions the headers under include/ declare."""
    names = set()
    for name in sorted(os.listdir(INCLUDE_DIR)):
        if name.endswith(".h"):
            with open(os.path.join(INCLUDE_DIR, name)) as f:
                text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
            names |= set(re.findall(r"\b((?:moe|moedec)_\w+)\s*\(", text))
    return sorted(names)


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoedecError(fn, status, lib().moedec_status_string(status).decode())


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


# ------------------------------------------------------------------- types

@dataclass
class Worklist:
    """Batch union written by route_topk (device tensors, see moedec_worklist)."""
    n_active: torch.Tensor   # int32 [1]
    expert_id: torch.Tensor  # int32 [max_active]
    seg: torch.Tensor        # int32 [max_active + 1]
    assign: torch.Tensor     # int32 [T * (K + S)]

    @staticmethod
    def empty(T: int, top_k: int, n_experts: int, n_shared: int, device) -> "Worklist":
        max_active = min(n_experts, T * top_k) + n_shared
        z = dict(dtype=torch.int32, device=device)
        return Worklist(torch.zeros(1, **z), torch.zeros(max_active, **z), torch.zeros(max_active + 1, **z),
                        torch.zeros(T * (top_k + n_shared), **z))

    def struct(self) -> _Worklist:
        return _Worklist(_dev(self.n_active, torch.int32, "n_active"),
                         _dev(self.expert_id, torch.int32, "expert_id"),
                         _dev(self.seg, torch.int32, "seg"), _dev(self.assign, torch.int32, "assign"))


@dataclass
class Experts:
    """One layer's experts as device tensors (see moedec_experts)."""
    q_gate: torch.Tensor   # uint8 [(E+S), I, H*bits/8]
    q_up: torch.Tensor     # uint8 [(E+S), I, H*bits/8]
    q_down: torch.Tensor   # uint8 [(E+S), H, I*bits/8]
    s_gate: torch.Tensor   # fp32 [(E+S), I]
    s_up: torch.Tensor     # fp32 [(E+S), I]
    s_down: torch.Tensor   # fp32 [(E+S), H]
    n_experts: int
    n_shared: int
    bits: int

    @property
    def hidden(self) -> int:
        return self.q_down.shape[1]

    @property
    def inter(self) -> int:
        return self.q_gate.shape[1]

    def struct(self) -> _Experts:
        n = self.n_experts + self.n_shared
        H, I, b = self.hidden, self.inter, self.bits
        shapes = {"q_gate": (n, I, H * b // 8), "q_up": (n, I, H * b // 8), "q_down": (n, H, I * b // 8),
                  "s_gate": (n, I), "s_up": (n, I), "s_down": (n, H)}
        for k, shp in shapes.items():
            if tuple(getattr(self, k).shape) != shp:
                raise ValueError(f"{k} has shape {tuple(getattr(self, k).shape)}, expected {shp}")
        return _Experts(H, I, self.n_experts, self.n_shared, b,
                        _dev(self.q_gate, torch.uint8, "q_gate"), _dev(self.q_up, torch.uint8, "q_up"),
                        _dev(self.q_down, torch.uint8, "q_down"), _dev(self.s_gate, torch.float32, "s_gate"),
                        _dev(self.s_up, torch.float32, "s_up"), _dev(self.s_down, torch.float32, "s_down"))

    @staticmethod
    def from_layer(layer: dict, n_experts: int, n_shared: int, bits: int) -> "Experts":
        return Experts(layer["q_gate"], layer["q_up"], layer["q_down"], layer["s_gate"], layer["s_up"],
                       layer["s_down"], n_experts, n_shared, bits)


@dataclass
class Route:
    scores: torch.Tensor     # fp32 [T, E]
    topk_idx: torch.Tensor   # int32 [T, K]
    topk_w: torch.Tensor     # fp32 [T, K]
    worklist: Worklist


# ------------------------------------------------------------------- calls

def route_topk(x: torch.Tensor, router_w: torch.Tensor, bias: torch.Tensor, *, n_group: int, topk_group: int,
               top_k: int, n_shared: int, rsf: float, out: Route | None = None, top_p: float | None = None) -> Route:
    """moe_route_topk: sigmoid scores, group-limited top-k, weights, worklist
    (moe_route_topp when top_p is given: adaptive expert top-p after top-k)."""
    T, H = x.shape
    E = router_w.shape[0]
    if router_w.shape != (E, H) or bias.shape != (E,):
        raise ValueError("router_w must be [E, H] and bias [E]")
    if out is None:
        dev = x.device
        out = Route(torch.empty((T, E), dtype=torch.float32, device=dev),
                    torch.empty((T, top_k), dtype=torch.int32, device=dev),
                    torch.empty((T, top_k), dtype=torch.float32, device=dev),
                    Worklist.empty(T, top_k, E, n_shared, dev))
    wl = out.worklist.struct()
    head = (_dev(x, torch.float32, "x"), _dev(router_w, torch.float32, "router_w"), _dev(bias, torch.float32, "bias"),
            T, H, E, n_group, topk_group, top_k, n_shared, float(rsf))
    tail = (_dev(out.scores, torch.float32, "scores"), _dev(out.topk_idx, torch.int32, "topk_idx"),
            _dev(out.topk_w, torch.float32, "topk_w"), ctypes.byref(wl), _stream(x))
    if top_p is None:
        _check("moe_route_topk", lib().moe_route_topk(*head, *tail))
    else:
        _check("moe_route_topp", lib().moe_route_topp(*head, float(top_p), *tail))
    return out


def _suffix(bits: int) -> str:
    if bits not in (4, 8, 2):
        raise ValueError("bits must be 4, 8 or 2")
    return f"q{bits}"


def gate_up_silu(x: torch.Tensor, ex: Experts, wl: Worklist, top_k: int, out: torch.Tensor | None = None):
    """moe_expert_gate_up_silu_q{bits}: h[a] = silu(Wg x_t) * (Wu x_t) per assignment a."""
    T = x.shape[0]
    A = T * (top_k + ex.n_shared)
    if out is None:
        out = torch.empty((A, ex.inter), dtype=torch.float32, device=x.device)
    if out.shape != (A, ex.inter):
        raise ValueError("h must be [T*(K+S), I]")
    s_ex, s_wl = ex.struct(), wl.struct()
    fn = getattr(lib(), f"moe_expert_gate_up_silu_{_suffix(ex.bits)}")
    st = fn(_dev(x, torch.float32, "x"), ctypes.byref(s_ex), ctypes.byref(s_wl), T, top_k,
            _dev(out, torch.float32, "h"), _stream(x))
    _check(fn.__name__, st)
    return out


def down_combine(h: torch.Tensor, ex: Experts, wl: Worklist, topk_w: torch.Tensor, top_k: int,
                 out: torch.Tensor | None = None, part: torch.Tensor | None = None,
                 topk_idx: torch.Tensor | None = None):
    """moe_expert_down_combine_q{bits}: y[t] = sum_k w[t,k] o(t,k) + sum_shared o.
    With part (fp32 [T*(top_k+S), hidden] scratch): the expert-major form,
    moe_expert_down_combine_em_q{bits} (topk_idx: skip top-p's dropped slots)."""
    T = topk_w.shape[0]
    if out is None:
        out = torch.empty((T, ex.hidden), dtype=torch.float32, device=h.device)
    if out.shape != (T, ex.hidden) or h.shape != (T * (top_k + ex.n_shared), ex.inter):
        raise ValueError("shape mismatch between h, topk_w and y")
    s_ex, s_wl = ex.struct(), wl.struct()
    if part is not None:
        if part.shape != (T * (top_k + ex.n_shared), ex.hidden):
            raise ValueError("part must be [T*(top_k+S), hidden]")
        name = f"moe_expert_down_combine_em_{_suffix(ex.bits)}"
        idx = _dev(topk_idx, torch.int32, "topk_idx") if topk_idx is not None else None
        st = getattr(lib(), name)(_dev(h, torch.float32, "h"), ctypes.byref(s_ex), ctypes.byref(s_wl),
                                  _dev(topk_w, torch.float32, "topk_w"), idx, T, top_k,
                                  _dev(part, torch.float32, "part"), _dev(out, torch.float32, "y"), _stream(h))
        _check(name, st)
        return out
    fn = getattr(lib(), f"moe_expert_down_combine_{_suffix(ex.bits)}")
    st = fn(_dev(h, torch.float32, "h"), ctypes.byref(s_ex), ctypes.byref(s_wl),
            _dev(topk_w, torch.float32, "topk_w"), T, top_k, _dev(out, torch.float32, "y"), _stream(h))
    _check(fn.__name__, st)
    return out


NOALLOC_PART_FLOATS = 1 << 20   # the static partial-output array of the no-allocation down call


def down_combine_noalloc(h: torch.Tensor, ex: Experts, wl: Worklist, topk_w: torch.Tensor, top_k: int,
                         out: torch.Tensor, topk_idx: torch.Tensor | None = None) -> torch.Tensor:
    """moe_expert_down_combine_em_noalloc_q4: the expert-major down call with
    its partial outputs in the library's static per-GPU array (int4 experts;
    T*(top_k+S)*hidden <= NOALLOC_PART_FLOATS; calls on one GPU must not
    overlap).  Allocates nothing: out must be given."""
    T = topk_w.shape[0]
    if ex.bits != 4:
        raise ValueError("the no-allocation down call takes int4 experts")
    if out.shape != (T, ex.hidden) or h.shape != (T * (top_k + ex.n_shared), ex.inter):
        raise ValueError("shape mismatch between h, topk_w and y")
    s_ex, s_wl = ex.struct(), wl.struct()
    idx = _dev(topk_idx, torch.int32, "topk_idx") if topk_idx is not None else None
    name = "moe_expert_down_combine_em_noalloc_q4"
    st = getattr(lib(), name)(_dev(h, torch.float32, "h"), ctypes.byref(s_ex), ctypes.byref(s_wl),
                              _dev(topk_w, torch.float32, "topk_w"), idx, T, top_k, _dev(out, torch.float32, "y"),
                              _stream(h))
    _check(name, st)
    return out


def pack(codes: torch.Tensor, bits: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """moe_pack_q{bits}: int8 codes [rows, n] -> uint8 [rows, n*bits/8]."""
    rows, n = codes.shape
    if out is None:
        out = torch.empty((rows, n * bits // 8), dtype=torch.uint8, device=codes.device)
    fn = getattr(lib(), f"moe_pack_{_suffix(bits)}")
    st = fn(_dev(codes, torch.int8, "codes"), _dev(out, torch.uint8, "packed"), rows, n, _stream(codes))
    _check(fn.__name__, st)
    return out


def unpack(packed: torch.Tensor, bits: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """moe_unpack_q{bits}: uint8 [rows, nb] -> int8 codes [rows, nb*8/bits]."""
    rows, nb = packed.shape
    n = nb * 8 // bits
    if out is None:
        out = torch.empty((rows, n), dtype=torch.int8, device=packed.device)
    fn = getattr(lib(), f"moe_unpack_{_suffix(bits)}")
    st = fn(_dev(packed, torch.uint8, "packed"), _dev(out, torch.int8, "codes"), rows, n, _stream(packed))
    _check(fn.__name__, st)
    return out


def quantize_rows(w: torch.Tensor, bits: int, pack: bool = False, out: torch.Tensor | None = None,
                  scales: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """moe_quantize_rows_q{bits} (pack=False: int8 codes [rows, n]) or
    moe_quantize_pack_rows_q{bits} (pack=True: uint8 [rows, n*bits/8]) from
    fp32 rows [rows, n]; returns (codes or packed, fp32 scales [rows])."""
    rows, n = w.shape
    if out is None:
        out = (torch.empty((rows, n * bits // 8), dtype=torch.uint8, device=w.device) if pack
               else torch.empty((rows, n), dtype=torch.int8, device=w.device))
    if scales is None:
        scales = torch.empty(rows, dtype=torch.float32, device=w.device)
    name = f"moe_quantize_pack_rows_{_suffix(bits)}" if pack else f"moe_quantize_rows_{_suffix(bits)}"
    fn = getattr(lib(), name)
    st = fn(_dev(w, torch.float32, "w"), _dev(out, torch.uint8 if pack else torch.int8, "out"),
            _dev(scales, torch.float32, "scales"), rows, n, _stream(w))
    _check(name, st)
    return out, scales


def stream_read(buf: torch.Tensor, sink: torch.Tensor, grid: int, threads: int = 512, unroll: int = 8,
                nbytes: int | None = None) -> None:
    """moe_bench_stream_read: a plain streaming read of buf (a measurement
    aid, not part of the path); sink: uint32 [grid * threads]."""
    nb = buf.numel() * buf.element_size() if nbytes is None else nbytes
    if not buf.is_cuda or not buf.is_contiguous() or nb > buf.numel() * buf.element_size():
        raise ValueError("buf must be a contiguous GPU tensor holding nbytes")
    if sink.numel() < grid * threads:
        raise ValueError("sink must hold grid * threads words")
    st = lib().moe_bench_stream_read(buf.data_ptr(), nb, _dev(sink, torch.int32, "sink"), grid, threads, unroll,
                                     _stream(buf))
    _check("moe_bench_stream_read", st)


def residual_rmsnorm(x: torch.Tensor, y: torch.Tensor | None, xn: torch.Tensor, eps: float = 1e-6) -> None:
    """moe_residual_rmsnorm: x += y (if given), xn = x / sqrt(mean(x^2) + eps)."""
    T, H = x.shape
    yp = _dev(y, torch.float32, "y") if y is not None else None
    st = lib().moe_residual_rmsnorm(_dev(x, torch.float32, "x"), yp, _dev(xn, torch.float32, "xn"), T, H,
                                    float(eps), _stream(x))
    _check("moe_residual_rmsnorm", st)


# ------------------------------------------------------------- a whole layer

@dataclass
class LayerBuffers:
    """Every intermediate of one layer call, allocated once and reused; the
    workspace (zeroed here, once) holds the fused launch's barrier state."""
    route: Route
    h: torch.Tensor
    y: torch.Tensor
    workspace: torch.Tensor   # int32 [FUSED_WORKSPACE_INTS]
    part: torch.Tensor | None = None   # fp32 [T*(K+S), H]: the expert-major down's partial outputs

    @staticmethod
    def allocate(T: int, H: int, I: int, E: int, top_k: int, n_shared: int, device) -> "LayerBuffers":
        f = dict(dtype=torch.float32, device=device)
        route = Route(torch.empty((T, E), **f), torch.empty((T, top_k), dtype=torch.int32, device=device),
                      torch.empty((T, top_k), **f), Worklist.empty(T, top_k, E, n_shared, device))
        part = torch.empty((T * (top_k + n_shared), H), **f) if T >= DOWN_EM_MIN_TOKENS else None
        return LayerBuffers(route, torch.empty((T * (top_k + n_shared), I), **f), torch.empty((T, H), **f),
                            torch.zeros(FUSED_WORKSPACE_INTS, dtype=torch.int32, device=device), part)

    def fused_error(self) -> bool:
        """True if a fused launch's wait timed out (synchronises).  While the
        word is set, the outputs of the launch that set it are invalid."""
        return bool(self.workspace[FUSED_WS_ERROR].item() != 0)

    def check_fused(self, name: str = "moe_layer_fused") -> None:
        """Raise if a fused launch on this workspace timed out (synchronises);
        the workspace is zeroed again first, so the next launch starts clean."""
        if self.fused_error():
            self.workspace.zero_()
            raise MoedecError(name, MOEDEC_ERR_DEVICE, "a grid-wide wait of the fused launch timed out (not every "
                              "workgroup was resident at once: the GPU is shared); its outputs are invalid")


def fused_arrivals(workspace: torch.Tensor) -> int:
    """Arrivals the int8-activation fused call counted in a workspace so far:
    the sum of its counters (synchronises).  Each launch adds two per workgroup."""
    c = workspace[:FUSED_WS_GATES * FUSED_WS_GATE_STRIDE].view(torch.int64)[::FUSED_WS_GATE_STRIDE // 2]
    return int(c.sum().item())


def pipe_arrivals(workspace: torch.Tensor) -> int:
    """Arrivals the plain / top-p / residual fused calls counted on a
    workspace's scores exchange so far, one per workgroup per launch
    (synchronises)."""
    c = workspace[PIPE_WS_BASE:PIPE_WS_BASE + FUSED_WS_GATES * PIPE_WS_STRIDE].view(torch.int64)
    return int(c[::PIPE_WS_STRIDE // 2].sum().item())


def fused_supported(T: int, ex: Experts) -> bool:
    return T <= FUSED_MAX_TOKENS and ex.n_experts <= FUSED_MAX_EXPERTS


def layer_fused(x: torch.Tensor, router_w: torch.Tensor, bias: torch.Tensor, ex: Experts, *, n_group: int,
                topk_group: int, top_k: int, rsf: float, buf: LayerBuffers, top_p: float | None = None,
                x_out: torch.Tensor | None = None, eps: float = 1e-6, act8: bool = False,
                check: bool | None = None) -> LayerBuffers:
    """moe_layer_fused_q{bits} (moe_layer_fused_topp_q{bits} when top_p is
    given): the whole layer in one launch (outputs in buf).  With x_out:
    moe_layer_fused_resid_q{bits}, x_out = x + MoE(rmsnorm(x)) (x_out may be x).
    act8: moe_layer_fused_act8_q{bits} (Q8_0-style int8 activations).

    The launch needs every workgroup resident at once; if the GPU is shared
    and a grid-wide wait times out, the launch ends with invalid outputs and
    raises the workspace's error word.  check=True synchronises after the
    launch and raises MoedecError if the word is set (zeroing the workspace);
    check=None (the default) does so unless the stream is being captured into
    a graph; check=False leaves it to the caller (buf.check_fused())."""
    T, H = x.shape
    E = ex.n_experts
    if router_w.shape != (E, H) or bias.shape != (E,) or H != ex.hidden:
        raise ValueError("router_w must be [E, H], bias [E], x [T, hidden]")
    r = buf.route
    if r.scores.shape != (T, E) or r.topk_idx.shape != (T, top_k) or buf.y.shape != (T, H) or \
            buf.h.shape != (T * (top_k + ex.n_shared), ex.inter) or buf.workspace.numel() < FUSED_WORKSPACE_INTS:
        raise ValueError("buffers do not match the call's shapes")
    s_ex, s_wl = ex.struct(), r.worklist.struct()
    if act8:
        if x_out is not None:
            raise ValueError("the int8-activation call has no residual form")
        name = f"moe_layer_fused_act8_{_suffix(ex.bits)}"
        pre = (float(rsf), 1.0 if top_p is None else float(top_p))
    elif x_out is not None:
        if x_out.shape != (T, H):
            raise ValueError("x_out must be [T, hidden]")
        name = f"moe_layer_fused_resid_{_suffix(ex.bits)}"
        pre = (float(rsf), 1.0 if top_p is None else float(top_p), float(eps), _dev(x_out, torch.float32, "x_out"))
    elif top_p is None:
        name, pre = f"moe_layer_fused_{_suffix(ex.bits)}", (float(rsf),)
    else:
        name, pre = f"moe_layer_fused_topp_{_suffix(ex.bits)}", (float(rsf), float(top_p))
    fn = getattr(lib(), name)
    st = fn(_dev(x, torch.float32, "x"), _dev(router_w, torch.float32, "router_w"), _dev(bias, torch.float32, "bias"),
            ctypes.byref(s_ex), T, n_group, topk_group, top_k, *pre,
            _dev(r.scores, torch.float32, "scores"), _dev(r.topk_idx, torch.int32, "topk_idx"),
            _dev(r.topk_w, torch.float32, "topk_w"), ctypes.byref(s_wl), _dev(buf.h, torch.float32, "h"),
            _dev(buf.y, torch.float32, "y"), _dev(buf.workspace, torch.int32, "workspace"), _stream(x))
    _check(name, st)
    if check or (check is None and not torch.cuda.is_current_stream_capturing()):
        buf.check_fused(name)
    return buf


def moe_layer(x: torch.Tensor, router_w: torch.Tensor, bias: torch.Tensor, ex: Experts, *, n_group: int,
              topk_group: int, top_k: int, rsf: float, buf: LayerBuffers | None = None,
              fused: bool | None = None, top_p: float | None = None, act8: bool = False,
              check: bool | None = None) -> LayerBuffers:
    """One layer on x's stream; returns the buffers (y in .y).  fused=None takes
    the single-launch path where its limits allow, else route_topk ->
    gate_up_silu -> down_combine; True / False force one of them.  check: as
    for layer_fused (the fused path's timed-out waits)."""
    T = x.shape[0]
    if buf is None:
        buf = LayerBuffers.allocate(T, ex.hidden, ex.inter, ex.n_experts, top_k, ex.n_shared, x.device)
    if act8:                        # only the fused call has int8 activations
        return layer_fused(x, router_w, bias, ex, n_group=n_group, topk_group=topk_group, top_k=top_k, rsf=rsf,
                           buf=buf, top_p=top_p, act8=True, check=check)
    if fused is None:
        if fused_supported(T, ex):
            try:
                return layer_fused(x, router_w, bias, ex, n_group=n_group, topk_group=topk_group, top_k=top_k,
                                   rsf=rsf, buf=buf, top_p=top_p, check=check)
            except MoedecError as err:
                if err.status != MOEDEC_ERR_UNSUPPORTED:   # the shape does not fit the fused plan
                    raise
    elif fused:
        return layer_fused(x, router_w, bias, ex, n_group=n_group, topk_group=topk_group, top_k=top_k, rsf=rsf,
                           buf=buf, top_p=top_p, check=check)
    route_topk(x, router_w, bias, n_group=n_group, topk_group=topk_group, top_k=top_k, n_shared=ex.n_shared,
               rsf=rsf, out=buf.route, top_p=top_p)
    gate_up_silu(x, ex, buf.route.worklist, top_k, out=buf.h)
    down_combine(buf.h, ex, buf.route.worklist, buf.route.topk_w, top_k, out=buf.y, part=buf.part,
                 topk_idx=buf.route.topk_idx if buf.part is not None else None)
    return buf


def stack_forward(x: torch.Tensor, layers: list, bufs: list, *, n_group: int, topk_group: int, top_k: int,
                  rsf: float, eps: float = 1e-6, top_p: float | None = None, fused: bool | None = None,
                  xn: torch.Tensor | None = None, check: bool | None = None) -> bool:
    """x <- x + MoE_l(rmsnorm(x)) for every layer l, in place on x (the
    pre-norm residual stack).  layers[l] = (router_w, bias, Experts); bufs[l]
    a LayerBuffers.  Fused: one moe_layer_fused_resid launch per layer (the
    norm and the residual inside it); else the separate calls with
    moe_residual_rmsnorm between them (xn: a [T, H] scratch for the normalised
    tokens).  fused=None tries the fused form on the first layer and keeps
    whichever runs; returns whether the fused form ran.

    A fused layer whose grid-wide wait timed out writes an invalid x for every
    later layer; check=True (or None outside graph capture) synchronises once
    after the last layer and raises MoedecError if any layer's workspace
    reports it (zeroing those workspaces)."""
    T, H = x.shape
    kw = dict(n_group=n_group, topk_group=topk_group, top_k=top_k, rsf=rsf)
    if check is None:
        check = not torch.cuda.is_current_stream_capturing()

    def run_fused(items) -> None:
        for (rw, b, ex), buf in items:
            layer_fused(x, rw, b, ex, buf=buf, top_p=top_p, x_out=x, eps=eps, check=False, **kw)

    def finish() -> bool:
        if check:
            bad = [buf for buf in bufs if buf.fused_error()]
            for buf in bad:
                buf.workspace.zero_()
            if bad:
                raise MoedecError("moe_layer_fused_resid", MOEDEC_ERR_DEVICE,
                                  f"{len(bad)} layer(s) timed out in a grid-wide wait; x is invalid")
        return True

    if fused is None:
        fused = fused_supported(T, layers[0][2])
        if fused:
            try:
                run_fused(list(zip(layers, bufs))[:1])
            except MoedecError as err:
                if err.status != MOEDEC_ERR_UNSUPPORTED:
                    raise
                fused = False
            else:
                run_fused(list(zip(layers, bufs))[1:])
                return finish()
    if fused:
        run_fused(list(zip(layers, bufs)))
        return finish()
    if xn is None:
        xn = torch.empty_like(x)
    residual_rmsnorm(x, None, xn, eps)
    for (rw, b, ex), buf in zip(layers, bufs):
        moe_layer(xn, rw, b, ex, buf=buf, fused=False, top_p=top_p, **kw)
        residual_rmsnorm(x, buf.y, xn, eps)
    return False

"""ctypes wrapper of moe_ref.c, the plain-C CPU implementation of the layer
(TEST INFRASTRUCTURE: tests, the smoke entry and the benchmark's CPU-baseline
leg only).  build() compiles it with gcc; layer() runs it.  Nothing here
imports the NumPy oracle or the HIP package.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_ref.c")
LIB = os.path.join(HERE, "libmoe_ref.so")
CC = os.environ.get("CC", "gcc")

_lib = None


def build() -> str:
    """Compile libmoe_ref.so (OpenMP, -O2, no fast-math) next to its source."""
    tmp = LIB + ".tmp"
    subprocess.run([CC, "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, SRC, "-lm"],
                   check=True, capture_output=True, text=True)
    os.replace(tmp, LIB)
    return LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        h = ctypes.CDLL(LIB)
        P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        h.moe_ref_layer.argtypes = [P, I, I, I, I, I, I, I, I, F, I, P, P, P, P, P, P, P, P, I, P, P, P, P, P]
        h.moe_ref_layer.restype = I
        h.moe_ref_max_threads.argtypes = []
        h.moe_ref_max_threads.restype = I
        _lib = h
    return _lib


def max_threads() -> int:
    return int(lib().moe_ref_max_threads())


class Result:
    def __init__(self, scores64, idx, w, h, y):
        self.scores64, self.idx, self.w, self.h, self.y = scores64, idx, w, h, y


def layer(x, router_w, bias, experts: dict, *, n_group: int, topk_group: int, top_k: int, n_shared: int, rsf: float,
          bits: int, threads: int = 1) -> Result:
    """One layer.  experts[e] = {q_gate, q_up, q_down, s_gate, s_up, s_down}
    for every expert a token may select (missing ones are passed as NULL; the
    call fails if a selected expert is missing)."""
    x = np.ascontiguousarray(x, np.float32)
    rw = np.ascontiguousarray(router_w, np.float32)
    b = np.ascontiguousarray(bias, np.float32)
    T, H = x.shape
    E = rw.shape[0]
    n_all = E + n_shared
    keep = []                                   # keeps the arrays alive during the call

    def ptrs(key, dtype):
        arr = (ctypes.c_void_p * n_all)()
        for e in range(n_all):
            if e in experts:
                a = np.ascontiguousarray(experts[e][key], dtype)
                keep.append(a)
                arr[e] = a.ctypes.data
        return arr

    first = experts[min(experts)]
    I = first["q_gate"].shape[0]
    qg, qu, qd = ptrs("q_gate", np.uint8), ptrs("q_up", np.uint8), ptrs("q_down", np.uint8)
    sg, su, sd = ptrs("s_gate", np.float32), ptrs("s_up", np.float32), ptrs("s_down", np.float32)
    slots = top_k + n_shared
    scores = np.zeros((T, E), np.float64)
    idx = np.zeros((T, top_k), np.int32)
    w = np.zeros((T, top_k), np.float32)
    h = np.zeros((T * slots, I), np.float64)
    y = np.zeros((T, H), np.float64)
    st = lib().moe_ref_layer(x.ctypes.data, T, H, I, E, n_group, topk_group, top_k, n_shared, float(rsf), bits,
                             rw.ctypes.data, b.ctypes.data, qg, qu, qd, sg, su, sd, int(threads),
                             scores.ctypes.data, idx.ctypes.data, w.ctypes.data, h.ctypes.data, y.ctypes.data)
    if st != 0:
        raise RuntimeError(f"moe_ref_layer failed with status {st}")
    return Result(scores, idx, w, h, y)

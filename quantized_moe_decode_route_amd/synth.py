"""Seeded synthetic inputs for the routed-MoE decode step.

This module only draws inputs: it holds none of the method's arithmetic (no
routing, no packing rule, no dequantisation, no FFN).  Both sides of every
parity check take their inputs from here: the CPU oracle (through the tests)
and the HIP library (through the tests and the benchmark).

Value distributions (the same for every workload):
  activations x ~ N(0, 1) fp32; router weight ~ N(0, 0.05) fp32;
  correction bias ~ U(-0.1, 0.1) fp32 (the 16-layer stack: Zipf, see below);
  weight codes = uniform random bytes, so every 8/4/2-bit field is uniform over
  its codes; per-row scales ~ U(0.005, 0.02) fp32; routed scaling factor 2.5.

Streams.  Every tensor has its own stream keyed by (seed, layer, kind, expert,
bits), so one expert of one layer can be regenerated alone:
  * code bytes come from SplitMix64 (Steele, Lea & Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014; the 64-bit finaliser with the
    golden-gamma counter), a counter-based generator that is cheap to evaluate
    both with numpy on the host and with torch int64 arithmetic on a device,
    bit-identically (little-endian bytes of each 64-bit output);
  * everything else (normals, uniforms, permutations) comes from numpy's PCG64
    seeded with the same key, on the host only, and is uploaded.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Callable

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

# stream kinds
K_ROUTER, K_BIAS, K_TOKENS, K_GATE, K_UP, K_DOWN, K_SGATE, K_SUP, K_SDOWN, K_ZIPF, K_FLOATW = range(11)
_CODE_KIND = {"gate": K_GATE, "up": K_UP, "down": K_DOWN}
_SCALE_KIND = {"gate": K_SGATE, "up": K_SUP, "down": K_SDOWN}


@dataclass(frozen=True)
class MoEConfig:
    """Shapes of one routed-MoE layer workload.

    tokens T, hidden H, expert intermediate I, routed experts E in n_group
    groups of which topk_group are kept, top_k experts per token, n_shared
    always-on experts, bits per weight code, layers in the stack.
    """
    name: str
    tokens: int
    hidden: int
    inter: int
    n_experts: int
    n_group: int
    topk_group: int
    top_k: int
    n_shared: int
    bits: int
    layers: int = 1
    rsf: float = 2.5
    seed: int = 0
    token_mix: float | None = None   # correlation of later tokens with token 0
    zipf_s: float | None = None      # Zipf exponent of the correction bias
    pool: int = 64                   # token pool rotated through by the benchmark

    @property
    def slots(self) -> int:
        """Assignments per token: routed slots plus shared slots."""
        return self.top_k + self.n_shared

    def row_bytes(self, in_dim: int) -> int:
        return in_dim * self.bits // 8

    def expert_bytes(self) -> int:
        """Packed codes of gate, up and down plus one fp32 scale per output row."""
        H, I = self.hidden, self.inter
        return 2 * I * self.row_bytes(H) + H * self.row_bytes(I) + 4 * (2 * I + H)


CONFIGS: dict[str, MoEConfig] = {
    # tiny layer checked element by element
    "tiny": MoEConfig("tiny", 1, 256, 128, 16, 4, 2, 4, 1, 4, seed=0),
    # GLM-5.2-shaped layer, one decode token
    "glm_t1": MoEConfig("glm_t1", 1, 6144, 2048, 256, 8, 4, 8, 1, 4, seed=1),
    # the same layer verifying one accepted and two draft tokens together
    "glm_t3": MoEConfig("glm_t3", 3, 6144, 2048, 256, 8, 4, 8, 1, 4, seed=2, token_mix=0.45),
    # precision sweep on the same layer
    "glm_t1_q8": MoEConfig("glm_t1_q8", 1, 6144, 2048, 256, 8, 4, 8, 1, 8, seed=3),
    "glm_t1_q2": MoEConfig("glm_t1_q2", 1, 6144, 2048, 256, 8, 4, 8, 1, 2, seed=3),
    # 16 consecutive layers, 16 tokens, Zipf-skewed correction bias
    "glm_stack16": MoEConfig("glm_stack16", 16, 6144, 2048, 256, 8, 4, 8, 1, 4, layers=16,
                             seed=4, zipf_s=1.1),
}


def scaled(cfg: MoEConfig, **kw) -> MoEConfig:
    """A copy of cfg with some fields replaced (smaller parity cases)."""
    return replace(cfg, **kw)


# ---------------------------------------------------------------- stream keys

def _mix64(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def stream_key(seed: int, layer: int, kind: int, expert: int = 0, bits: int = 0) -> int:
    """64-bit key of one tensor's stream: fields folded in one at a time."""
    k = 0
    for f in (seed, layer, kind, expert, bits):
        k = _mix64(k ^ (((f + 1) * GAMMA) & MASK64))
    return k


def _pcg(key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(
        [key & 0xFFFFFFFF, key >> 32])))


# ------------------------------------------------------------- code bytes

def splitmix_bytes(key: int, nbytes: int) -> np.ndarray:
    """nbytes of the SplitMix64 stream `key` (host, numpy, in-place ops)."""
    n64 = (nbytes + 7) // 8
    z = np.arange(1, n64 + 1, dtype=np.uint64)
    z *= np.uint64(GAMMA)
    z += np.uint64(key)
    t = np.empty_like(z)
    np.right_shift(z, np.uint64(30), out=t); z ^= t; z *= np.uint64(MIX1)
    np.right_shift(z, np.uint64(27), out=t); z ^= t; z *= np.uint64(MIX2)
    np.right_shift(z, np.uint64(31), out=t); z ^= t
    return z.view(np.uint8)[:nbytes]


def _s64(c: int) -> int:
    """Two's-complement signed value of a 64-bit constant (torch has no uint64 math)."""
    return c - (1 << 64) if c >= 1 << 63 else c


def splitmix_bytes_torch(keys: list[int], nbytes: int, device) -> "torch.Tensor":
    """The same bytes as splitmix_bytes(keys[i], nbytes), for each key, as one
    uint8 tensor [len(keys), nbytes] on `device` (torch int64 wraps like uint64)."""
    import torch
    n64 = (nbytes + 7) // 8
    kt = torch.tensor([_s64(k) for k in keys], dtype=torch.int64, device=device)
    z = torch.arange(1, n64 + 1, dtype=torch.int64, device=device).unsqueeze(0) * _s64(GAMMA)
    z = z + kt.unsqueeze(1)

    def lsr(v, s):
        return (v >> s) & ((1 << (64 - s)) - 1)

    z = (z ^ lsr(z, 30)) * _s64(MIX1)
    z = (z ^ lsr(z, 27)) * _s64(MIX2)
    z = z ^ lsr(z, 31)
    return z.view(torch.uint8).view(len(keys), n64 * 8)[:, :nbytes]


# --------------------------------------------------------------- one layer

def matrix_shape(cfg: MoEConfig, which: str) -> tuple[int, int]:
    """(rows, packed row bytes) of one expert matrix: rows are output rows,
    packed along the input dimension."""
    if which in ("gate", "up"):
        return cfg.inter, cfg.row_bytes(cfg.hidden)
    return cfg.hidden, cfg.row_bytes(cfg.inter)


def expert_codes(cfg: MoEConfig, layer: int, expert: int, which: str) -> np.ndarray:
    rows, rb = matrix_shape(cfg, which)
    key = stream_key(cfg.seed, layer, _CODE_KIND[which], expert, cfg.bits)
    return splitmix_bytes(key, rows * rb).reshape(rows, rb)


def expert_scales(cfg: MoEConfig, layer: int, expert: int, which: str) -> np.ndarray:
    rows, _ = matrix_shape(cfg, which)
    g = _pcg(stream_key(cfg.seed, layer, _SCALE_KIND[which], expert, cfg.bits))
    return g.uniform(0.005, 0.02, size=rows).astype(np.float32)


def expert_arrays(cfg: MoEConfig, layer: int, expert: int) -> dict[str, np.ndarray]:
    """Packed codes and row scales of one expert (routed 0..E-1, shared E..E+S-1)."""
    out = {}
    for m in ("gate", "up", "down"):
        out["q_" + m] = expert_codes(cfg, layer, expert, m)
        out["s_" + m] = expert_scales(cfg, layer, expert, m)
    return out


def router_weight(cfg: MoEConfig, layer: int) -> np.ndarray:
    g = _pcg(stream_key(cfg.seed, layer, K_ROUTER))
    return (g.standard_normal((cfg.n_experts, cfg.hidden)) * 0.05).astype(np.float32)


def router_bias(cfg: MoEConfig, layer: int) -> np.ndarray:
    if cfg.zipf_s is not None:
        # Zipf-skewed: expert with random rank r gets 0.1 * r^-s
        g = _pcg(stream_key(cfg.seed, layer, K_ZIPF))
        rank = g.permutation(cfg.n_experts) + 1
        return (0.1 * rank.astype(np.float64) ** (-cfg.zipf_s)).astype(np.float32)
    g = _pcg(stream_key(cfg.seed, layer, K_BIAS))
    return g.uniform(-0.1, 0.1, size=cfg.n_experts).astype(np.float32)


def token_pool(cfg: MoEConfig, n: int | None = None) -> np.ndarray:
    """n token activations [n, H] fp32.  With token_mix c, token k of each
    batch of cfg.tokens is c*x0 + sqrt(1-c^2)*z_k, x0 being the batch's first
    token, so that the batch's tokens partly share their routed experts."""
    n = cfg.pool * cfg.tokens if n is None else n
    g = _pcg(stream_key(cfg.seed, 0, K_TOKENS))
    z = g.standard_normal((n, cfg.hidden))
    if cfg.token_mix is not None and cfg.tokens > 1:
        c = cfg.token_mix
        for b0 in range(0, n, cfg.tokens):
            for k in range(b0 + 1, min(b0 + cfg.tokens, n)):
                z[k] = c * z[b0] + np.sqrt(1.0 - c * c) * z[k]
    return z.astype(np.float32)


def batch_tokens(cfg: MoEConfig, step: int) -> np.ndarray:
    """The [T, H] batch the benchmark feeds at `step` (rotating over the pool)."""
    pool = token_pool(cfg)
    b = step % cfg.pool
    return pool[b * cfg.tokens:(b + 1) * cfg.tokens]


def expert_loader(cfg: MoEConfig, layer: int) -> Callable[[int], dict[str, np.ndarray]]:
    """Callable returning one expert's arrays on demand (host)."""
    return lambda e: expert_arrays(cfg, layer, e)


def layer_host(cfg: MoEConfig, layer: int = 0) -> dict[str, np.ndarray]:
    """Every tensor of one layer on the host (small configs only)."""
    n = cfg.n_experts + cfg.n_shared
    ex = [expert_arrays(cfg, layer, e) for e in range(n)]
    out = {"router_w": router_weight(cfg, layer), "bias": router_bias(cfg, layer)}
    for k in ex[0]:
        out[k] = np.stack([d[k] for d in ex])
    return out


def layer_device(cfg: MoEConfig, layer: int, device, chunk: int = 32) -> dict:
    """Every tensor of one layer as torch tensors on `device`; code bytes are
    generated on the device, the rest on the host and uploaded."""
    import torch
    n = cfg.n_experts + cfg.n_shared
    out = {"router_w": torch.from_numpy(router_weight(cfg, layer)).to(device),
           "bias": torch.from_numpy(router_bias(cfg, layer)).to(device)}
    for m in ("gate", "up", "down"):
        rows, rb = matrix_shape(cfg, m)
        q = torch.empty((n, rows, rb), dtype=torch.uint8, device=device)
        for e0 in range(0, n, chunk):
            e1 = min(n, e0 + chunk)
            keys = [stream_key(cfg.seed, layer, _CODE_KIND[m], e, cfg.bits) for e in range(e0, e1)]
            q[e0:e1] = splitmix_bytes_torch(keys, rows * rb, device).view(e1 - e0, rows, rb)
        out["q_" + m] = q
        s = np.stack([expert_scales(cfg, layer, e, m) for e in range(n)])
        out["s_" + m] = torch.from_numpy(s).to(device)
    return out


# ------------------------------------------------- float rows to quantise

def float_weight_rows(seed: int, rows: int, n: int, block: int = 128) -> np.ndarray:
    """fp32 rows standing in for a dequantised block-scaled checkpoint (the
    input of the row quantiser): N(0, 1) values times one magnitude per
    block x block tile, log-uniform over 1e-4 .. 1e-1, with every ninth row
    heavy-tailed (Student t, 3 degrees of freedom)."""
    rng = _pcg(stream_key(seed, 0, K_FLOATW, rows, n))
    w = rng.standard_normal((rows, n))
    heavy = np.arange(rows) % 9 == 4
    if heavy.any():
        w[heavy] = rng.standard_t(3, size=(int(heavy.sum()), n))
    tiles = 10.0 ** rng.uniform(-4.0, -1.0, size=((rows + block - 1) // block, (n + block - 1) // block))
    w *= np.repeat(np.repeat(tiles, block, axis=0), block, axis=1)[:rows, :n]
    return w.astype(np.float32)


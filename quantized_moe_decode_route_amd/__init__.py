"""Routed Mixture-of-Experts decode step (sigmoid noaux_tc group-limited top-k
router, SwiGLU experts on int8/int4/int2 row-scaled weights) on AMD Instinct
MI355X (gfx950).

The compute runs in the HIP library libmoedec.so (C ABI, include/moedec.h);
`quantized_moe_decode_route_amd.ops` is a thin binding over it that only
marshals torch tensors to device pointers.  Importing this package loads
nothing; the library is loaded on first use of `ops`.
"""
__all__ = ["ops", "synth"]

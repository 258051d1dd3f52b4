"""Build libmoedec.so (HIP, gfx950 only) in-tree with hipcc.

    python -m quantized_moe_decode_route_amd.build [--jobs N] [--asm]

Each csrc/*.hip is compiled to an object in _build/, then linked into
quantized_moe_decode_route_amd/libmoedec.so.  --asm also writes the gfx950
assembly of every object to _build/asm/ for inspection.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoedec.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-fvisibility=hidden",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions anywhere (device pass; the host pass ignores it)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{os.path.join(ROOT, 'include')}",
]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}): {os.path.basename(cmd[-1])}")
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if err and "warning" in err:
        sys.stderr.write(err + "\n")


def compile_one(src: str, asm: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src).replace(".hip", ".o"))
    _run([HIPCC, *FLAGS, "-c", "-o", obj, src])
    if asm:
        os.makedirs(os.path.join(BUILD, "asm"), exist_ok=True)
        out = os.path.join(BUILD, "asm", os.path.basename(src).replace(".hip", ".s"))
        _run([HIPCC, *FLAGS, "--cuda-device-only", "-S", "-o", out, src])
    return obj


def build(jobs: int = 4, asm: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: compile_one(s, asm), srcs))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    return LIB


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--asm", action="store_true")
    args = ap.parse_args()
    print(build(args.jobs, args.asm))


if __name__ == "__main__":
    main()

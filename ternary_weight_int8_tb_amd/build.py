"""Build libtb.so, the HIP library of this package, for gfx950 (in-tree)."""

from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "tb.hip")
PROBE_SRC = os.path.join(PKG, "csrc", "probe.hip")
PROBE_LIB = os.path.join(PKG, "libtb_probe.so")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libtb.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "--offload-arch=gfx950", "-std=c++17", "-fPIC", "-shared",
    # one IEEE rounding per fp32 operation: no fused multiply-add, correctly rounded division
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # leading scalar kernel arguments arrive preloaded in SGPRs (no kernel-argument fetch
    # before the first loads); the code object keeps a fallback for firmware without it
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _compile(src: str, out: str, extra: list[str] | None = None) -> str:
    cmd = [HIPCC, *FLAGS, *(extra or []), "-I", INCLUDE, src, "-o", out + ".tmp"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(out: str = LIB, extra: list[str] | None = None) -> str:
    """Build libtb.so (the path) and libtb_probe.so (benchmark probes)."""
    _compile(PROBE_SRC, PROBE_LIB)
    return _compile(SRC, out, extra)


if __name__ == "__main__":
    print(build())

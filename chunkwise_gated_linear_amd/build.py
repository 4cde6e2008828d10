"""Build libgla.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgla.so")
SOURCES = ["gla_kernels.hip", "gla_walk_bf16.hip", "gla_bwd.hip", "gla_wy.hip", "gla_host.hip"]
ARCH = os.environ.get("GLA_OFFLOAD_ARCH", "gfx950")


def _flags():
    """hipcc flags of every compilation of the sources, in two parts (the
    library build puts its own flags between them)."""
    head = [f"--offload-arch={ARCH}", "-O3", "-std=c++17"]
    tail = [
        # packed fp32 VALU forms are kept out of the generated code on purpose
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]
    return head, tail


def hipcc_command(out: str) -> list:
    head, tail = _flags()
    return (["hipcc"] + head + ["-fPIC", "-shared"] + tail + ["-o", out]
            + [os.path.join(CSRC, s) for s in SOURCES])


def device_asm_command(source: str, out: str) -> list:
    """The gfx950 assembly of one source file's device code, as the library builds it."""
    head, tail = _flags()
    return ["hipcc"] + head + tail + ["--cuda-device-only", "-S", "-o", out, os.path.join(CSRC, source)]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libgla.so")
    if verbose:
        msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                        if "packed-fp32-ops" not in l)
        if msg.strip():
            sys.stderr.write(msg + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

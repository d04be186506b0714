"""Build libqad.so (the HIP kernels + C-ABI) for gfx950 with hipcc, in-tree.

    python -m nvfp4_quantization_aware_amd.build

Flags: -ffp-contract=off keeps every multiply and add a separate IEEE
operation (the quantizer's arithmetic is specified operation by operation;
fused multiply-adds are written explicitly where intended); packed-fp32
instruction selection is disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libqad.so")
SOURCES = ["libqad.hip", "nvfp4_kernels.hip", "kl_kernels.hip", "linear.hip"]
LIBS = []
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-fno-fast-math", "-Wall", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + compile_flags() + ["-shared", "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES] + LIBS
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_test_pins(verbose: bool = False) -> list:
    """GPU check programs the test-suite runs (tests/pins/*.hip)."""
    pins = os.path.join(ROOT, "tests", "pins")
    out_dir = os.path.join(pins, "_build")
    os.makedirs(out_dir, exist_ok=True)
    outs = []
    for name in sorted(os.listdir(pins)):
        if not name.endswith(".hip"):
            continue
        out = os.path.join(out_dir, name[:-4])
        cmd = [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-ffp-contract=off", "-Xclang",
               "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", out, os.path.join(pins, name)]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        outs.append(out)
    return outs


def emit_asm(out_dir: str) -> list:
    """Device assembly of each kernel source (for reading the gfx950 code)."""
    os.makedirs(out_dir, exist_ok=True)
    outs = []
    for s in SOURCES[1:]:
        out = os.path.join(out_dir, s.replace(".hip", ".s"))
        subprocess.run([hipcc()] + compile_flags() + ["--cuda-device-only", "-S", "-o", out,
                                                      os.path.join(CSRC, s)], check=True)
        outs.append(out)
    return outs


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_test_pins(verbose=True))
    sys.exit(0)

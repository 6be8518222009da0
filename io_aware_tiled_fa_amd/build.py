"""Build libfa.so (the gfx950 HIP kernels and their C ABI) in-tree with hipcc.

    python -m io_aware_tiled_fa_amd.build [--asm DIR]

``--asm DIR`` also keeps the device assembly (for reading register use and
instruction schedules).
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build libfa.so)")
    return path


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep the compiler from forming packed fp32 VALU instructions
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # matrix-core accumulators in VGPRs: no AGPR <-> VGPR copies around
        # the softmax and the rescale of O
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        "-I", INCLUDE, "-I", CSRC,
    ]


def build(asm_dir: str | None = None, verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + flags() + srcs + ["-o", tmp]
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        cmd += ["-save-temps", "-Rpass-analysis=kernel-resource-usage"]
    cwd = asm_dir if asm_dir else None
    if asm_dir:
        cmd[cmd.index("-o") + 1] = os.path.abspath(tmp)
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    out = "\n".join(line for line in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", default=None, help="keep device assembly in this folder")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(args.asm, verbose=args.verbose or bool(args.asm))
    print(path)


if __name__ == "__main__":
    sys.exit(main())

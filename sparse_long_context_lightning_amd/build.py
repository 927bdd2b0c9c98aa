"""Build the HIP library libdsa.so in-tree for gfx950.

    python -m sparse_long_context_lightning_amd.build [--verbose]

Every source under csrc/ is compiled and linked in one hipcc invocation.  Packed-fp32 VALU
instructions are disabled for all device code.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libdsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results stay in VGPRs so the fused epilogues read them without accvgpr moves.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile libdsa.so and return its path.  Raises CalledProcessError on failure."""
    tmp_dir = tempfile.mkdtemp(prefix="dsa_build_")
    try:
        out = os.path.join(tmp_dir, "libdsa.so")
        cmd = [HIPCC, *FLAGS, *(extra_flags or []), "-o", out, *sources()]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
        if res.returncode != 0:
            sys.stderr.write(err + "\n")
            raise subprocess.CalledProcessError(res.returncode, cmd, res.stdout, res.stderr)
        if verbose and err.strip():
            sys.stderr.write(err + "\n")
        # Replace atomically so a process that has the old library mapped keeps working.
        tmp_final = LIB + ".tmp"
        shutil.copyfile(out, tmp_final)
        os.replace(tmp_final, LIB)
        return LIB
    finally:
        shutil.rmtree(tmp_dir, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))

"""Build the HIP libraries in-tree for gfx950.

    python -m sparse_long_context_lightning_amd.build [--verbose]

libdsa.so         the DSA path: every source under csrc/ (the C ABI of include/dsa.h)
libdsa_probes.so  the measurement probes under probes/ (include/dsa_probes.h), used by the
                  benchmark only

Each source is compiled to an object in parallel, then linked.  Packed-fp32 VALU instructions
are disabled for all device code.
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
PROBES = os.path.join(PKG, "probes")
LIB = os.path.join(PKG, "libdsa.so")
PROBES_LIB = os.path.join(PKG, "libdsa_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMPILE_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results stay in VGPRs so the fused epilogues read them without accvgpr moves.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]
LINK_FLAGS = ["--offload-arch=gfx950", "-shared", "-fPIC"]
# libdsa.so marks each library call as a roctx range (ROCm's marker library).
ROCTX_LIBS = ["-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx"]

_NOISE = "is not a recognized feature for this target"


def sources(folder=CSRC):
    return sorted(glob.glob(os.path.join(folder, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if _NOISE not in l)
    if res.returncode != 0:
        sys.stderr.write(err + "\n")
        raise subprocess.CalledProcessError(res.returncode, cmd, res.stdout, res.stderr)
    if verbose and err.strip():
        sys.stderr.write(err + "\n")


def _build_lib(srcs, dest, tmp_dir, verbose, extra_flags, jobs, libs=()):
    objs = [os.path.join(tmp_dir, os.path.basename(s) + ".o") for s in srcs]
    cmds = [[HIPCC, *COMPILE_FLAGS, *(extra_flags or []), "-c", "-o", o, s] for s, o in zip(srcs, objs)]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for f in [ex.submit(_run, c, verbose) for c in cmds]:
            f.result()
    out = os.path.join(tmp_dir, os.path.basename(dest))
    _run([HIPCC, *LINK_FLAGS, "-o", out, *objs, *libs], verbose)
    # Replace atomically so a process that has the old library mapped keeps working.
    tmp_final = dest + ".tmp"
    shutil.copyfile(out, tmp_final)
    os.replace(tmp_final, dest)
    return dest


def build(verbose: bool = False, extra_flags=None) -> str:
    """Compile libdsa.so and libdsa_probes.so; return the path of libdsa.so.  Raises
    CalledProcessError on failure."""
    jobs = max(1, min(8, os.cpu_count() or 1))
    tmp_dir = tempfile.mkdtemp(prefix="dsa_build_")
    try:
        _build_lib(sources(CSRC), LIB, tmp_dir, verbose, extra_flags, jobs, ROCTX_LIBS)
        _build_lib(sources(PROBES), PROBES_LIB, tmp_dir, verbose, extra_flags, jobs)
        return LIB
    finally:
        shutil.rmtree(tmp_dir, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))

"""Build libmla.so (the HIP kernels and their C ABI) for gfx950, in-tree.

Usage: python -m head_latent_attention_11_amd.build [-v]
Every .hip file under csrc/ is compiled with hipcc and linked into
head_latent_attention_11_amd/libmla.so.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmla.so")
BUILD = os.path.join(PKG, "_build")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]

# Per-file additions.  The small-row attention kernel rescales its matrix
# accumulators with vector instructions: keeping them in ordinary VGPRs
# (rather than the accumulation registers) avoids copying them back and
# forth on every tile.
FILE_FLAGS = {
    "decode_small.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libmla.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False, out_dir: str | None = None,
          host_flags: tuple = ()) -> str:
    """Compile every source and link the library; returns its path.

    out_dir: build folder and library location (default: in-tree libmla.so).
    host_flags: extra flags for the host side only (each passed as
    `-Xarch_host <flag>`, e.g. sanitizers); device code is unchanged."""
    hipcc = _hipcc()
    build_dir = BUILD if out_dir is None else os.path.join(out_dir, "_build")
    lib = LIB if out_dir is None else os.path.join(out_dir, "libmla.so")
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    objs = [os.path.join(build_dir, f[:-4] + ".o") for f in srcs]
    host = [a for f in host_flags for a in ("-Xarch_host", f)]

    def compile_one(args):
        src, obj = args
        _run([hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), *host, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)

    jobs = min(len(srcs), max(1, (os.cpu_count() or 4)), 16)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(compile_one, zip(srcs, objs)))
    tmp = lib + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *host, *objs, "-o", tmp], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

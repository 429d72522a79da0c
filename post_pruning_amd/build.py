"""Build libsg.so (the gfx950 SparseGPT layer solver) in-tree with hipcc."""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsg.so")
# machine-peak probes for the roofline figures (measurement only, its own library)
PEAKS_LIB = os.path.join(HERE, "libsg_peaks.so")
PEAKS_SOURCES = ["peaks.hip"]
BUILD = os.path.join(HERE, "_build")
SOURCES = ["api.hip", "hessian.hip", "factor.hip", "prune.hip", "sweep_plain.hip", "sweep_quant.hip",
           "sweep_joint.hip", "recon.hip", "export.hip"]

HIPCC_FLAGS = [
    "-std=c++17",
    "-O3",
    "--offload-arch=gfx950",
    "-fPIC",
    # keep the compiler from forming packed fp32 VALU ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]

# Per-source options.  The column sweep keeps its block tiles in registers and
# updates them with MFMAs between the column steps: with the MFMA operands in
# ordinary VGPRs there are no accumulator-register copies in that loop.
SOURCE_FLAGS = {s: ["-mllvm", "-amdgpu-mfma-vgpr-form"]
                for s in ("sweep_plain.hip", "sweep_quant.hip", "sweep_joint.hip")}
# The peak probes' MFMA chains: in accumulator registers the compiler shuffles
# the loop-carried tuples with accvgpr moves between the MFMAs; in VGPRs the
# loop is the eight MFMAs alone.
SOURCE_FLAGS["peaks.hip"] = ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [_hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    if verbose:
        sys.stderr.write(f"compiled {src}\n")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link libsg.so (and the peak
    probes' libsg_peaks.so) next to this file."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PEAKS_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PEAKS_SOURCES], PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))

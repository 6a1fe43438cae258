"""Build step: compiles libkvlr.so (and the synthetic-input helper library)
for gfx950 with hipcc, in-tree, next to the Python binding.

    python -m rank_compressed_kv_kvlr_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvlr.so")
SYNTH_SRC = os.path.join(ROOT, "synth", "csrc", "synth_gen.hip")
SYNTH_LIB = os.path.join(ROOT, "synth", "libkvlr_synth.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU forms are switched off for all device code.
COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Sources of libkvlr.so with their extra flags. The joint-value decode keeps its
# MFMA accumulators in ordinary VGPRs (its softmax rescales them between MFMAs), and
# so does the compression (its stores convert them straight from VGPRs).
SOURCES = {
    "api.hip": [],
    "decode.hip": [],
    "decode_joint.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "compress.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    return err


def _compile_all(objdir: str) -> tuple[list, str]:
    """Compiles every source to an object (in parallel); returns the objects and the log."""
    procs, objs = [], []
    for src, extra in SOURCES.items():
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        cmd = [HIPCC, *COMMON, *extra, "-fvisibility=hidden", "-c", "-o", obj, os.path.join(CSRC, src)]
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    log = ""
    for cmd, pr in procs:
        _, err = pr.communicate()
        err = "\n".join(l for l in err.splitlines() if "not a recognized feature" not in l)
        if pr.returncode != 0:
            raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
        log += err
    return objs, log


def build(verbose: bool = False) -> None:
    """Compile every HIP library of the repository (always recompiles)."""
    with tempfile.TemporaryDirectory(prefix="kvlr_build_") as objdir:
        objs, log = _compile_all(objdir)
        tmp = LIB + ".tmp"
        log += _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    tmp = SYNTH_LIB + ".tmp"
    log += _run([HIPCC, *COMMON, "-shared", "-ffp-contract=off", "-o", tmp, SYNTH_SRC])
    os.replace(tmp, SYNTH_LIB)
    if verbose and log.strip():
        print(log, file=sys.stderr)


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    print(SYNTH_LIB)

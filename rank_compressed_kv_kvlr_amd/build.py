"""Build step: compiles libkvlr.so (and the synthetic-input helper library)
for gfx950 with hipcc, in-tree, next to the Python binding.

    python -m rank_compressed_kv_kvlr_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libkvlr.so")
SYNTH_SRC = os.path.join(ROOT, "synth", "csrc", "synth_gen.hip")
SYNTH_LIB = os.path.join(ROOT, "synth", "libkvlr_synth.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU forms are switched off for all device code.
COMMON = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCES = ["api.hip", "decode.hip", "compress.hip"]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in res.stderr.splitlines() if "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False) -> None:
    """Compile every HIP library of the repository (always recompiles)."""
    tmp = LIB + ".tmp"
    log = _run([HIPCC, *COMMON, "-fvisibility=hidden", "-o", tmp, *[os.path.join(CSRC, s) for s in SOURCES]])
    os.replace(tmp, LIB)
    tmp = SYNTH_LIB + ".tmp"
    log += _run([HIPCC, *COMMON, "-ffp-contract=off", "-o", tmp, SYNTH_SRC])
    os.replace(tmp, SYNTH_LIB)
    if verbose and log.strip():
        print(log, file=sys.stderr)


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    print(SYNTH_LIB)

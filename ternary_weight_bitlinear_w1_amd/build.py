"""Build the gfx950 HIP library (libbitlinear.so) and the input generator (libsynth.so) in-tree.

    python -m ternary_weight_bitlinear_w1_amd.build [-v]
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libbitlinear.so")
SYNTH_LIB = os.path.join(HERE, "libsynth.so")

SOURCES = ["quant_acts.hip", "quant_weights.hip", "gemm_prefill.hip", "gemv_decode.hip", "decode_fused.hip", "base3.hip", "head.hip", "attention.hip", "noalloc.hip", "probes.hip", "api.cpp"]

# -ffp-contract=off: every fp operation rounds as written (no fused multiply-add).
# Division and sqrt stay correctly rounded. Packed-fp32 instructions are turned off.
HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"build step failed: {' '.join(cmd[:3])} ... ({r.returncode})")
    noise = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build_synth(verbose: bool = False) -> str:
    tmp = SYNTH_LIB + ".tmp"
    _run(["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-Wall", "-o", tmp,
          os.path.join(HERE, "synth.c"), "-lm", "-lpthread"], verbose)
    os.replace(tmp, SYNTH_LIB)
    return SYNTH_LIB


def build_hip(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmds.append(["hipcc", *HIPCC_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run(["hipcc", "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


def build(verbose: bool = False) -> None:
    build_synth(verbose)
    build_hip(verbose)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)

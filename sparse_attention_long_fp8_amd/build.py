"""Build libdsa.so, libdsa_proj.so (the hipBLASLt output projections) and the
test-only MFMA probe library for gfx950 with hipcc.

Usage: python -m sparse_attention_long_fp8_amd.build [-v]
The libraries are written next to this file, so they travel with the tree.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
INCLUDE = os.path.join(ROOT, "include")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 instructions are disabled: hipcc -O3 would otherwise emit them
# from ordinary float code.
COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC]

LIB_SOURCES = ["indexer.hip", "topk.hip", "sparse_mla.hip", "cache_append.hip", "module.hip", "validate.hip",
               "noalloc.hip", "libdsa.cpp", "module.cpp"]
# the output projections are plain GEMMs, run by hipBLASLt, in a library of
# their own (libdsa_proj.so) so that libdsa.so loads no GEMM library
PROJ_SOURCES = ["projection.cpp"]
PROJ_LINK = ["-L" + PKG, "-ldsa", "-Wl,-rpath,$ORIGIN", "-L/opt/rocm/lib", "-lhipblaslt", "-Wl,-rpath,/opt/rocm/lib"]

# Per-source flags.  The FP8 indexer reads every MFMA result with VALU code
# (ReLU, head weights); keeping the accumulators in ordinary VGPRs saves one
# AGPR->VGPR move per element.
# The rate probes keep their accumulators in VGPRs too: with AGPR accumulators
# the compiler rotates them through v_accvgpr moves inside the timed loops.
SOURCE_FLAGS = {"indexer.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
                "rates.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
PROBE_SOURCES = ["probe.hip", "rates.hip"]

LIB_PATH = os.path.join(PKG, "libdsa.so")
PROJ_PATH = os.path.join(PKG, "libdsa_proj.so")
PROBE_PATH = os.path.join(PKG, "libdsa_probe.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature: drop that note
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), err))
    if verbose and err.strip():
        print(err)


SCRATCH_LIMIT = 16  # bytes per lane


def _check_no_scratch(src, verbose):
    """Fail the build if a kernel keeps more than a few dwords in scratch
    memory.  A spilled or dynamically indexed register array (>= 128 bytes
    per lane here) costs far more than any of these kernels' arithmetic; a
    few spilled loop-invariant dwords outside the hot loops do not."""
    cmd = [HIPCC] + COMMON + SOURCE_FLAGS.get(src, []) + [
        "-x", "hip", "--cuda-device-only", "-c", os.path.join(CSRC, src), "-o", os.devnull,
        "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    fn, bad = None, []
    for line in r.stderr.splitlines():
        if "Function Name:" in line:
            fn = line.split("Function Name:")[1].split("[")[0].strip()
        elif "ScratchSize [bytes/lane]:" in line:
            n = int(line.split("ScratchSize [bytes/lane]:")[1].split("[")[0])
            if n > SCRATCH_LIMIT:
                bad.append("%s (%d bytes/lane)" % (fn, n))
    if bad:
        raise RuntimeError("%s: kernels spill to scratch memory: %s" % (src, ", ".join(bad)))


def _compile(src, verbose):
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    _run([HIPCC] + COMMON + SOURCE_FLAGS.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj], verbose)
    if src.endswith(".hip"):
        _check_no_scratch(src, verbose)
    return obj


def _link(objs, out, verbose, libs=()):
    tmp = out + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs + list(libs), verbose)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source and link the three libraries; returns libdsa.so's path."""
    srcs = LIB_SOURCES + PROJ_SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(min(len(srcs), 8)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in LIB_SOURCES], LIB_PATH, verbose)
    _link([objs[s] for s in PROJ_SOURCES], PROJ_PATH, verbose, PROJ_LINK)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build liblinattn.so (HIP, gfx950) in-tree with hipcc.

Every translation unit is compiled for gfx950 only, with packed-fp32 instruction
selection disabled, then linked into one shared library next to this file.
Usage: python -m chunked_causal_linear_k1_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "liblinattn.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["la_api.cpp", "la_decode.hip", "la_scan.hip", "la_prefill_bf16.hip", "la_prefill_f32.hip", "la_gla.hip",
           "la_backward.hip",
           "la_prefill_bf16_c64_d64.hip", "la_prefill_bf16_c64_d128.hip", "la_prefill_prf.hip", "la_noalloc.hip",
           "la_backward_prf.hip", "la_backward_gen.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -amdgpu-mfma-vgpr-form: MFMA accumulators in ordinary VGPRs. The fp32 states are also
# scaled and split by VALU code every chunk; with the accumulation-register form the compiler
# copied every state tile between the two register files around each MFMA chain.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=true",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


# The backward kernels keep two states and their operands live at once: with the VGPR form
# their accumulators would share the 256 architectural VGPRs with everything else (and this
# compiler's AGPR-copy rewrite pass crashes on them), so they keep the accumulation registers.
NO_VGPR_FORM = {"la_backward.hip"}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    flags = COMMON
    if src in NO_VGPR_FORM:  # drop "-mllvm -amdgpu-mfma-vgpr-form=true"
        i = COMMON.index("-amdgpu-mfma-vgpr-form=true")
        flags = COMMON[:i - 1] + COMMON[i + 1:]
    cmd = [HIPCC] + flags + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


PROBE_SRC = os.path.join(HERE, "probe", "stream_probe.hip")
PROBE_LIB = os.path.join(HERE, "libstreamprobe.so")


def build_probe(verbose: bool = True) -> str:
    """The streaming reference kernels bench.py times beside the prefill passes (a library of
    their own: measurement only, not part of liblinattn)."""
    tmp = PROBE_LIB + ".tmp"
    flags = [f for f in COMMON if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form=true")]
    cmd = [HIPCC] + flags + ["-shared", "-x", "hip", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 4)) as ex:
        probe = ex.submit(build_probe, verbose)
        objs = list(ex.map(_compile, SOURCES))
        probe.result()
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)

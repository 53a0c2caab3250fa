"""Build the HIP library in-tree: hipcc for gfx950 -> libstepdllm.so."""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = ["mask_kernels.hip", "attn_kernels.hip", "quality_kernels.hip", "col_kernels.hip",
           "api.hip", "noalloc.hip"]
LIB = os.path.join(PKG, "libstepdllm.so")
# Standalone measurement aids, not linked into the library: the sustained
# MFMA rate and shader clock, and the data-path rates (buffer->LDS fills, LDS
# reads, a step's traffic with its matrix products, streaming HBM reads).
PROBES = {"mfma_rate.hip": os.path.join(PKG, "mfma_rate"),
          "path_rates.hip": os.path.join(PKG, "path_rates")}
PROBE = PROBES["mfma_rate.hip"]
BUILD_DIR = os.path.join(PKG, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs: the online-softmax rescale of the output
    # accumulators is then plain VALU work instead of AGPR round trips.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src, extra):
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(extra_flags=(), verbose=False):
    """Compile every source for gfx950 and link the shared library."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra_flags)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    for src, exe in PROBES.items():
        cmd = [HIPCC, *FLAGS, *extra_flags, os.path.join(CSRC, src), "-o", exe + ".tmp"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        os.replace(exe + ".tmp", exe)
    if verbose:
        print("built", LIB, "and", ", ".join(PROBES.values()))
    return LIB


def clean():
    shutil.rmtree(BUILD_DIR, ignore_errors=True)


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:], verbose=True)

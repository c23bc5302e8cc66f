"""Build librfx.so (host encoder + HIP kernels for gfx950) in-tree.

    python -m bit_block_quantized_amd.build        # or build() from Python

Always compiles (it is the "does it build" check); the library lands next
to this file as librfx.so.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(HERE, "librfx.so")

SOURCES = ["rfx_host.cpp", "rfx_gemv.hip", "rfx_moe.hip", "rfx_moe_layer.hip", "rfx_prefill.hip", "rfx_probe.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # Packed fp32 VALU ops (v_pk_*_f32) stay off: scalar fp32 only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # IEEE-exact fp32 division and sqrt (the quantizers depend on it).
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # MFMA results in ordinary VGPRs (the epilogues read them with VALU ops;
    # accumulation registers would need a copy per element).
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-command-line-argument",
]

BUILD_DIR = os.path.join(ROOT, "_build")


def _compile(src: str, extra, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False, extra=()) -> str:
    """Compile every source (in parallel, one process each) and link."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    with ThreadPoolExecutor(len(srcs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, verbose), srcs))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])

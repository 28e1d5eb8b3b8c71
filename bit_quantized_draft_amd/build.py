"""Build the gfx950 shared library libsubspec.so in-tree with hipcc.

Usage: python -m bit_quantized_draft_amd.build   (or build() from Python)
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libsubspec.so")

SOURCES = ["gemm_w4.hip", "gemm_w4_tt1.hip", "gemm_w4_tt2.hip", "gemm_w4_tt3.hip", "gemm_w4_tt4.hip", "gemm_bf16.hip", "quant.hip", "attention.hip", "misc.hip", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # bit-exact float steps: no contraction, correctly rounded division, IEEE denormals
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # keep the compiler from emitting packed fp32 math
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + FLAGS + [f"-D{d}" for d in defines] + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = True, out: str = LIB, build_dir: str = BUILD, defines=()) -> str:
    """Compile every source and link libsubspec.so; always rebuilds.

    `defines` (e.g. ["SS_GEMM_PF=6"]) and `out` build a tuning variant elsewhere.
    """
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, defines), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


if __name__ == "__main__":
    build()

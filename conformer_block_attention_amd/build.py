"""Build libgsattn.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgsattn.so")

SOURCES = ["gsattn_api.hip", "gemm_bf16.hip", "gemm_pp_bf16.hip", "gemm_f32.hip", "attn_bf16.hip",
           "attn_f32.hip", "window_xattn.hip", "ctc_pool.hip"]

# Per-source code-generation options (none at present).
# The attention kernel never produces NaN from finite inputs; without NaN
# semantics its max reductions compile to plain v_max/v_max3 (no quieting of
# each operand first).
SOURCE_FLAGS: dict = {"attn_bf16.hip": ["-fno-honor-nans"]}

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # keep the compiler from forming packed-fp32 (v_pk_*_f32) instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _run(cmd, verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)


def build(out: str = LIB, verbose: bool = False) -> str:
    """Compile every source to an object (with its own options), then link."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        _run([hipcc(), *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), f"-I{INCLUDE}", f"-I{CSRC}",
              "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out + ".tmp"], verbose)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))

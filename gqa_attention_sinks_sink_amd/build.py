"""Build libattnsink.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m gqa_attention_sinks_sink_amd.build`` or ``build()`` from Python.
Objects go to ``_build/`` next to this file; the shared library lands beside this file
so that the Python binding and the tests load it from the source tree.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libattnsink.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "prefill.hip", "decode.hip", "merge.hip", "rope.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
        # packed FP32 instructions stay off: plain fp32 code only
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # keep MFMA accumulators in VGPRs: the softmax reads every score tile with VALU ops,
        # and AGPR-resident results would be copied back and forth on every tile
        "-mllvm", "-amdgpu-mfma-vgpr-form=1",
        "-I", os.path.join(ROOT, "include"), "-Wno-unused-result",
    ]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "is not a recognized feature for this target" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{msg}")
    if verbose and msg.strip():
        print(msg, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the shared library. Returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))

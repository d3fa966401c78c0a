"""Build libattn.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m tiled_exact_attention_flashattention_amd.build

The library's sources under csrc/ are compiled by hipcc for gfx950 only and
linked into ``libattn.so`` next to this file.  The benchmark's read-only
bandwidth probe (csrc/hbm_probe.hip) is linked on its own into
``libattn_probe.so``, which the library never loads.  Packed-FP32
instructions are disabled for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libattn.so")
PROBE_LIB_PATH = os.path.join(HERE, "libattn_probe.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

SOURCES = ["attn_api.cpp", "prefill_bf16.hip", "prefill_f32.hip", "decode_paged.hip",
           "backward_bf16.hip"]
PROBE_SOURCES = ["hbm_probe.hip"]

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    noise = "not a recognized feature for this target"
    for line in (res.stderr or "").splitlines():
        if line.strip() and noise not in line:
            print(f"[{src}] {line}", file=sys.stderr)
    return obj


def _link(objs, path):
    tmp = path + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, path)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(6, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB_PATH)
    _link(objs[len(SOURCES):], PROBE_LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH} and {PROBE_LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build()

"""Build libsparse_attn.so (the C ABI of include/sparse_attn.h) for gfx950 with hipcc.

Each translation unit is compiled separately into _build/ (in parallel), then
linked into sparse_attention_attn_amd/libsparse_attn.so next to this file.
No fast-math: the kernels rely on IEEE infinities and NaNs, and call expf.
Packed-fp32 instructions are disabled for every HIP file. The driver cannot hand
that -Xclang target feature to the device pass alone (-Xarch_device refuses options
that take an argument), so the host pass sees it too and prints that it ignores an
unknown feature; that one line is dropped from the compiler output, nothing else.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libsparse_attn.so")
SOURCES = ["sa_api.cpp", "sa_attn.hip", "sa_attn_split.hip", "sa_attn_f32.hip", "sa_attn_f32_split.hip", "sa_topk.hip",
           "sa_pad.hip", "sa_noalloc.hip", "sa_probe.hip"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}", "-fno-fast-math",
          "-Wno-unused-command-line-argument"]
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HOST_FEATURE_NOTICE = "'-packed-fp32-ops' is not a recognized feature for this target"


def _compile(src: str, save_temps: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [HIPCC, *COMMON, "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = HIP_FLAGS
        if save_temps:
            cmd += ["-save-temps=obj"]
    else:
        cmd += ["-D__HIP_PLATFORM_AMD__", "-x", "c++"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    for stream, text in ((sys.stdout, r.stdout), (sys.stderr, r.stderr)):
        lines = [ln for ln in text.splitlines(keepends=True) if HOST_FEATURE_NOTICE not in ln]
        stream.write("".join(lines))
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, cmd)
    return obj


def build(save_temps: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, save_temps), SOURCES))
    tmp = LIB + ".tmp"
    subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(save_temps="--save-temps" in sys.argv))

"""Build libbha.so (HIP, gfx950) in-tree.

    python -m linear_attention_block_amd.build

Every source under ``csrc/`` is compiled with hipcc for gfx950 only and linked
into ``linear_attention_block_amd/libbha.so``. Packed fp32 instructions are
disabled on the device side (``-packed-fp32-ops``); hipcc's host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libbha.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["bha_api.cpp", "bha_validate.cpp", "generic.hip", "mfma.hip", "softmax_attn.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libbha.so)")


def common_flags() -> list[str]:
    return [
        "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(HERE, "..", "include"),
    ]


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
                if "packed-fp32-ops" not in ln]
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(4, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

"""Build libbha.so (HIP, gfx950) in-tree.

    python -m linear_attention_block_amd.build

The library's sources under ``csrc/`` are compiled with hipcc for gfx950 only
and linked into ``linear_attention_block_amd/libbha.so``; the HBM streaming
probe (``csrc/stream_probe.hip``, interface ``include/bha_probe.h``) is linked
on its own into ``linear_attention_block_amd/libbha_probe.so``. Packed fp32 instructions are
disabled on the device side (``-packed-fp32-ops``); hipcc's host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libbha.so")
PROBE_OUT = os.path.join(HERE, "libbha_probe.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["bha_api.cpp", "bha_validate.cpp", "generic.hip", "softmax_attn.hip",
           # one translation unit per matrix-core kernel family (mfma_common.hpp)
           "mfma_forward.hip", "mfma_gqa.hip", "mfma_gqa8.hip", "mfma_commit.hip", "mfma_fused.hip",
           "mfma_prefill.hip", "mfma_feature_map.hip"]
PROBE_SOURCES = ["stream_probe.hip"]
HEADER = os.path.join(HERE, "..", "include", "bha.h")


def library_sources() -> list[str]:
    """Every file libbha.so is built from: its sources, the csrc headers and
    include/bha.h."""
    headers = sorted(f for f in os.listdir(CSRC) if f.endswith(".hpp"))
    return [os.path.join(CSRC, f) for f in SOURCES + headers] + [HEADER]


def source_hash() -> str:
    """First 16 hex digits of a SHA-256 over the library's source files (name
    and contents, in library_sources() order). Compiled into libbha.so
    (bha_source_hash), so a library can be matched with the sources on disk."""
    h = hashlib.sha256()
    for path in library_sources():
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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
    src_hash = source_hash()

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *common_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        if src == "bha_api.cpp":
            cmd.append(f'-DBHA_SOURCE_HASH="{src_hash}"')
        res = subprocess.run(cmd, capture_output=True, text=True)
        msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
                if "packed-fp32-ops" not in ln]
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
        if verbose and msgs:
            print("\n".join(msgs))
        return obj

    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one, SOURCES + PROBE_SOURCES))

    def link(objects, out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objects, "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"link of {os.path.basename(out)} failed:\n" + res.stdout + res.stderr)
        os.replace(tmp, out)

    link(objs[:len(SOURCES)], OUT)
    link(objs[len(SOURCES):], PROBE_OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))

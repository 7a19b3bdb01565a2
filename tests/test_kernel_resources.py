"""Register, scratch and occupancy budgets of the matrix-core kernels (CPU).

The kernels' designs rest on budgets the compiler enforces silently: the
persistent forward, the fused step, the commit, the prefill and the grouped
forwards at d = 128, FW <= 64 are laid out for two resident work-groups per CU
with no register spills, and a spill in the streaming loops (scratch
traffic whose waits drain the state stream) or a lost work-group costs far more
than the edit that caused it. These tests compile every matrix-core source to
gfx950 assembly with the library's own flags and read the compiler's
per-kernel resource report (ScratchSize, Occupancy).
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from linear_attention_block_amd import build

SOURCES = [s for s in build.SOURCES if s.startswith("mfma_")]

# the one instantiation known to spill: four query heads per K/V head at
# d = 64, FW = 128 (80 bytes per lane at one work-group per CU)
SCRATCH_ALLOWED = {("forward_gqa_mfma_kernel", (64, 128, 4)): 80}

# resident waves per SIMD the decode-size kernels are built for
MIN_OCCUPANCY = {
    ("forward_mfma_kernel", (128, 64, 1, 0)): 2,
    ("forward_mfma_kernel", (128, 32, 1, 0)): 2,
    ("forward_mfma_kernel", (128, 64, 2, 0)): 2,
    ("forward_mfma_kernel", (64, 64, 1, 0)): 2,
    # d = 64 at one wave per SIMD, compiled for that budget
    ("forward_mfma_kernel", (64, 64, 1, 1)): 1,
    ("forward_mfma_kernel", (64, 32, 1, 1)): 1,
    ("forward_commit_mfma_kernel", (128, 64, 0)): 2,
    ("forward_commit_mfma_kernel", (128, 64, 1)): 2,
    ("commit_mfma_kernel", (128, 64, 0)): 2,
    ("commit_mfma_kernel", (128, 64, 1)): 2,
    ("prefill_mfma_kernel", (128, 64)): 2,
    ("forward_gqa_mfma_kernel", (128, 64, 2)): 2,
    ("forward_gqa_mfma_kernel", (128, 64, 4)): 2,
    ("forward_gqa8_kernel", (128, 64, 0)): 2,
    ("forward_gqa8_kernel", (128, 64, 1)): 2,
    ("feature_map_mfma_kernel", (128, 64, 0)): 2,
    ("feature_map_mfma_kernel", (128, 64, 1)): 2,
    ("forward_split_kernel", (128,)): 2,
}

_SYM = re.compile(r"^_ZN3bha12_GLOBAL__N_1(\d+)(\w+?)I((?:L[ib]\d+E)+)E\S*:")


def _kernel_key(sym_line):
    m = _SYM.match(sym_line)
    if not m:
        return None
    n = int(m.group(1))
    name = (m.group(2) + m.group(3))[:n]
    if "kernel" not in name:
        return None
    return name, tuple(int(x) for x in re.findall(r"L[ib](\d+)E", m.group(3)))


def _parse(path):
    out, cur = {}, None
    for line in open(path):
        key = _kernel_key(line)
        if key is not None:
            cur = key
            out[cur] = {}
            continue
        if cur is None:
            continue
        for field in ("ScratchSize", "Occupancy", "NumVgprs"):
            m = re.match(r"^\s*;\s*" + field + r":\s*(\d+)", line)
            if m and field not in out[cur]:
                out[cur][field] = int(m.group(1))
    return out


@pytest.fixture(scope="module")
def resources():
    try:
        cc = build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    tmp = tempfile.mkdtemp(prefix="bha_res_")
    try:
        def one(src):
            out = os.path.join(tmp, src + ".s")
            cmd = [cc, *build.common_flags(), "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", out]
            res = subprocess.run(cmd, capture_output=True, text=True)
            assert res.returncode == 0, f"hipcc failed on {src}:\n{res.stderr[-2000:]}"
            return _parse(out)

        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            parts = list(ex.map(one, SOURCES))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    table = {}
    for p in parts:
        table.update(p)
    return table


def test_every_source_has_kernels(resources):
    names = {k[0] for k in resources}
    for want in ("forward_mfma_kernel", "forward_split_kernel", "forward_gqa_mfma_kernel", "forward_gqa8_kernel",
                 "commit_mfma_kernel", "forward_commit_mfma_kernel", "prefill_mfma_kernel",
                 "feature_map_mfma_kernel"):
        assert want in names, f"{want} not found in the compiled sources"
    for key, v in resources.items():
        assert {"ScratchSize", "Occupancy", "NumVgprs"} <= set(v), f"no resource report for {key}"


def test_no_register_spills(resources):
    spills = {k: v["ScratchSize"] for k, v in resources.items() if v["ScratchSize"] > SCRATCH_ALLOWED.get(k, 0)}
    assert not spills, f"kernels using scratch beyond their allowance: {spills}"


def test_decode_kernels_keep_their_occupancy(resources):
    short = {k: (resources[k]["Occupancy"] if k in resources else None) for k in MIN_OCCUPANCY}
    missing = [k for k, occ in short.items() if occ is None]
    assert not missing, f"kernels not compiled: {missing}"
    low = {k: occ for k, occ in short.items() if occ < MIN_OCCUPANCY[k]}
    assert not low, f"kernels below their designed occupancy: {low}"

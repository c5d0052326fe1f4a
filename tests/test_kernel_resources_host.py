"""Every kernel compiles for gfx950 without private-memory traffic: no VGPR
spills and no scratch (a kernel that indexes its by-value arguments with a
per-thread value, or runs out of registers, gets scratch, and its loads and
stores then cost HBM traffic in the hot loop).  Host-only: hipcc's resource
report of the kernels built here."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from kv_cached_decode_amd import build as kbuild

SOURCES = [s for s in kbuild.SOURCES if s.endswith(".hip")]


def resources(src):
    cmd = [kbuild.HIPCC, "-x", "hip"] + kbuild.COMMON + [
        "-c", os.path.join(kbuild.CSRC, src), "-o", os.devnull,
        "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, name, res = r.stderr, None, {}
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            res[name] = {}
            continue
        m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs Spill|VGPRs): (\d+)", line)
        if m and name:
            res[name][m.group(1)] = int(m.group(2))
    return res


@pytest.fixture(scope="module")
def report():
    if not os.path.exists(kbuild.HIPCC):
        pytest.skip("hipcc not available")
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        parts = list(ex.map(resources, SOURCES))
    return {k: v for p in parts for k, v in p.items()}


def test_no_scratch_and_no_spills(report):
    assert len(report) >= 6
    bad = {k: v for k, v in report.items()
           if v.get("ScratchSize [bytes/lane]", 0) or v.get("VGPRs Spill", 0)}
    assert not bad, bad


def test_hot_kernels_keep_two_waves_per_simd(report):
    """The decode kernels run two waves per SIMD: at most 256 VGPRs."""
    for k, v in report.items():
        if "attn_mfma_kernel" in k or "decode_step_mfma_kernel" in k or "attn_prefill_kernel" in k:
            assert v["VGPRs"] <= 256, (k, v["VGPRs"])

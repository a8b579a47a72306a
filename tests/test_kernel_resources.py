"""Register and scratch use of the specialised kernels, read from the compiler on the CPU: every kernel of
the decode, append and prefill sources compiles without VGPR spills and without scratch memory (private
segment), since a spill to scratch would put memory traffic into the hot loops.  SGPR spills are allowed:
they go to VGPR lanes (v_writelane / v_readlane), not to memory."""

import os
import re
import subprocess

import pytest

from mla_latent_kv_cache_amd import build as B

SOURCES = ["decode.hip", "append.hip", "prefill.hip"]


def _resources(src):
    cmd = [B.HIPCC, *B.FLAGS, "--cuda-device-only", "-c", os.path.join(B.CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
            continue
        m = re.search(r"remark: +(ScratchSize \[bytes/lane\]|VGPRs Spill|SGPRs Spill|VGPRs|AGPRs|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and name:
            out[name][m.group(1)] = int(m.group(2))
    return out


@pytest.mark.timeout(600)
@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch_and_no_vgpr_spills(src):
    res = _resources(src)
    kernels = {k: v for k, v in res.items() if "ScratchSize [bytes/lane]" in v}
    assert kernels, f"no kernel resource remarks for {src}"
    bad = {k: v for k, v in kernels.items() if v["ScratchSize [bytes/lane]"] or v.get("VGPRs Spill", 0)}
    assert not bad, f"{src}: kernels with scratch or VGPR spills: {bad}"

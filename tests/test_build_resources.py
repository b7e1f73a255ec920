"""Register use of every kernel, from the compiler's resource-usage remarks
(CPU only: each source is compiled to a throw-away object for gfx950).

"Optimizing Triton kernels for custom attention patterns on H100", Common
Failure Modes, names register spills as a silent cause of slow kernels. On
gfx950 a VGPR spill goes to scratch memory: no kernel may have one, nor any
scratch. A spilled SGPR goes to a lane of a VGPR (v_writelane /
v_readlane, no memory traffic); none is allowed either."""

from concurrent.futures import ThreadPoolExecutor

import pytest

from tiled_attention_amd import build

KERNEL_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]


@pytest.fixture(scope="module")
def usage():
    with ThreadPoolExecutor(max_workers=len(KERNEL_SOURCES)) as ex:
        parts = list(ex.map(build.resource_usage, KERNEL_SOURCES))
    out = {}
    for p in parts:
        out.update(p)
    return out


def test_every_kernel_reports_its_resources(usage):
    assert len(usage) >= 20
    for name, u in usage.items():
        for field in ("VGPRs", "ScratchSize", "VGPRs Spill", "SGPRs Spill", "Occupancy"):
            assert field in u, (name, field)


def test_no_vgpr_spill_and_no_scratch(usage):
    bad = {n: u for n, u in usage.items() if u["VGPRs Spill"] or u["ScratchSize"]}
    assert not bad, bad


def test_no_sgpr_spill(usage):
    bad = {n: u["SGPRs Spill"] for n, u in usage.items() if u["SGPRs Spill"]}
    assert not bad, bad


def test_forward_kernels_keep_two_waves_per_simd(usage):
    """Two workgroups of four waves share a CU: every forward kernel fits 256
    VGPRs per wave (occupancy 2)."""
    for n, u in usage.items():
        if "fwd_mfma_kernel" in n:
            assert u["Occupancy"] >= 2 and u["VGPRs"] <= 256, (n, u)

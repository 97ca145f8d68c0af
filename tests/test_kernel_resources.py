"""The step kernels' register, scratch and LDS budgets, from the compiler's own resource report
(host-side compilation for gfx950; no GPU).  A d = 128 workgroup is four waves, one per SIMD, so
"waves per SIMD" is the number of workgroups a CU holds: four for the fused step, the split
writeback and the encode (at most 128 VGPRs and 40 KB of LDS each), five for the split readout
(at most 96 VGPRs and 32 KB).  Scratch would mean spilled registers: a scratch reload inside a
tile waits on memory, so none is allowed."""
import os
import re
import shutil

import pytest

from quantized_delta_rule_amd import build

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
pytestmark = pytest.mark.skipif(not shutil.which(HIPCC), reason="hipcc not available")

KERNEL = re.compile(r"_ZN5stepq3dev5k_(gdn|kda)ILi(\d+)ELi(\d+)EEEvNS_8StepArgsE$")
READ = 1  # mode 1: the split readout


@pytest.fixture(scope="module")
def resources():
    return build.kernel_resources()


def test_every_step_kernel_is_reported(resources):
    found = {(m.group(1), int(m.group(2)), int(m.group(3)))
             for m in map(KERNEL.match, resources) if m}
    want = {(kind, d, mode) for kind in ("gdn", "kda") for d in (64, 128) for mode in range(4)}
    assert found == want


def test_no_kernel_spills(resources):
    for name, r in resources.items():
        assert r["ScratchSize"] == 0, f"{name}: {r['ScratchSize']} bytes of scratch per lane"
        assert r["VGPRs Spill"] == 0 and r["SGPRs Spill"] == 0, f"{name}: {r}"


def test_workgroups_per_cu_at_d128(resources):
    for name, r in resources.items():
        m = KERNEL.match(name)
        if not m or int(m.group(2)) != 128:
            continue
        if int(m.group(3)) == READ:
            assert r["Occupancy"] >= 5 and r["VGPRs"] <= 96 and r["LDS Size"] <= 32768, (name, r)
        else:
            assert r["Occupancy"] >= 4 and r["VGPRs"] <= 128 and r["LDS Size"] <= 40960, (name, r)

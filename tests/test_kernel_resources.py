"""Register budgets of the HIP kernels, from the compiler's resource report.

No kernel may spill to scratch memory (a spill turns register traffic into
memory traffic and once cost the derived dispatch a fifth of its speed), and the
persistent pull-form kernels must fit their grid at once: 16 waves per compute
unit (4 per SIMD), since every wave of an XCD takes a share of every group's
tasks.  Compiles each source with -c on the CPU (no GPU needed)."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from combine_ep_get_02_amd import build as hip_build

PULL_KERNELS = ("dispatch_pull_kernel", "dispatch_grouped_pull_kernel")


def _report(src: str) -> dict:
    flags = [f for f in hip_build.FLAGS if f != "-shared"]
    cmd = ["hipcc", *flags, "-c", src, "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    out = subprocess.run(cmd, capture_output=True, text=True, check=True).stderr
    kernels, cur = {}, None
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        for key, name in (("VGPRs", "vgprs"), (r"ScratchSize \[bytes/lane\]", "scratch"),
                          (r"Occupancy \[waves/SIMD\]", "occupancy")):
            m = re.search(key + r": (\d+)", line)
            if m and cur:
                kernels[cur][name] = int(m.group(1))
    return kernels


@pytest.fixture(scope="module")
def resources():
    with ThreadPoolExecutor(max_workers=4) as pool:
        reports = list(pool.map(_report, hip_build.SOURCES))
    merged = {}
    for r in reports:
        merged.update(r)
    assert merged, "no kernel found in the compiler's report"
    return merged


def test_no_kernel_spills_to_scratch(resources):
    spills = {k: v for k, v in resources.items() if v.get("scratch", 0) != 0}
    assert spills == {}


def test_pull_kernels_hold_their_grid(resources):
    pull = {k: v for k, v in resources.items() if any(n in k for n in PULL_KERNELS)}
    assert pull, "pull-form kernels missing from the report"
    assert all(v["occupancy"] >= 4 for v in pull.values()), pull

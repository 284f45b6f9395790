"""The compiler's resource report for every HIP kernel (CPU only: hipcc cross-compiles for
gfx950).  No kernel may spill registers to scratch memory: a spill inside a tile loop adds
vector-memory traffic that the kernels' hand-counted memory waits do not account for, and
slows the loop besides."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from sparse_attention_05_amd import build as hip_build

KERNEL_SOURCES = [s for s in hip_build.SOURCES + hip_build.PEAKS_SOURCES if s.endswith(".hip")]


def _report(src):
    cmd = [hip_build.HIPCC, *hip_build.FLAGS, *hip_build.EXTRA.get(src, []), "-x", "hip", "-c",
           os.path.join(hip_build.CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage", "--offload-device-only"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    names = re.findall(r"remark:\s+Function Name: (\S+)", r.stderr)
    scratch = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)]
    assert names and len(names) == len(scratch), "unexpected resource report for %s" % src
    return dict(zip(names, scratch))


@pytest.fixture(scope="module")
def reports():
    if not os.path.exists(hip_build.HIPCC):
        pytest.skip("hipcc not available")
    with ThreadPoolExecutor(max_workers=4) as ex:
        return dict(zip(KERNEL_SOURCES, ex.map(_report, KERNEL_SOURCES)))


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_kernel_spills_to_scratch(reports, src):
    spilled = {k: v for k, v in reports[src].items() if v}
    assert not spilled, "%s: kernels with scratch (bytes per lane): %s" % (src, spilled)


def test_sparse_mla_kernel_is_in_the_report(reports):
    assert any("sparse_mla_kernel" in k for k in reports["sparse_mla.hip"])

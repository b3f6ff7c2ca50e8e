"""Every HIP kernel of the library compiles for gfx950 with no scratch memory
(CPU only: hipcc cross-compiles).

A kernel whose registers spill, or that indexes a register array at run
time, gets per-lane scratch memory: slow, and a sign the code does not do
what its design says.  Each source under csrc/ is compiled with the
compiler's kernel resource report, with the library's own flags, and every
kernel must report ScratchSize 0.  The compiles run in parallel.
"""
import concurrent.futures
import glob
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from moe_token_routing_amd import build as B

SOURCES = sorted(glob.glob(os.path.join(B.CSRC, "*.hip")))


def _report(src):
    """(kernel name, scratch bytes per lane, VGPRs) for every kernel in src."""
    with tempfile.TemporaryDirectory() as tmp:
        flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
        cmd = [B.HIPCC, *flags, "-c", src, "-o", os.path.join(tmp, "k.o"), "-Rpass-analysis=kernel-resource-usage"]
        res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    out, name = [], None
    for line in res.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            out.append((name, int(m.group(1))))
    return src, out


@pytest.fixture(scope="module")
def reports():
    if not os.path.exists(B.HIPCC) and not shutil.which(B.HIPCC):
        pytest.skip("hipcc not available")
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return dict(ex.map(_report, SOURCES))


def test_every_kernel_has_no_scratch(reports):
    kernels = [(os.path.basename(src), name, scratch) for src, rows in reports.items() for name, scratch in rows]
    assert len(kernels) >= 10, kernels
    spilled = [k for k in kernels if k[2] != 0]
    assert not spilled, spilled


def test_every_source_reports_its_kernels(reports):
    for src, rows in reports.items():
        if os.path.basename(src) == "static_scratch.hip":
            continue  # holds a device array and host code only
        assert rows, f"{src}: no kernel in the resource report"

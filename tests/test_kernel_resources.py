"""Every HIP kernel keeps its working set in registers: compiled for gfx950
with the library's flags, no kernel may use scratch (private, per-lane) memory.

Scratch in these streaming kernels means the row chunks or the batched top-k
ids spilled to memory, which costs both bandwidth and latency; a helper that
stops being inlined (arrays passed by reference) does that silently.  Runs the
compiler only, no GPU."""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

from combine_ep_layout_07_amd import _build

KERNEL_SOURCES = [s for s in _build.SOURCES if s.endswith(".hip")]


def _resource_remarks(src):
    cmd = ([_build.HIPCC] + _build.FLAGS + ["-x", "hip", "-c", os.path.join(_build.CSRC, src), "-o", os.devnull,
                                            "-Rpass-analysis=kernel-resource-usage"])
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    usage, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            usage[name] = int(m.group(1))
    return src, usage


@pytest.fixture(scope="module")
def scratch_by_kernel():
    with cf.ThreadPoolExecutor(len(KERNEL_SOURCES)) as ex:
        return dict(ex.map(_resource_remarks, KERNEL_SOURCES))


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_kernel_uses_scratch(scratch_by_kernel, src):
    usage = scratch_by_kernel[src]
    assert usage, f"no kernel resource remarks for {src}"
    spilled = {k: v for k, v in usage.items() if v}
    assert not spilled, f"kernels using scratch memory in {src}: {spilled}"

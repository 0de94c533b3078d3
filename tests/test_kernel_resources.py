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
    usage, occupancy, name = {}, {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            continue
        m = re.search(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            usage[name] = int(m.group(1))
        m = re.search(r"remark:\s+Occupancy \[waves/SIMD\]: (\d+)", line)
        if m and name:
            occupancy[name] = int(m.group(1))
    return src, (usage, occupancy)


@pytest.fixture(scope="module")
def remarks_by_source():
    with cf.ThreadPoolExecutor(len(KERNEL_SOURCES)) as ex:
        return dict(ex.map(_resource_remarks, KERNEL_SOURCES))


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_kernel_uses_scratch(remarks_by_source, src):
    usage = remarks_by_source[src][0]
    assert usage, f"no kernel resource remarks for {src}"
    spilled = {k: v for k, v in usage.items() if v}
    assert not spilled, f"kernels using scratch memory in {src}: {spilled}"


# Waves per SIMD the register allocation must leave to the streaming kernels
# at the workloads' row sizes (14 KiB rows: 14 chunks per lane; the 2 KiB
# pieces and the combine's passes: 2 chunks per lane): the allocation each was
# measured at; a register increase that dropped the combine below it cost
# 2-3%.  The piece kernels keep the most waves the hardware holds.
MIN_OCCUPANCY = {
    ("ep_dispatch.hip", "k_scatterILi14E"): 4,
    ("ep_dispatch.hip", "k_scatter_pfILi14E"): 2,
    ("ep_dispatch.hip", "k_epilogue_pfILi14E"): 2,
    ("ep_dispatch.hip", "k_epilogue_indexedILi2E"): 8,
    ("ep_dispatch.hip", "k_epilogue_expand_indexedILi2E"): 8,
    ("ep_dispatch.hip", "k_epilogue_expand_piecesILi2E"): 8,
    ("ep_combine.hip", "k_combineILi2E"): 4,
}


@pytest.mark.parametrize("src,kernel", sorted(MIN_OCCUPANCY))
def test_streaming_kernels_keep_their_occupancy(remarks_by_source, src, kernel):
    occ = remarks_by_source[src][1]
    hits = {k: v for k, v in occ.items() if kernel in k}
    assert hits, f"{kernel} not found in {src}"
    for k, v in hits.items():
        assert v >= MIN_OCCUPANCY[(src, kernel)], f"{k}: {v} waves per SIMD"

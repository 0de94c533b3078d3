"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The four library sources are compiled with the sanitizers on the host side
only (``-Xarch_host``; device code is compiled as usual and never runs) and
linked with ``tests/host_sanitize_driver.cpp``, which pushes millions of
configurations mixing ordinary and extreme values through ``ep_query_sizes``
and the argument checks of every call.  Any signed overflow, bad shift or
out-of-bounds access in the configuration checks, the buffer sizes or the
layout geometry ends the run with an error.  CPU only (hipcc cross-compiles).
"""
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "combine_ep_layout_07_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
COMMON = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def _compile(src: str, obj: str, hip: bool) -> str:
    cmd = [HIPCC, *COMMON, *HOST_SAN] + (["-x", "hip"] if hip else []) + ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return obj


def test_host_code_clean_under_sanitizers(tmp_path):
    srcs = [(os.path.join(CSRC, f), f.endswith(".hip"))
            for f in ("ep_api.cpp", "ep_layout.hip", "ep_dispatch.hip", "ep_combine.hip")]
    srcs.append((os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"), False))
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(lambda a: _compile(a[0], str(tmp_path / (os.path.basename(a[0]) + ".o")), a[1]), srcs))
    exe = str(tmp_path / "host_san")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "--hip-link", *HOST_SAN[:4], *objs, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    for seed in (1, 2):
        run = subprocess.run([exe, "2000000", str(seed)], capture_output=True, text=True, timeout=300, env=env)
        assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-4000:]
        assert ": ok" in run.stdout

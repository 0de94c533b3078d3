"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

``tests/oracle_sanitize_driver.c`` calls every oracle entry point over random
small configurations (masked, invalid and duplicated lanes, empty sources,
hybrid topologies, both layouts, bf16 and fp8) with each array allocated at
exactly its documented size; built with ``-fsanitize=address,undefined`` and
no recovery, any access outside an array or any undefined arithmetic ends the
run with an error.  A copy of the oracle with a planted out-of-bounds store
shows that the harness catches one.  CPU only (gcc).
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_DIR = os.path.join(ROOT, "oracle")
ORACLE_SRC = os.path.join(ORACLE_DIR, "ep_oracle.c")
DRIVER = os.path.join(ROOT, "tests", "oracle_sanitize_driver.c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _build(src: str, exe: str) -> str:
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", *SAN, "-ffp-contract=off", "-Wall", "-Wextra",
           "-Werror", "-I", ORACLE_DIR, src, DRIVER, "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe: str, n: int, seed: int) -> subprocess.CompletedProcess:
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe, str(n), str(seed)], capture_output=True, text=True, timeout=300, env=env)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_oracle_clean_under_sanitizers(tmp_path, seed):
    exe = _build(ORACLE_SRC, str(tmp_path / "oracle_san"))
    r = _run(exe, 1000, seed)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "1000 configurations ok" in r.stdout


def test_sanitizers_catch_a_planted_out_of_bounds_store(tmp_path):
    anchor = "recv_src_idx[i] = (int32_t)((int64_t)s * T + meta[0]);"
    src = open(ORACLE_SRC).read()
    assert src.count(anchor) == 1
    bad = tmp_path / "ep_oracle_oob.c"
    bad.write_text(src.replace(anchor, "recv_src_idx[i + 1] = (int32_t)((int64_t)s * T + meta[0]);"))
    exe = _build(str(bad), str(tmp_path / "oracle_oob"))
    r = _run(exe, 200, 1)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr

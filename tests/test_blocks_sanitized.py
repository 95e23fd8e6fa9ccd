"""The native block manager under AddressSanitizer and UndefinedBehaviorSanitizer.

Host code only: csrc/pa_blocks.cpp and a stress driver (tests/native/bm_stress.cpp)
are compiled with g++ -fsanitize=address,undefined (no HIP, no GPU) and run through
20,000 random operations and every error path; any invalid access, leak or undefined
behaviour fails the test."""

from __future__ import annotations

import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_block_manager_under_sanitizers(tmp_path):
    exe = tmp_path / "bm_stress"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", f"-I{ROOT / 'include'}",
           f"-I{ROOT / 'paged_kv_cache_414_amd' / 'csrc'}",
           str(ROOT / "tests" / "native" / "bm_stress.cpp"),
           str(ROOT / "paged_kv_cache_414_amd" / "csrc" / "pa_blocks.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                         env={"ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
                              "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "bm_stress ok" in run.stdout

"""Host-side invariants of the decode schedule, checked by a small C++ program
compiled here with g++ against the library's host source (no GPU, no HIP
runtime): key ranges covered exactly once per request, pieces inside their
request and on 32-key (one decode tile) boundaries, consecutive partial slots
per request, direct writes only for whole requests in the decode kernel, and
equal shares across the split form's work-groups (3000 random batches,
windows, groups and forms)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_decode_schedule_invariants(tmp_path):
    exe = tmp_path / "decode_schedule_check"
    src = os.path.join(ROOT, "tests", "cpp", "decode_schedule_check.cpp")
    host = os.path.join(ROOT, "paged_sliding_window_page_amd", "csrc", "psw_host.cpp")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(ROOT, "paged_sliding_window_page_amd", "csrc"),
                    src, host, "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr

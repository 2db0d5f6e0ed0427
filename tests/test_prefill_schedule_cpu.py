"""Host-side invariants of the prefill schedule, checked by a small C++
program compiled here with g++ against the library's host source (no GPU, no
HIP runtime).  For 3000 random batches (chunked prefills included), windows,
GQA groups and both head dims: the items of each request start on its query
tiles and cover them exactly once, each item's key range is exactly the keys
its tokens may see (window start of its first token to its last token's
position; PR "feat(kernels): Rust wrapper for the hd256 windowed paged
prefill", Description: inclusive window_left), items come heaviest first
with total_tiles their sum, and the pre-launch item check accepts the
schedule and rejects planted mistakes."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_prefill_schedule_invariants(tmp_path):
    exe = tmp_path / "prefill_schedule_check"
    src = os.path.join(ROOT, "tests", "cpp", "prefill_schedule_check.cpp")
    host = os.path.join(ROOT, "paged_sliding_window_page_amd", "csrc", "psw_host.cpp")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(ROOT, "paged_sliding_window_page_amd", "csrc"),
                    src, host, "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr

"""Host-side properties of the prep work items, checked by a small C++ program
compiled here with g++ against the library's host source (no GPU, no HIP
runtime).  For 4000 random plans the prep entries' own checks accept (batches
at random start positions, page sizes 8..64, resident windows whose pages wrap
as a ring): every item lies inside one page and holds at most 16 tokens, takes
its page from its own request's table at the page of its position, stays
below kv_len (so inside the RoPE table the entry checked), the items cover
each request's new tokens exactly once and no pool slot twice, and the
library's pre-launch item check accepts them and rejects planted mistakes.
These are the conditions the prep kernels' device-side check records in the
device error word, which the entries therefore never reach (issue "gemma4:
serving prep needs pool-write forms", Proposed Plan: host checks first, a
kernel-side check behind them)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_prep_item_invariants(tmp_path):
    exe = tmp_path / "prep_items_check"
    src = os.path.join(ROOT, "tests", "cpp", "prep_items_check.cpp")
    host = os.path.join(ROOT, "paged_sliding_window_page_amd", "csrc", "psw_host.cpp")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(ROOT, "paged_sliding_window_page_amd", "csrc"),
                    src, host, "-o", str(exe)], check=True, capture_output=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr

"""The head_dim-512 prefill's inline-assembly MFMAs (the QK chain, whose
accumulators stay in VGPRs while O fills the accumulator registers) against
the hardware's MFMA wait states, checked on the compiled gfx950 code: the
translation unit is compiled here with hipcc (no GPU needed) and its
assembly scanned for a read of an MFMA result, or a VALU write of an MFMA
source, inside the wait states (tests/isa_hazards.py).  The checker itself is
pinned on a hand-written sequence with known hazards."""
import os
import shutil
import subprocess

import pytest

from isa_hazards import find_hazards

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_sliding_window_page_amd", "csrc")


def test_checker_flags_known_hazards():
    seq = "\n".join([
        "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]",
        "\tds_read_b128 v[24:27], v40",
        "\tv_mov_b32_e32 v30, v3",                 # result read 1 wait state later
        "\tv_add_u32_e32 v17, v1, v2",             # source of the next MFMA written
        "\ts_nop 0",
        "\tv_mfma_f32_32x32x16_bf16 v[32:47], v[16:19], v[20:23], 0",
        "\tv_mfma_f32_32x32x16_bf16 v[32:47], v[24:27], v[20:23], v[32:47]",  # chained: fine
        "\ts_nop 11",
        "\tv_mov_b32_e32 v50, v33",                # after the wait states: fine
    ])
    found = find_hazards(seq)
    assert len(found) == 2, found
    assert "line 3" in found[0] and "line 4 writes" in found[1]


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc") and shutil.which("hipcc") is None,
                    reason="hipcc not available")
def test_prefill512_inline_mfma_keeps_wait_states(tmp_path):
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else shutil.which("hipcc")
    obj = tmp_path / "p512.o"
    subprocess.run([hipcc, "-O3", "-std=c++17", "-fPIC", f"-I{os.path.join(ROOT, 'include')}",
                    f"-I{CSRC}", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", "-c", os.path.join(CSRC, "psw_prefill512.hip"), "-o",
                    str(obj), "-save-temps=obj"], check=True, capture_output=True, timeout=600)
    asm = [p for p in tmp_path.iterdir() if p.name.endswith("gfx950.s")]
    assert asm, list(tmp_path.iterdir())
    text = asm[0].read_text()
    assert "prefill512_kernel" in text
    found = find_hazards(text)
    assert not found, "\n".join(found[:20])

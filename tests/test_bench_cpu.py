"""Host-side logic of bench.py: the one-GPU guard, the HBM-traffic summary
built from two rocprofv3 counter runs (scaled by a copy of known size), and
the digest check that keeps a stale summary out of the JSON line."""
import csv
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_short_kernel_name():
    n = ("void psw_dev::(anonymous namespace)::prefill256_pp_kernel<true, true>"
         "(psw_dev::AttnParams)")
    assert bench.short_kernel_name(n) == "prefill256_pp_kernel<true, true>"


def _counter_csv(path, counter, dispatches):
    """dispatches: (id, kernel name, [values of the per-XCD pieces])."""
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                           "Counter_Value"])
        w.writeheader()
        for did, name, values in dispatches:
            for v in values:
                w.writerow({"Dispatch_Id": did, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": v})


COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"
PREF = "void psw_dev::(anonymous namespace)::prefill256_pp_kernel<true, true>(psw_dev::AttnParams)"


def test_pmc_summary_scales_by_the_copy(tmp_path):
    # a 256 MiB copy whose FETCH_SIZE reads half its bytes and WRITE_SIZE all
    # of them; the prefill's counters come in 8 per-XCD pieces per dispatch
    kib = 256 * 1024
    f = tmp_path / "fetch.csv"
    wr = tmp_path / "write.csv"
    _counter_csv(f, "FETCH_SIZE", [(1, COPY, [kib / 2]),
                                   (2, PREF, [1000.0] * 8), (3, PREF, [1100.0] * 8),
                                   (4, PREF, [1200.0] * 8)])
    _counter_csv(wr, "WRITE_SIZE", [(1, COPY, [kib]),
                                    (2, PREF, [500.0] * 8), (3, PREF, [500.0] * 8),
                                    (4, PREF, [600.0] * 8)])
    text = bench.pmc_summary(str(f), str(wr), 256)
    assert f"source_digest: {bench.source_digest()}" in text
    assert "x 2.000" in text and "x 1.000" in text
    row = [l for l in text.splitlines() if l.startswith("| `prefill256_pp_kernel<true, true>` |")]
    assert len(row) == 1
    cells = [c.strip() for c in row[0].strip("|").split("|")]
    assert cells[1] == "3"                       # dispatches
    assert float(cells[2]) == 8800.0             # median FETCH_SIZE KiB (8 x 1100)
    assert float(cells[3]) == 4000.0             # median WRITE_SIZE KiB (8 x 500)
    assert int(cells[6]) == 8800 * 1024 * 2 + 4000 * 1024
    # the copy itself is the calibration, not a row
    assert "neg_kernel" not in "".join(l for l in text.splitlines() if l.startswith("| `"))


def test_pmc_summary_needs_the_copy(tmp_path):
    f = tmp_path / "fetch.csv"
    wr = tmp_path / "write.csv"
    _counter_csv(f, "FETCH_SIZE", [(2, PREF, [1.0])])
    _counter_csv(wr, "WRITE_SIZE", [(2, PREF, [1.0])])
    with pytest.raises(SystemExit):
        bench.pmc_summary(str(f), str(wr), 256)


def test_traffic_is_read_only_for_the_current_sources(tmp_path, monkeypatch):
    row = "| `prefill256_pp_kernel<true, true>` | 2 | 1.0 | 1.0 | 0.00 | 0.00 | 123456 |"
    good = tmp_path / "good.md"
    good.write_text(f"source_digest: {bench.source_digest()}\n\n{row}\n")
    stale = tmp_path / "stale.md"
    stale.write_text("source_digest: 0000\n\n" + row + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(good))
    assert bench.read_traffic("prefill256_pp_kernel<true, true>") == 123456
    assert bench.read_traffic("decode_kernel<256, 1>") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(stale))
    assert bench.read_traffic("prefill256_pp_kernel<true, true>") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.read_traffic("prefill256_pp_kernel<true, true>") is None

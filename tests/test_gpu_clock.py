"""The shader-clock diagnostic (psw_measure_mfma_clock): a clock the part can
run at (the benchmark scales the MFMA peak by it for the clock-adjusted
fraction it reports next to the nominal one)."""
import pytest

pytestmark = pytest.mark.gpu


def test_mfma_clock_is_plausible():
    import paged_sliding_window_page_amd as psw
    from gpu_util import say
    say("[gpu] shader clock under MFMA load")
    mhz = psw.measure_mfma_clock()
    say(f"[gpu] {mhz:.0f} MHz")
    assert 300.0 < mhz < 3000.0

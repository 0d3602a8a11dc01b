"""bench.py's command line on the host: more than one GPU is refused with a
message and exit status 2, before anything is built, loaded or launched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 2, (r.returncode, r.stderr[-500:])
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_clock_sampler_reads_the_current_level(tmp_path):
    """The shader-clock sampler takes the default line marked '*' (the current
    level, whether a listed DPM level or the 'S:' line) and averages samples."""
    sys.path.insert(0, ROOT)
    import bench
    for text, mhz in [("S: 2104Mhz *\n0: 500Mhz\n1: 2400Mhz\n", 2104.0),
                      ("0: 500Mhz\n1: 2400Mhz *\n", 2400.0),
                      ("0: 500Mhz\n1: 2400Mhz\n", None)]:
        f = tmp_path / "pp_dpm_sclk"
        f.write_text(text)
        c = bench.ClockSampler()
        c.path = str(f)
        assert c._read() == mhz
    c = bench.ClockSampler()
    c.path, c.samples = None, [2000.0, 2100.0]
    assert c.mhz() == 2050.0


def test_clock_fields_drop_an_impossible_fraction():
    """A rate above the peak at the sampled clock means the samples missed the
    running clock: the peak at that clock is still reported, the fraction is not."""
    sys.path.insert(0, ROOT)
    import bench
    c = bench.ClockSampler()
    c.path, c.samples = None, [1728.0]
    f = bench.clock_fields(c, 1312.0)
    assert f["peak_at_sclk"] == 1800.0 and f["frac_at_sclk"] == round(1312.0 / 1800.0, 4)
    c.samples = [1024.0]
    f = bench.clock_fields(c, 1312.0)
    assert f["peak_at_sclk"] == round(2500.0 * 1024 / 2400, 1) and f["frac_at_sclk"] is None
    assert "sclk_note" in f
    c.samples = []
    assert bench.clock_fields(c, 1312.0)["sclk_mhz"] is None

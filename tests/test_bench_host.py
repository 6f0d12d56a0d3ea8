"""Host-side parts of bench.py: the sysfs clock / power readers and the
multi-GPU refusal (no GPU needed)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _card(tmp_path, sclk_lines, power_uw=None, cap_uw=None):
    dev = tmp_path / "device"
    dev.mkdir()
    (dev / "pp_dpm_sclk").write_text("".join(l + "\n" for l in sclk_lines))
    if power_uw is not None:
        hw = dev / "hwmon" / "hwmon3"
        hw.mkdir(parents=True)
        (hw / "power1_input").write_text(f"{power_uw}\n")
        (hw / "power1_cap").write_text(f"{cap_uw}\n")
    return str(dev)


def test_current_clock_is_the_starred_line(tmp_path):
    # idle: a separate current-level line; under load: one of the DPM levels
    assert bench._sclk_mhz(_card(tmp_path, ["S: 112Mhz *", "0: 500Mhz", "1: 2400Mhz"])) == 112.0


def test_clock_level_marked(tmp_path):
    assert bench._sclk_mhz(_card(tmp_path, ["0: 500Mhz", "1: 1735Mhz *", "2: 2400Mhz"])) == 1735.0


def test_no_marked_level_gives_none(tmp_path):
    assert bench._sclk_mhz(_card(tmp_path, ["0: 500Mhz", "1: 2400Mhz"])) is None


def test_power_microwatts_to_watts(tmp_path):
    dev = _card(tmp_path, ["0: 500Mhz *"], power_uw=1_234_500_000, cap_uw=1_400_000_000)
    assert bench._power_w(dev) == 1234.5
    assert bench._power_w(dev, "power1_cap") == 1400.0


def test_no_card_no_telemetry():
    # this container has no GPU: no sysfs card, so the bench reports null telemetry
    if bench._gpu_sysfs() is None:
        assert bench.telemetry(lambda: None, 0.01) is None


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_floor_probe_library_validates_arguments():
    """The streaming-read probe (bench.py --floor) is built beside the GEMM
    library and refuses bad arguments before any GPU call."""
    import ctypes

    from dense_gemm_preshuffle_amd import build as b

    lib = ctypes.CDLL(b.PROBE_LIB)
    f = lib.gp_probe_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    buf, sink = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    assert f(None, 1 << 20, 256, 4, sink, None) == 1                       # null buffer
    assert f(ctypes.c_void_p(0x100008), 1 << 20, 256, 4, sink, None) == 1  # misaligned
    assert f(buf, 1 << 20, 0, 4, sink, None) == 1                          # no workgroups
    assert f(buf, 1 << 20, 256, 17, sink, None) == 1                       # too many waves
    assert f(buf, (1 << 20) + 16, 256, 4, sink, None) == 1                 # not whole lanes of the grid


def test_mfma_rate_probe_validates_arguments():
    """The MFMA issue-rate probe (bench.py --mfma-rate) shares the probe
    library and refuses bad arguments before any GPU call."""
    import ctypes

    from dense_gemm_preshuffle_amd import build as b

    lib = ctypes.CDLL(b.PROBE_LIB)
    f = lib.gp_probe_mfma_rate
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    out, cyc = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x200000)
    assert f(-1, out, cyc, 100, 256, None) == 1        # no such form
    assert f(10, out, cyc, 100, 256, None) == 1
    assert f(0, None, cyc, 100, 256, None) == 1        # null output
    assert f(0, out, None, 100, 256, None) == 1        # null cycle buffer
    assert f(0, out, cyc, 0, 256, None) == 1           # no iterations
    assert f(0, out, cyc, 100, 0, None) == 1           # no workgroups
    assert f(0, out, cyc, 100, 4097, None) == 1

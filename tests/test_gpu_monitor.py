"""Host logic of the GPU-state summary in bench.py (no GPU, no amdsmi needed):
only readings the firmware refreshed inside the sampled window are used, each
once."""
from bf16_gemm_decode_amd.gpu_monitor import GpuMonitor


def _sample(t, stamp, gfx, power, ppt=None, acc=None):
    return {"t": t, "gfx_mhz": gfx, "uclk_mhz": 2000.0, "power_w": power, "hotspot_c": 50.0, "hbm_c": 40.0,
            "stamp": stamp, "ppt_acc": ppt, "acc": acc}


def test_stale_first_reading_is_dropped():
    m = GpuMonitor.__new__(GpuMonitor)
    m.period, m.error, m.power_cap_w = 0.005, None, 1400.0
    # three samples of a reading taken before the window (idle), then two
    # refreshed readings seen several times each
    m.samples = ([_sample(0.000 + 0.005 * i, 100, 150.0, 270.0, 10, 1000) for i in range(3)] +
                 [_sample(0.9 + 0.005 * i, 200, 1850.0, 1395.0, 700, 2000) for i in range(5)] +
                 [_sample(1.9 + 0.005 * i, 300, 1810.0, 1397.0, 1500, 3000) for i in range(2)])
    out = m.summary()
    assert out["samples"] == 10 and out["distinct_readings"] == 3 and out["readings_used"] == 2
    assert out["gfx_clock_ghz"] == {"mean": 1.83, "min": 1.81, "max": 1.85}
    assert out["socket_power_w"] == {"mean": 1396.0, "min": 1395.0, "max": 1397.0}
    # power-limit residency over the whole window: (1500 - 10) / (3000 - 1000)
    assert out["at_power_limit_fraction"] == round(1490 / 2000, 3)
    assert "note" not in out


def test_single_reading_is_flagged():
    m = GpuMonitor.__new__(GpuMonitor)
    m.period, m.error, m.power_cap_w = 0.005, None, None
    m.samples = [_sample(0.005 * i, 100, 2200.0, 296.0) for i in range(4)]
    out = m.summary()
    assert out["distinct_readings"] == 1 and out["readings_used"] == 1
    assert "no refresh" in out["note"]
    assert out["socket_power_w"]["mean"] == 296.0

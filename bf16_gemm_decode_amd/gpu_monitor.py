"""Clock, power and temperature of one GPU while a measured region runs.

A background thread reads the GPU's firmware metrics table through the
amdsmi library every few milliseconds: the graphics clock of each XCD, the
memory clock, the socket power, the hotspot and HBM temperatures, and the
accumulated time spent at the package power limit ("PPT residency").  The
summary reports means and extremes over the samples and, from the PPT
residency counter, the fraction of the region the power limit was holding the
clock down.  Monitoring is best effort: without amdsmi, or on a field the
firmware does not report, the summary says so instead of failing the
measurement.
"""
import threading
import time

_NA = 0xFFFF


def _num(v):
    """A metrics value as a float, or None for 'N/A' and the not-reported
    sentinels."""
    if isinstance(v, (int, float)) and v not in (_NA, 0xFFFFFFFF, 0xFFFFFFFFFFFFFFFF):
        return float(v)
    return None


class GpuMonitor:
    def __init__(self, index=0, period_s=0.002):
        self.period = period_s
        self.samples = []
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        self.power_cap_w = None
        try:
            import amdsmi
            self._smi = amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self._handle = handles[index]
            try:
                cap = amdsmi.amdsmi_get_power_cap_info(self._handle)
                self.power_cap_w = cap["power_cap"] / 1e6 if _num(cap.get("power_cap")) else None
            except Exception:      # the cap is context, not required
                self.power_cap_w = None
        except Exception as e:     # no amdsmi, no permission, no device
            self.error = "%s: %s" % (type(e).__name__, e)

    def _read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = [c for c in (_num(x) for x in (m.get("current_gfxclks") or [])) if c]
        return {
            "t": time.perf_counter(),
            "gfx_mhz": sum(clks) / len(clks) if clks else _num(m.get("current_gfxclk")),
            "uclk_mhz": _num(m.get("current_uclk")),
            "power_w": _num(m.get("current_socket_power")),
            "hotspot_c": _num(m.get("temperature_hotspot")),
            "hbm_c": _num(m.get("temperature_mem")),
            "stamp": _num(m.get("system_clock_counter")),
            "ppt_acc": _num(m.get("ppt_residency_acc")),
            "acc": _num(m.get("accumulation_counter")),
        }

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception as e:
                self.error = "%s: %s" % (type(e).__name__, e)
                return
            time.sleep(self.period)

    def start(self):
        if self._handle is None:
            return self
        self.samples = []
        self._stop.clear()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()
        return self

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
            self._thread = None
        return self.summary()

    def summary(self):
        s = self.samples
        out = {"source": "amdsmi GPU metrics table, sampled every %.0f ms" % (self.period * 1e3),
               "samples": len(s),
               # the firmware refreshes the table at its own pace (about once
               # a second on MI355X): the number of distinct table time
               # stamps among the samples
               "distinct_readings": len({x["stamp"] for x in s}) if s else 0,
               "window_s": round(s[-1]["t"] - s[0]["t"], 3) if len(s) > 1 else 0.0}
        if self.error:
            out["error"] = self.error
        if not s:
            return out
        # The reading in place when the window opened describes the time
        # before it: use only readings refreshed inside the window, each once.
        fresh = {}
        for x in s:
            if x["stamp"] != s[0]["stamp"]:
                fresh.setdefault(x["stamp"], x)
        out["readings_used"] = len(fresh) if fresh else 1
        if not fresh:
            out["note"] = "no refresh of the table inside the window: the one reading predates it"
        r = list(fresh.values()) if fresh else s[:1]

        def stat(key, scale=1.0):
            v = [x[key] for x in r if x[key] is not None]
            if not v:
                return None
            return {"mean": round(sum(v) / len(v) * scale, 3), "min": round(min(v) * scale, 3),
                    "max": round(max(v) * scale, 3)}

        out["gfx_clock_ghz"] = stat("gfx_mhz", 1e-3)
        out["mem_clock_mhz"] = stat("uclk_mhz")
        out["socket_power_w"] = stat("power_w")
        out["hotspot_c"] = stat("hotspot_c")
        out["hbm_c"] = stat("hbm_c")
        out["power_cap_w"] = self.power_cap_w
        a0, a1 = s[0], s[-1]
        if None not in (a0["ppt_acc"], a1["ppt_acc"], a0["acc"], a1["acc"]) and a1["acc"] > a0["acc"]:
            out["at_power_limit_fraction"] = round((a1["ppt_acc"] - a0["ppt_acc"]) / (a1["acc"] - a0["acc"]), 3)
        return out

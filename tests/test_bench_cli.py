"""bench.py's command line on the CPU: it measures one GPU and refuses more."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_amd_smi_reading_is_parsed_and_failures_give_none(monkeypatch):
    # bench.py's gpu_state reads `amd-smi metric -g 0 -c -p --json`: the gfx clock of every XCD
    # and the socket power; a missing tool, a failed call or other output gives None
    import json
    import subprocess as sp

    sys.path.insert(0, ROOT)
    import bench

    gfx = {f"gfx_{i}": {"clk": {"value": 2000 + i, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"}}
           for i in range(8)}
    reply = {"gpu_data": [{"gpu": 0, "power": {"socket_power": {"value": 1376, "unit": "W"}},
                           "clock": dict(gfx, mem_0={"clk": {"value": 2000, "unit": "MHz"}}, fclk_0={"clk": "N/A"})}]}

    class Done:
        def __init__(self, rc, out):
            self.returncode, self.stdout = rc, out

    monkeypatch.setattr(bench.shutil, "which", lambda name: "/opt/rocm/bin/amd-smi")
    monkeypatch.setattr(bench.subprocess, "run", lambda *a, **k: Done(0, "warning line\n" + json.dumps(reply)))
    s = bench._smi_sample()
    assert s == {"gfx_mhz": [2000.0 + i for i in range(8)], "power_w": 1376.0}
    monkeypatch.setattr(bench.subprocess, "run", lambda *a, **k: Done(1, ""))
    assert bench._smi_sample() is None
    monkeypatch.setattr(bench.subprocess, "run", lambda *a, **k: Done(0, "{\"gpu_data\": []}"))
    assert bench._smi_sample() is None

    def timeout(*a, **k):
        raise sp.TimeoutExpired("amd-smi", 30)

    monkeypatch.setattr(bench.subprocess, "run", timeout)
    assert bench._smi_sample() is None
    monkeypatch.setattr(bench.shutil, "which", lambda name: None)
    assert bench._smi_sample() is None

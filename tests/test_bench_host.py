"""Host-side pieces of bench.py: argument contract, the amd-smi clock parser
and the single-core oracle child (CPU only)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

AMD_SMI_TEXT = """GPU: 0
    CLOCK:
        GFX_0:
            CLK: 1945 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        GFX_1:
            CLK: 1888 MHz
        MEM_0:
            CLK: 2000 MHz
            MIN_CLK: 900 MHz
        VCLK_0:
            CLK: 59 MHz
    POWER:
        SOCKET_POWER: 1366 W
"""


def test_parse_amd_smi_clocks():
    r = bench.parse_amd_smi_clocks(AMD_SMI_TEXT)
    assert r["sclk_mhz_min"] == 1888 and r["sclk_mhz_max"] == 1945
    assert r["mclk_mhz"] == 2000
    assert r["socket_power_w"] == 1366.0
    assert r["clocks_mhz"] == {"GFX_0": 1945, "GFX_1": 1888, "MEM_0": 2000, "VCLK_0": 59}


def test_parse_amd_smi_clocks_without_gfx():
    assert "error" in bench.parse_amd_smi_clocks("GPU: 0\n    POWER:\n        SOCKET_POWER: N/A\n")


def test_multi_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_single_core_oracle_child():
    r = bench.cpu_baseline_single_core("c1", 32)
    assert "error" not in r, r
    assert r["cores"] == 1 and r["kind"] == "oracle" and r["value"] > 0

"""Host-side logic of bench.py that needs no GPU: the amd-smi power / clock parser."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402

SAMPLE = """GPU: 0
    POWER:
        SOCKET_POWER: 1316 W
        GFX_VOLTAGE: N/A
    CLOCK:
        GFX_0:
            CLK: 2061 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
            CLK_LOCKED: DISABLED
        GFX_1:
            CLK: 1995 MHz
            MIN_CLK: 500 MHz
            MAX_CLK: 2400 MHz
        MEM_0:
            CLK: 1900 MHz
            MIN_CLK: 900 MHz
        VCLK_0:
            CLK: 29 MHz
"""


def test_parse_smi_power_reads_socket_power_and_gfx_clocks_only():
    power, clocks = bench._parse_smi_power(SAMPLE)
    assert power == 1316.0
    # the memory and video clocks, and the MIN/MAX limits, are not GFX clocks
    assert clocks == [2061.0, 1995.0]


def test_parse_smi_power_missing_fields():
    assert bench._parse_smi_power("") == (None, [])
    assert bench._parse_smi_power("GPU: 0\n    POWER:\n        SOCKET_POWER: N/A\n") == (None, [])

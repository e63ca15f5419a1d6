"""GPU: the conversion instructions the quantizers and GEMMs use agree with
the library's software encoders (which the parity tests pin to the oracle)
on every fp32 input: E2M1 round-to-nearest and stochastic rounding, E4M3 on
inputs clamped to +-448, and the FP4 / FP8 / NVFP4-to-fp16 decoders. The
sweep itself is tests/helpers/hw_convert_check.hip, built by build()."""
import json
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "helpers", "hw_convert_check")


def test_hardware_converts_match_software_encoders():
    assert os.path.exists(BIN), "tests/helpers/hw_convert_check is missing: run __graft_entry__.build()"
    print("running exhaustive hardware-convert sweep", flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=100)
    print(res.stdout, flush=True)
    out = json.loads(res.stdout.strip().splitlines()[-1])
    bad = {k: v for k, v in out.items() if v["mismatches"] != 0}
    assert not bad, f"hardware converts differ from the software encoders: {bad}"
    assert res.returncode == 0

"""The library driven from plain C (tests/c_abi_roundtrip.c, built by the
package build step): layout, notify, dispatch, combine, the grouping by expert
and the fp8 path (quantiser, quantising dispatch and its cached mode,
dequantiser) through include/ep.h with device memory from the HIP runtime
alone, checked on the host for properties that hold for any routing."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROGRAM = os.path.join(ROOT, "tests", "c_abi_roundtrip")

pytestmark = pytest.mark.gpu


def test_c_program_round_trip():
    assert os.path.exists(PROGRAM), "tests/c_abi_roundtrip is not built: run the package build step first"
    print("[c abi] running tests/c_abi_roundtrip", flush=True)
    p = subprocess.run([PROGRAM], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "c abi roundtrip ok" in p.stdout, p.stdout

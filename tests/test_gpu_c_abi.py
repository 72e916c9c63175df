"""The C ABI used from plain C: tests/c/ep_roundtrip.c (layout, bf16 dispatch
and combine through include/ep.h alone, identity experts, weights summing to
one) must return every token bit for bit on the GPU."""
import subprocess

import pytest

from test_abi import compile_c_roundtrip

pytestmark = pytest.mark.gpu


def test_c_program_round_trip(tmp_path):
    exe = str(tmp_path / "ep_roundtrip")
    r = compile_c_roundtrip(exe)
    assert r.returncode == 0, r.stderr
    print("[gpu-c-abi] running %s" % exe, flush=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(run.stdout.strip(), flush=True)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ep_roundtrip: ok" in run.stdout

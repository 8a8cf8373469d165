"""The hardware E4M3 encoder against the library's software encoder, and the
FP8 quantizers' division-free quotient code against the divided one.

Runs ``tests/e4m3_encoder_check`` (built with the library from
``tests/e4m3_encoder_check.hip``): every finite fp32 input below 464 in
magnitude, both signs, through both encoders; then 2^35 random quotients of
a row value by its row scale, through ``e4m3_of_quotient`` and through an
fp32 division plus the software encoder.  Both must agree everywhere: the
FP8 append and scatter take their codes from the fast path.
"""

import os
import subprocess

import pytest

from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "e4m3_encoder_check")


def test_e4m3_hardware_encoder_and_fast_quotient():
    if not os.path.exists(EXE):
        raise RuntimeError(f"{EXE} is missing: build the library first (__graft_entry__.build())")
    say("e4m3 encoder check: every finite |x| < 464, then random quotients")
    proc = subprocess.run([EXE], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=100)
    say(proc.stdout.strip())
    assert proc.returncode == 0, proc.stdout
    assert "encoder: 0 of" in proc.stdout and "quotient: 0 of" in proc.stdout

"""The C ABI's host code under AddressSanitizer (no GPU).

A copy of the library is built with AddressSanitizer on its host half (the
argument checks, the launch set-up and the precondition checks run on the
CPU; device code is unchanged), then the C-ABI tests and the validator tests
run against it in a child process with the sanitizer runtime preloaded.  Any
invalid host memory access in those paths ends the child with a report.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_and_validators_under_asan():
    from yoco_shared_kv_gather_amd import build

    try:
        lib = build.build_asan()
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"no AddressSanitizer build here: {e}")
    symbols = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_init" in symbols                      # the copy's host code is instrumented
    env = dict(os.environ)
    env.update({
        "YOCO_LIBRARY": lib,
        "LD_PRELOAD": runtime,
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0:alloc_dealloc_mismatch=0",
    })
    probe = subprocess.run([sys.executable, "-c", "from yoco_shared_kv_gather_amd import binding as yb; "
                            "yb.lib(); print(yb.library_path()); "
                            "maps = open('/proc/self/maps').read(); "
                            "print('libclang_rt.asan' in maps and yb.library_path() in maps)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.split() == [lib, "True"], probe.stdout
    proc = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "tests/test_abi.py",
                           "tests/test_validate.py", "tests/test_tile_addressing.py",
                           "tests/test_zz_no_alloc.py", "-m", "not gpu"],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = proc.stdout + proc.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert proc.returncode == 0, out[-4000:]
    assert " passed" in proc.stdout

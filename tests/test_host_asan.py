"""The host half of libdg under AddressSanitizer, without a GPU.

The same sources are built with the sanitizer on the host compilation only
(build.build_host_asan: the GPU code is compiled as usual), and the CPU tests
of the C ABI (tests/test_abi.py: model creation and layout, argument
validation of every entry point, the host sampler arithmetic over every
sampler input) run against that build in a child process that preloads the
sanitizer runtime.  Any heap, stack or global out-of-bounds access, use after
free or double free in the host runtime aborts the child with a report."""
import os
import subprocess
import sys

import pytest

from discrete_diffusion_decoding_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHECK_LOADED = """
import ctypes, os, sys
from discrete_diffusion_decoding_amd import dg
dg.lib()
assert dg._LIB_PATH == os.environ["DG_LIBRARY"], dg._LIB_PATH
ctypes.CDLL(None).__asan_init  # the sanitizer runtime is live in this process
print("asan build loaded")
"""


def test_host_runtime_clean_under_address_sanitizer():
    try:
        rt = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = build.build_host_asan(verbose=False)
    env = dict(os.environ, LD_PRELOAD=rt, DG_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1")
    env["PYTHONPATH"] = ROOT + os.pathsep + env.get("PYTHONPATH", "")
    r = subprocess.run([sys.executable, "-c", _CHECK_LOADED], env=env, cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "asan build loaded" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-6000:]
    assert "AddressSanitizer" not in r.stderr, r.stderr[-6000:]
    assert " passed" in r.stdout and " failed" not in r.stdout, r.stdout[-3000:]

"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, no GPU code).

- The oracle, built with ``-fsanitize=address,undefined``, runs every pin of ``pins.py``.
- The C ABI's host side (``conv1d_api.cpp``: validation, spans, workspace sizing), built with g++
  and the same sanitizers against launch stubs that abort, runs ``test_abi.py``.  Every ABI case
  must be decided on the host without reaching a launch, with no sanitizer report.

Each run happens in a child process with the sanitizer runtimes preloaded.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.join(ROOT, "tests")
CSRC = os.path.join(ROOT, "causal_depthwise_conv1d_width_amd", "csrc")
SAN = ("-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-g")


def _runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _child(code, tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc sanitizer runtimes not installed")
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0",
               OMP_NUM_THREADS="4", PYTHONPATH=os.pathsep.join([ROOT, TESTS]))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, cwd=str(tmp_path),
                       timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    return r.stdout


def test_oracle_pins_under_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    code = f"""
from oracle import Oracle
from oracle.build import build
import pins
o = Oracle(build(out={lib!r}, extra={SAN!r}))
for p in pins.ALL_PINS:
    p(o)
print("pins", len(pins.ALL_PINS))
"""
    assert f"pins" in _child(code, tmp_path)


def test_abi_host_validation_under_sanitizers(tmp_path):
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    if not os.path.exists(os.path.join(rocm, "include", "hip", "hip_runtime.h")):
        pytest.skip("HIP headers not installed")
    lib = str(tmp_path / "libapi_san.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-fPIC", "-shared", *SAN, "-D__HIP_PLATFORM_AMD__",
                    f"-I{rocm}/include", f"-I{ROOT}/include", f"-I{CSRC}", os.path.join(CSRC, "conv1d_api.cpp"),
                    os.path.join(TESTS, "host_stub_launch.cpp"), "-o", lib], check=True, capture_output=True)
    code = f"""
import sys
import pytest
from causal_depthwise_conv1d_width_amd import _lib
_lib.LIB_PATH = {lib!r}
_lib.load.__defaults__ = ({lib!r},)
assert _lib.load()._name == {lib!r}
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {os.path.join(TESTS, "test_abi.py")!r}]))
"""
    out = _child(code, tmp_path)
    assert "passed" in out and "failed" not in out

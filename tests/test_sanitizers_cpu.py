"""Host sanitizer runs (CPU only, no GPU code executes).

* The fp64 oracle (``oracle/efla_oracle.c``) built with gcc and
  AddressSanitizer + UndefinedBehaviorSanitizer, driven through every exported
  routine by ``tests/sanitize/oracle_driver.c``.
* The C ABI's host validation layer (``csrc/efla_api.hip``) built for the host
  with the same sanitizers (the device side gets none), with the kernel launch
  entry points replaced by counting stubs (``tests/sanitize/abi_driver.cpp``):
  valid calls reach exactly one launch, invalid ones return their status with
  none.

Any sanitizer report is fatal (-fno-sanitize-recover=all), so a clean exit is
the pass condition.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def test_oracle_under_asan_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=all", os.path.join(ROOT, "oracle", "efla_oracle.c"),
          os.path.join(SAN, "oracle_driver.c"), "-lm", "-lpthread", "-o", exe])
    r = _run([exe])
    assert "0 failed checks" in r.stdout


def test_abi_validation_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path / "abi_san")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all"]
    _run([HIPCC, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *san,
          "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "delta_rule_recurrent_efla_amd", "csrc", "efla_api.hip"),
          os.path.join(SAN, "abi_driver.cpp"), "-o", exe])
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    r = _run([exe], env=env)
    assert "0 failed checks" in r.stdout

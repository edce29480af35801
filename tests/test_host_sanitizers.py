"""Host AddressSanitizer / UndefinedBehaviorSanitizer build of the C ABI's argument validation.

The C ABI source (aqlm_api.hip) is compiled with the sanitizers on its host pass
only, together with tests/host_sanitize/api_validation_driver.hip, which replaces
every kernel launcher with a counting stub and calls every entry point with valid,
NULL, misaligned and extreme arguments (INT64_MIN/MAX sizes, host arrays of exactly
n_layers entries).  No GPU is touched.  A second build plants a host-array
over-read and must be stopped by AddressSanitizer, which shows the build is armed.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
API = os.path.join(ROOT, "extreme_weight_quantization_amd", "csrc", "aqlm_api.hip")
DRIVER = os.path.join(ROOT, "tests", "host_sanitize", "api_validation_driver.hip")


def _hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc not available")


def _build(tmp_path, name, extra=()):
    exe = str(tmp_path / name)
    # sanitizers on the host pass only (each -fsanitize= right after -Xarch_host)
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           *extra, API, DRIVER, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    return subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)


def test_api_validation_is_clean_under_asan_and_ubsan(tmp_path):
    r = _run(_build(tmp_path, "api_check"))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "api validation ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_sanitizer_build_catches_a_planted_overread(tmp_path):
    r = _run(_build(tmp_path, "api_check_planted", ("-DAQLM_PLANT_OVERREAD",)))
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr

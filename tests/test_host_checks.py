"""Host-only checks of library code: tests/native/host_checks.hip includes the
shipped csrc/topk.hpp and is compiled for the host (hipcc, no device code),
so the GPU kernels' own key-interval and certificate functions are checked
on the CPU:

* every one of the 2^32 order-preserving score keys against the digit
  intervals the top-k kernels classify with (monotone digit, key inside
  [digit_lo_key(d), digit_hi_key(d)], intervals tiling the key space);
* the candidate-list certificate verdicts, including a list of exactly k
  candidates under a finite threshold (it must be counted, not taken whole);
* the relative bins of candidate lists over every coarse key (monotone bins,
  each key inside its bin's interval, the reached bins tiling the key space).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "host_checks.hip")
CSRC = os.path.join(ROOT, "long_context_pool_amd", "csrc")
BUILD = os.path.join(ROOT, "tests", "native", "_build")
EXE = os.path.join(BUILD, "host_checks")


@pytest.fixture(scope="module")
def host_checks():
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    os.makedirs(BUILD, exist_ok=True)
    subprocess.check_call([hipcc, "-x", "hip", "--offload-host-only", "-O2", "-std=c++17",
                           "-I", CSRC, SRC, "-o", EXE, "-pthread"])
    return EXE


def _run(exe, what):
    r = subprocess.run([exe, what], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


def test_certificate_verdicts(host_checks):
    assert "ok certificate" in _run(host_checks, "certificate")


def test_digit_intervals_over_all_keys(host_checks):
    out = _run(host_checks, "digits")
    assert "ok digits" in out
    # Every non-NaN float image: 2^32 - 2 * (2^23 - 1) NaN patterns - 1 (the
    # key of -0 is that of +0).
    assert f"({2**32 - 2 * (2**23 - 1) - 1} keys)" in out


def test_relative_bins_over_all_coarse_keys(host_checks):
    assert "ok relbins" in _run(host_checks, "relbins")

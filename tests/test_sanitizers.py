"""Host code under sanitizers (no GPU): the CPU oracle built with
AddressSanitizer + UndefinedBehaviorSanitizer and, separately, with
ThreadSanitizer (it runs one work item per thread over a shared counter), and
the library's host layer (argument validation of every entry point and the
planner, the source that ships in libgdn.so) built with AddressSanitizer +
UndefinedBehaviorSanitizer on the host side only.  Each build runs a driver
under tests/sanitize/ and must finish with exit status 0 and no sanitizer
report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "chunked_gated_delta_prefill_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", TSAN_OPTIONS="halt_on_error=1")
REPORT_MARKERS = ("ERROR: AddressSanitizer", "runtime error:", "WARNING: ThreadSanitizer", "ERROR: ThreadSanitizer")


def _run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    text = r.stdout + r.stderr
    assert r.returncode == 0, text[-4000:]
    for m in REPORT_MARKERS:
        assert m not in text, text[-4000:]
    return text


def _build(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("kind", ["address,undefined", "thread"])
def test_oracle_under_sanitizers(tmp_path, kind):
    exe = str(tmp_path / "oracle_driver")
    _build(["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", f"-fsanitize={kind}",
            "-fno-sanitize-recover=all", os.path.join(ROOT, "oracle", "gdn_oracle.c"),
            os.path.join(SAN, "oracle_driver.c"), "-o", exe, "-lpthread", "-lm"])
    assert "oracle driver: ok" in _run(exe)


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="needs hipcc")
def test_host_layer_under_sanitizers(tmp_path):
    """gdn_api.hip with host-side ASan + UBSan (the kernels replaced by stand-ins
    that are never reached without a GPU)."""
    exe = str(tmp_path / "abi_driver")
    host_san = []
    for f in ("address", "undefined"):
        host_san += ["-Xarch_host", f"-fsanitize={f}"]
    _build(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fno-omit-frame-pointer",
            *host_san, "-Xarch_host", "-fno-sanitize-recover=all",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            os.path.join(CSRC, "gdn_api.hip"), os.path.join(SAN, "launch_stubs.hip"),
            os.path.join(SAN, "abi_driver.cpp"), "-o", exe])
    assert "host layer driver: ok" in _run(exe)

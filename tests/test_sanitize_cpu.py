"""Sanitizer builds of the host code (no GPU).

- The host side of the C ABI (argument validation, the workspace layout, the
  router's launch plan, the expert FFN's gather rule) built with AddressSanitizer and UndefinedBehavior-
  Sanitizer against launcher stubs that read the first and last byte of every
  buffer a launch touches, every "device" buffer a host allocation of the
  size the header documents (tests/sanitize/abi_host_check.cpp).  A planted
  layout mistake (two workspace regions overlapping) must be caught.
- The CPU oracle (oracle/moe_oracle.c) built with the same sanitizers and
  driven by its own pin tests, in a child process that preloads the
  AddressSanitizer runtime.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mixture_experts_layer_09_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
# host code only; every sanitizer flag applies to the host compilation
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all"]


def _need(tool):
    if not os.path.exists(tool) and not shutil.which(tool):
        pytest.skip(f"{tool} not available")


def _build_abi_check(root, out):
    cmd = [HIPCC, "-x", "hip", "--offload-host-only", "-O1", "-g", "-std=c++17",
           "-fno-omit-frame-pointer", *SAN, "-I", os.path.join(root, "include"),
           os.path.join(root, "mixture_experts_layer_09_amd", "csrc", "moe_api.cpp"),
           os.path.join(root, "mixture_experts_layer_09_amd", "csrc", "route_plan.cpp"),
           os.path.join(root, "mixture_experts_layer_09_amd", "csrc", "ffn_plan.cpp"),
           os.path.join(root, "tests", "sanitize", "abi_host_check.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    _need(HIPCC)
    exe = str(tmp_path / "abi_check")
    _build_abi_check(ROOT, exe)
    r = _run(exe)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "failures: 0, overlapping workspace regions: 0" in r.stdout


def test_abi_host_check_catches_an_overlapping_region(tmp_path):
    """A copy of the sources whose layout gives Yp half its bytes: the
    expert FFN's Yp then overlaps Ys, and the check must fail."""
    _need(HIPCC)
    root = tmp_path / "tree"
    for rel in ("include/moe.h", "mixture_experts_layer_09_amd/csrc/moe_api.cpp",
                "mixture_experts_layer_09_amd/csrc/route_plan.cpp",
                "mixture_experts_layer_09_amd/csrc/ffn_plan.cpp",
                "mixture_experts_layer_09_amd/csrc/moe_internal.h",
                "tests/sanitize/abi_host_check.cpp"):
        dst = root / rel
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, rel), dst)
    h = root / "mixture_experts_layer_09_amd/csrc/moe_internal.h"
    src = h.read_text()
    good = "L.Yp = take(rows * h * act_bytes(s.precision));"
    assert good in src
    h.write_text(src.replace(good, "L.Yp = take(rows * h * act_bytes(s.precision) / 2);"))
    exe = str(tmp_path / "abi_check_bad")
    _build_abi_check(str(root), exe)
    r = _run(exe)
    assert r.returncode != 0
    assert "workspace regions overlap" in r.stderr


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not available")
    asan = subprocess.run([gcc, "-print-file-name=libasan.so"], capture_output=True,
                          text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("no AddressSanitizer runtime")
    so = str(tmp_path / "liboracle_san.so")
    subprocess.check_call([gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fopenmp", "-fPIC", "-shared", "-o", so,
                           os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm"])
    env = dict(os.environ, MOE_ORACLE_LIB=so, LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    probe = subprocess.run([sys.executable, "-c", "import oracle; oracle.lib(); print(oracle._LIB_PATH)"],
                           capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip() == so, probe.stderr[-2000:]
    # the pins call every oracle function; the planted-mistake tests build
    # other copies of the oracle and are left out
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-k", "not planted", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_backward_pins.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out

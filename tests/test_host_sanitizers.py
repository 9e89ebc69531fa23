"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The library's host code (argument validation, workspace plans, dispatch),
  compiled with hipcc with the sanitizers on the host pass only
  (``-Xarch_host -fsanitize=...``; device code is built as usual and never
  runs here), linked with tests/sanitize/abi_checks.cpp, which drives every
  validation path of every entry point without reaching a launch.
* The float64 oracle compiled with gcc and the sanitizers, driven by
  tests/sanitize/oracle_checks.c over small shapes and the edge cases.
Any sanitizer report or failed check fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "selective_state_space_vjp_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LIB_SOURCES = ["abi.cpp", "scan_seq.hip", "ssd_chunk.hip", "ssd_chunk16.hip", "ssd_blocked.hip", "ssd_fwd.hip",
               "delta_rule.hip", "noalloc.hip", "finite.hip", "ssd_pad.hip"]
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout[-4000:]}\n{res.stderr[-4000:]}"
    return res


def _clean(res):
    text = res.stdout + res.stderr
    for marker in ("ERROR: AddressSanitizer", "ERROR: LeakSanitizer", "runtime error:"):
        assert marker not in text, text[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_checks")
    _run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
          "-fno-sanitize-recover=undefined", "-static-libasan", "-o", exe, os.path.join(ROOT, "oracle", "ssm_oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_checks.c"), "-lm"])
    res = _run([exe], env=SAN_ENV, timeout=300)
    _clean(res)
    assert "0 failure(s)" in res.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_abi_host_code_under_sanitizers(tmp_path):
    flags = ["-O1", "-g", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include")]
    objs = []
    procs = []
    sources = [os.path.join(CSRC, s) for s in LIB_SOURCES] + [os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp")]
    for src in sources:
        obj = str(tmp_path / (os.path.basename(src).split(".")[0] + ".o"))
        objs.append(obj)
        procs.append(subprocess.Popen([HIPCC, "-x", "hip", "-c", src, "-o", obj] + flags,
                                      stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True))
    for p in procs:
        out, err = p.communicate()
        assert p.returncode == 0, err[-4000:]
    exe = str(tmp_path / "abi_checks")
    _run([HIPCC, "-fsanitize=address,undefined", "--offload-arch=gfx950", "-o", exe] + objs)
    env = dict(SAN_ENV)
    env.pop("SSMVJP_CHECK_FINITE", None)
    res = _run([exe], env=env, timeout=300)
    _clean(res)
    assert "0 failure(s)" in res.stdout

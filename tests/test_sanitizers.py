"""CPU tier under AddressSanitizer and UndefinedBehaviorSanitizer: the oracle
(plain C, built with gcc) and the library's host code (argument checks,
workspace plans, options; device code is compiled but never run) each driven
by a small program under tests/sanitize/. Any sanitizer report aborts the
driver, and a failed check makes it exit non-zero."""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "sparse_attention_long_anchor_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ENV = dict(os.environ, ASAN_OPTIONS="abort_on_error=1:detect_leaks=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed ({r.returncode}):\n{r.stdout[-3000:]}\n{err[-3000:]}"
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    # serial build (OpenMP pragmas ignored): the sanitizers see one thread's accesses
    _run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-Wall", "-Wno-unknown-pragmas", "-o", exe,
          os.path.join(SAN, "oracle_driver.c"), os.path.join(ROOT, "oracle", "kascade_oracle.c"), "-lm"])
    out = _run([exe], env=ENV)
    assert "0 failure(s)" in out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_library_host_code_under_asan_ubsan(tmp_path):
    # sanitizers on the host pass only (each -fsanitize= right after -Xarch_host);
    # the device pass is built unoptimised since nothing here launches it
    flags = ["-std=c++17", "-O1", "-g", "-fPIC", "--offload-arch=gfx950",
             "-Xarch_host", "-fsanitize=address,undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_device", "-O0",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    srcs = ["kascade_api.hip", "decode_kernels.hip", "prefill_kernels.hip"]

    def obj(src):
        o = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        _run([HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", o])
        return o

    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(obj, srcs))
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, *flags, "-x", "hip", os.path.join(SAN, "abi_driver.cpp"), "-x", "none", *objs, "-o", exe])
    # the HIP runtime keeps allocations until exit: leak checking is off for this driver
    env = dict(ENV, ASAN_OPTIONS="abort_on_error=1:detect_leaks=0", HIP_VISIBLE_DEVICES="")
    out = _run([exe], env=env)
    assert "0 failure(s)" in out

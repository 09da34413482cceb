"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU oracle
and of libtg's host code, run on the CPU.

* The oracle (oracle/tgref.c, oracle/tgref_attention.c) with a driver that
  allocates every operand at exactly its footprint (tests/sanitize/
  oracle_driver.c); a build of the same driver with one operand an element
  short must be reported by the sanitizer.
* The host code (tiled_dense_gemm_08_amd/csrc/tg_api.cpp: validation, plans,
  the tuning-cache parser, attention argument checks) with a driver of
  random plans, bad arguments and tuning files loaded while other threads
  plan (tests/sanitize/host_driver.cpp), linked against stand-ins for the
  kernel side (tests/sanitize/kernel_stubs.cpp) whose configuration table
  is checked here against the built library's.
"""
import os
import shutil
import subprocess

import pytest

import tiled_dense_gemm_08_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "tiled_dense_gemm_08_amd", "csrc")
ROCM = "/opt/rocm"
CLANG = os.path.join(ROCM, "llvm", "bin", "clang++")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or not os.path.exists(CLANG),
                                reason="needs gcc and ROCm's clang")


def sh(cmd, cwd):
    r = subprocess.run(cmd, cwd=cwd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, " ".join(cmd) + "\n" + r.stdout[-4000:]


def oracle_driver(tmp, extra=()):
    exe = os.path.join(tmp, "oracle_san" + "".join(extra).replace("-D", "_"))
    sh(["gcc", "-O1", "-g", "-pthread", "-ffp-contract=off"] + SAN_FLAGS + list(extra) +
       ["-o", exe, os.path.join(SAN, "oracle_driver.c"),
        os.path.join(ROOT, "oracle", "tgref.c"), os.path.join(ROOT, "oracle", "tgref_attention.c"),
        "-lm"], tmp)
    return exe


def test_oracle_under_sanitizers(tmp_path):
    exe = oracle_driver(str(tmp_path))
    r = subprocess.run([exe], env=ENV, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                       timeout=300)
    assert r.returncode == 0 and "oracle driver ok" in r.stdout, r.stderr[-4000:]
    assert r.stderr == ""


def test_sanitizer_reports_a_planted_short_buffer(tmp_path):
    exe = oracle_driver(str(tmp_path), ["-DTG_PLANT_SHORT_BUFFER"])
    r = subprocess.run([exe], env=ENV, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                       timeout=300)
    assert r.returncode != 0
    assert "heap-buffer-overflow" in r.stderr


@pytest.fixture(scope="module")
def host_driver(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("hostsan"))
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + CSRC, "-I" + os.path.join(ROCM, "include"),
           "-D__HIP_PLATFORM_AMD__"]
    base = ["-O1", "-g", "-std=c++20"]
    sh([CLANG] + base + SAN_FLAGS + inc + ["-c", "-o", "drv.o",
                                           os.path.join(SAN, "host_driver.cpp")], tmp)
    sh([CLANG] + base + SAN_FLAGS + inc + ["-c", "-o", "stubs.o",
                                           os.path.join(SAN, "kernel_stubs.cpp")], tmp)
    # the library's host code as hipcc compiles it, host side only, with the
    # sanitizers on the host compilation
    xh = []
    for f in SAN_FLAGS:
        xh += ["-Xarch_host", f]
    sh([HIPCC] + base + ["--offload-arch=gfx950", "--cuda-host-only", "-fPIC"] + xh + inc +
       ["-c", "-o", "api.o", os.path.join(CSRC, "tg_api.cpp")], tmp)
    exe = os.path.join(tmp, "host_san")
    sh([CLANG] + SAN_FLAGS + ["-o", exe, "drv.o", "api.o", "stubs.o",
                              "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
                              "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-pthread"], tmp)
    return exe, tmp


def test_host_code_under_sanitizers(host_driver):
    exe, tmp = host_driver
    r = subprocess.run([exe, tmp], env=ENV, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                       text=True, timeout=600)
    assert r.returncode == 0 and "host driver ok" in r.stdout, r.stderr[-4000:]
    # its configuration table is the library's
    rows = [l.split()[1:] for l in r.stdout.splitlines() if l.startswith("config ")]
    fields = ["id", "block_m", "block_n", "block_k", "stages", "waves_m", "waves_n", "mfma",
              "direct_lds", "lds_bytes", "ops", "elem_bytes", "whole_k", "name"]
    lib_rows = [[str(c[f]) for f in fields] for c in tg.configs()]
    assert rows == lib_rows

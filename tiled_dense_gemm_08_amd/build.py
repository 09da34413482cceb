"""Build libtg.so for gfx950 in-tree with hipcc.

    python tiled_dense_gemm_08_amd/build.py          # library
    python tiled_dense_gemm_08_amd/build.py --asm    # also write the device asm
                                                     # and print register use

(run by path: importing the package itself needs the built library)

The device assembly is also checked for M0: the direct-load kernels write M0
from inline assembly right before each global->LDS copy, so no other
instruction of the kernels may read or write it.
"""
import argparse
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtg.so")
SOURCES = [os.path.join(CSRC, "tg_api.cpp"), os.path.join(CSRC, "tg_kernels.hip")]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
FLAGS = ["-O3", "-std=c++20", "--offload-arch=" + ARCH,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wno-unused-command-line-argument"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "hip-link" not in l)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("build failed: " + " ".join(cmd))
    return out


def build_lib():
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC] + FLAGS + ["-fPIC", "-shared", "-o", tmp] + SOURCES)
    os.replace(tmp, LIB)
    return LIB


def device_asm(path=None):
    path = path or os.path.join(HERE, "_build", "tg_kernels.s")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    _run([HIPCC] + FLAGS + ["--cuda-device-only", "-S", "-o", path,
                            os.path.join(CSRC, "tg_kernels.hip")])
    return path


def check_m0(asm_text):
    """Every M0 use must be `s_mov_b32 m0, sX` directly followed by a
    buffer_load ... lds (the copy that consumes it)."""
    lines = [l.strip() for l in asm_text.splitlines()
             if l.strip() and not l.strip().startswith((";", "."))]
    bad = []
    for i, l in enumerate(lines):
        if re.search(r"\bm0\b", l):
            ok = (l.startswith("s_mov_b32 m0,") and i + 1 < len(lines)
                  and lines[i + 1].startswith("buffer_load_dword") and lines[i + 1].endswith("lds"))
            if not ok:
                bad.append(l)
    return bad


def resource_report(asm_text):
    rows = []
    # amdhsa metadata blocks list name, vgpr/agpr/sgpr counts and spill counts
    for blk in asm_text.split("  - .agpr_count:")[1:]:
        get = lambda k: (re.search(r"\." + k + r":\s+(\S+)", blk) or [None, "?"])[1]
        rows.append((get("name"), "agpr=" + blk.split()[0], "vgpr=" + get("vgpr_count"),
                     "sgpr=" + get("sgpr_count"), "lds=" + get("group_segment_fixed_size"),
                     "spill_v=" + get("vgpr_spill_count"), "spill_s=" + get("sgpr_spill_count")))
    return rows


def build(asm=False):
    lib = build_lib()
    if asm:
        path = device_asm()
        text = open(path).read()
        bad = check_m0(text)
        for r in resource_report(text):
            print(" ".join(r))
        if bad:
            raise RuntimeError("unexpected M0 uses in device code: %s" % bad[:5])
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    a = ap.parse_args()
    print(build(asm=a.asm))

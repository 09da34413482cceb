"""Build the CPU oracle's shared library (test infrastructure).

gcc -O2, never -ffast-math: the oracle's sums must round exactly as written.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "tgref.c")
SOURCES = [SRC, os.path.join(HERE, "tgref_attention.c")]
LIB = os.path.join(HERE, "libtgref.so")


def build(force=True):
    if (not force and os.path.exists(LIB) and
            os.path.getmtime(LIB) >= max(os.path.getmtime(s) for s in SOURCES)):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
                    "-ffp-contract=off", "-Wall", "-Wextra", "-o", tmp] + SOURCES + ["-lm"],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())

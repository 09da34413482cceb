"""Build libtg.so for gfx950 in-tree with hipcc, and its LDS-poison debug
twin libtg_poison.so (the same sources with -DTG_LDS_POISON: LDS is filled
with NaN before every write of it, so a read of LDS bytes that the current K
step did not write shows up as NaN in C; the GPU tests compare it with the
normal library bit for bit).

    python tiled_dense_gemm_08_amd/build.py          # both libraries
    python tiled_dense_gemm_08_amd/build.py --asm    # also write the device asm
                                                     # and print register use

(run by path: importing the package itself needs the built library)

The device assembly can also be checked for M0 (check_m0): the direct-load
kernels write M0 from inline assembly right before each global->LDS copy, so
no other instruction of the kernels may read or write it;
tests/test_device_asm_cpu.py runs that check and the spill check.
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
POISON_LIB = os.path.join(HERE, "libtg_poison.so")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
FLAGS = ["-O3", "-std=c++20", "--offload-arch=" + ARCH,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + INCLUDE, "-I" + CSRC, "-Wall", "-Wno-unused-command-line-argument"]


SHARDS = 8   # kernel compilations run in parallel (tg_kernels.hip, TG_SHARD=i)
ATTN = os.path.join(CSRC, "tg_attention.hip")
PACK = os.path.join(CSRC, "tg_pack.hip")
CEILING = os.path.join(CSRC, "tg_ceiling.hip")
STATIC = os.path.join(CSRC, "tg_static.hip")
BUILD_DIR = os.path.join(HERE, "_build")


def _filter(out):
    return "\n".join(l for l in out.splitlines()
                     if "packed-fp32-ops" not in l and "hip-link" not in l)


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = _filter(r.stdout)
    if r.returncode != 0:
        sys.stderr.write(out + "\n")
        raise RuntimeError("build failed: " + " ".join(cmd))
    return out


def _run_all(cmds, jobs=None):
    """Run the commands, at most `jobs` (default: the CPUs this process may
    use) at a time; raise if any fails."""
    try:
        jobs = jobs or len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        jobs = jobs or os.cpu_count() or 1
    pending, running, failed = list(cmds), [], []
    while pending or running:
        while pending and len(running) < jobs:
            c = pending.pop(0)
            running.append((c, subprocess.Popen(c, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
        c, pr = running.pop(0)
        out, _ = pr.communicate()
        if pr.returncode != 0:
            failed.append((c, _filter(out)))
    for c, out in failed:
        sys.stderr.write(out + "\n")
    if failed:
        raise RuntimeError("build failed: " + " ".join(failed[0][0]))


def _shard_flags(i):
    return ["-DTG_SHARD=%d" % i, "-DTG_SHARDS=%d" % SHARDS]


def _lib_commands(lib, extra, tag):
    """Object files and compile commands of one library variant."""
    kern = os.path.join(CSRC, "tg_kernels.hip")
    name = os.path.basename(lib)[:-3]
    objs, cmds = [], []
    for i in range(SHARDS):
        o = os.path.join(BUILD_DIR, "%s_kernels_%d.%s.o" % (name, i, tag))
        objs.append(o)
        cmds.append([HIPCC] + FLAGS + extra + _shard_flags(i) + ["-fPIC", "-c", "-o", o, kern])
    for src in (os.path.join(CSRC, "tg_api.cpp"), ATTN, PACK, CEILING, STATIC):
        o = os.path.join(BUILD_DIR, "%s_%s.%s.o" % (name, os.path.basename(src).split(".")[0],
                                                    tag))
        objs.append(o)
        cmds.append([HIPCC] + FLAGS + extra + ["-fPIC", "-c", "-o", o, src])
    return objs, cmds


def build_lib(poison=True):
    """libtg.so and (poison=True) libtg_poison.so; returns the paths."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    tag = "%d" % os.getpid()
    variants = [(LIB, [])] + ([(POISON_LIB, ["-DTG_LDS_POISON"])] if poison else [])
    plan = [(lib,) + _lib_commands(lib, extra, tag) for lib, extra in variants]
    try:
        _run_all([c for _, _, cmds in plan for c in cmds])
        for lib, objs, _ in plan:
            tmp = lib + ".tmp" + tag
            _run([HIPCC, "--offload-arch=" + ARCH, "-fPIC", "-shared", "-o", tmp] + objs)
            os.replace(tmp, lib)
    finally:
        for _, objs, _ in plan:
            for o in objs:
                if os.path.exists(o):
                    os.remove(o)
    return [lib for lib, _ in variants]


def device_asm(path=None):
    """Device assembly of every shard, concatenated into one file."""
    path = path or os.path.join(BUILD_DIR, "tg_kernels.s")
    os.makedirs(os.path.dirname(path), exist_ok=True)
    kern = os.path.join(CSRC, "tg_kernels.hip")
    extra = (ATTN, PACK, CEILING, STATIC)
    parts = [path + ".%d" % i for i in range(SHARDS)] + [path + ".x%d" % i for i in range(len(extra))]
    _run_all([[HIPCC] + FLAGS + _shard_flags(i) + ["--cuda-device-only", "-S", "-o", parts[i], kern]
              for i in range(SHARDS)] +
             [[HIPCC] + FLAGS + ["--cuda-device-only", "-S", "-o", parts[SHARDS + i], src]
              for i, src in enumerate(extra)])
    with open(path, "w") as f:
        for q in parts:
            f.write(open(q).read())
            os.remove(q)
    return path


def check_m0(asm_text):
    """Every M0 use must be a write of it (`s_mov_b32 m0, sX`, or
    `s_add_u32 m0, sX, imm` in the copies that form the address in M0), one
    wait state (`s_nop 0`), then the buffer_load ... lds that consumes it."""
    lines = [l.strip() for l in asm_text.splitlines()
             if l.strip() and not l.strip().startswith((";", "."))]
    bad = []
    for i, l in enumerate(lines):
        if re.search(r"\bm0\b", l):
            ok = (l.startswith(("s_mov_b32 m0,", "s_add_u32 m0,")) and i + 2 < len(lines)
                  and lines[i + 1] == "s_nop 0"
                  and lines[i + 2].startswith("buffer_load_dword") and lines[i + 2].endswith("lds"))
            if not ok:
                bad.append(l)
    return bad


def kernel_bodies(asm_text):
    """{kernel symbol: its instruction lines} of the device assembly."""
    out = {}
    for part in re.split(r"\n(?=\S+:\s*; @)", asm_text):
        m = re.match(r"(\S+):\s*; @", part)
        if m:
            out[m.group(1)] = [l.strip() for l in part.split("\n")]
    return out


def spill_report(asm_text):
    """{kernel: (scratch accesses, scratch accesses inside a loop)}.  Scratch
    (private) memory is where the compiler spills registers; a loop is the
    range from a block label to the last branch back to it."""
    rep = {}
    for name, lines in kernel_bodies(asm_text).items():
        scratch = [i for i, l in enumerate(lines) if l.startswith("scratch_")]
        labels, loops = {}, []
        for i, l in enumerate(lines):
            m = re.match(r"(\.LBB\w+):", l)
            if m:
                labels[m.group(1)] = i
            b = re.match(r"s_(?:cbranch_\w+|branch)\s+(\.LBB\w+)", l)
            if b and b.group(1) in labels and labels[b.group(1)] < i:
                loops.append((labels[b.group(1)], i))
        inside = [i for i in scratch if any(lo <= i <= hi for lo, hi in loops)]
        rep[name] = (len(scratch), len(inside))
    return rep


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
    lib = build_lib()[0]
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

"""The device assembly of libtg.so's kernels, checked on the CPU (hipcc
compiles gfx950 code without a GPU).

* M0: the direct-copy kernels set M0 from inline assembly right before each
  global->LDS copy (gfx9: one wait state between the write and the copy).
  The compiler does not know the register is written there, so no other
  instruction of any kernel may read or write M0.
* Register spills: no kernel may touch scratch (private) memory inside a
  loop, where it would run once per K step; the kernels that spill outside
  their loops are listed here.
* C stores: every GEMM kernel's epilogue has its non-temporal 16-byte store
  (wave tiles wholly inside C, rows on 16-byte boundaries).
"""
import importlib.util
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build():
    spec = importlib.util.spec_from_file_location(
        "_tg_build_asm", os.path.join(ROOT, "tiled_dense_gemm_08_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    b = _build()
    path = b.device_asm(str(tmp_path_factory.mktemp("asm") / "tg_kernels.s"))
    with open(path) as f:
        return b, f.read()


def test_no_stray_m0_use(asm):
    b, text = asm
    assert b.check_m0(text) == []


def test_m0_check_catches_a_planted_use(asm):
    b, text = asm
    # a copy whose wait state is missing, and a compiler-style M0 read
    planted = text + "\n\ts_mov_b32 m0, s7\n\tbuffer_load_dwordx4 v1, s[0:3], 0 offen lds\n"
    assert b.check_m0(planted) == ["s_mov_b32 m0, s7"]
    assert b.check_m0(text + "\n\ts_add_u32 s2, m0, 4\n") == ["s_add_u32 s2, m0, 4"]


# Kernels that spill registers outside their loops: Cfg<BM, BN, BK, WM, WN,
# STAGES, MI, SCHED, TA, TB, ES> of configurations 1 and 2 (256x256x32 with 4
# and 5 stages), configurations 0 and 12 (their fp16 epilogues),
# configurations 22 and 26 (a few registers before their loops, in some of
# their orientations and epilogues), and the matrix-core ceiling loop (one
# register, before its loop).
KNOWN_SPILLS = [r"CfgILi256ELi256ELi32ELi2ELi2ELi[45]ELi32ELi1ELi0ELi0ELi2EE",
                r"CfgILi256ELi256ELi64ELi2ELi2ELi2ELi32ELi[01]ELi0ELi0ELi2EE",
                r"CfgILi256ELi256ELi64ELi2ELi4ELi2ELi16ELi2ELi[01]ELi[01]ELi2EE",
                r"CfgILi256ELi256ELi64ELi2ELi2ELi2ELi16ELi3ELi[01]ELi[01]ELi2EE",
                r"mfma_ceiling_kernel"]


def test_no_spill_inside_a_loop(asm):
    b, text = asm
    rep = b.spill_report(text)
    assert len(rep) > 100   # every instance was parsed
    inside = {k: v for k, v in rep.items() if v[1]}
    assert inside == {}
    spilling = sorted(k for k, v in rep.items() if v[0])
    unknown = [k for k in spilling if not any(re.search(p, k) for p in KNOWN_SPILLS)]
    assert unknown == [], unknown


def test_spill_report_sees_a_planted_loop_spill(asm):
    b, _ = asm
    text = ("k:   ; @k\n.LBB0_1:\n\tv_add_u32 v1, v2, v3\n"
            "\tscratch_store_dword off, v1, off\n\ts_cbranch_scc1 .LBB0_1\n\ts_endpgm\n")
    assert b.spill_report(text) == {"k": (1, 1)}


def test_every_gemm_kernel_streams_whole_c_chunks(asm):
    _, text = asm
    starts = [m for m in re.finditer(r"^(_ZN2tg\w*gemm_(?:pipe|staged|single)\w*):", text, re.M)]
    assert len(starts) > 100
    missing = []
    for i, m in enumerate(starts):
        end = starts[i + 1].start() if i + 1 < len(starts) else len(text)
        body = text[m.end():end]
        if not re.search(r"^\s*global_store_dwordx4 [^\n]*\bnt\b", body, re.M):
            missing.append(m.group(1))
    assert missing == [], missing[:3]

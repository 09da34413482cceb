"""libtg.so on the CPU: it loads, exports every function include/tg.h and
include/tg_diag.h declare, imports no HIP allocation call, and rejects bad
arguments before any HIP call (no GPU needed)."""
import os
import re

import pytest

import tiled_dense_gemm_08_amd as tg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# fake, well-aligned "device" addresses: validation never dereferences them
PA, PB, PC, PBIAS = 0x100000, 0x200000, 0x300000, 0x400000
F16, F32 = tg.TG_DTYPE_F16, tg.TG_DTYPE_F32


def header_functions():
    names = set()
    for h in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if not h.endswith(".h"):
            continue
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(tg_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_function():
    declared = header_functions()
    assert declared == sorted(tg.EXPORTED)
    for name in declared:
        assert hasattr(tg.lib, name)


def test_library_imports_no_allocation_call():
    """The library allocates no device (or pinned host) memory: its dynamic
    symbol table imports none of HIP's allocation or free calls, nor a
    stream or device synchronisation."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", tg.LIB_PATH], check=True,
                         stdout=subprocess.PIPE, text=True).stdout
    imported = set(re.findall(r"\bU (\w+)", out))
    hip = sorted(n for n in imported if n.startswith("hip"))
    assert "hipLaunchKernel" in hip   # the table is read correctly
    bad = [n for n in hip if re.search(r"Malloc|Free|Alloc|HostRegister|Synchronize|MemPool", n)]
    assert bad == [], bad


def test_status_strings_and_version():
    for s in range(7):
        assert tg.tg_status_string(s).startswith("TG_")
    assert "gfx950" in tg.tg_version()


def test_config_table_is_consistent():
    n = tg.tg_num_configs()
    assert n >= 4
    names = set()
    for i, c in enumerate(tg.configs()):
        assert c["id"] == i
        assert c["lds_bytes"] <= 160 * 1024
        assert c["mfma"] in (16, 32)
        assert c["block_m"] % (c["mfma"] * c["waves_m"]) == 0
        assert c["block_n"] % (c["mfma"] * c["waves_n"]) == 0
        assert c["name"] not in names
        names.add(c["name"])
    with pytest.raises(tg.TgError):
        tg.tg_config_info(n)


def gemm_rc(*, A=PA, B=PB, C=PC, M=64, N=64, K=64, lda=None, ldb=None, ldc=None, dt=F32):
    return tg.tg_gemm(A, B, C, M, N, K, K if lda is None else lda, N if ldb is None else ldb,
                      N if ldc is None else ldc, dt, 0)


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(N=-1), dict(K=-1),
    dict(lda=63), dict(ldb=63), dict(ldc=63),
    dict(A=0), dict(B=0), dict(C=0),
    dict(dt=0), dict(dt=4),
    dict(A=PA + 1), dict(B=PB + 1), dict(C=PC + 2),
])
def test_invalid_arguments_rejected_without_gpu(kw):
    assert gemm_rc(**kw) == tg.TG_ERROR_INVALID_VALUE


def test_f16_output_needs_only_2_byte_alignment_and_null_bias_rejected():
    assert gemm_rc(C=PC + 2, dt=F16, M=0) == tg.TG_SUCCESS
    rc = tg.tg_gemm_bias_relu(PA, PB, None, PC, 64, 64, 64, 64, 64, 64, F16, 0)
    assert rc == tg.TG_ERROR_INVALID_VALUE
    rc = tg.tg_gemm_bias_relu(PA, PB, PBIAS + 2, PC, 64, 64, 64, 64, 64, 64, F16, 0)
    assert rc == tg.TG_ERROR_INVALID_VALUE


def test_empty_problems_succeed_without_touching_a_device():
    assert gemm_rc(M=0) == tg.TG_SUCCESS
    assert gemm_rc(N=0, ldb=0, ldc=0) == tg.TG_SUCCESS
    assert gemm_rc(M=0, C=0) == tg.TG_SUCCESS


def test_huge_dimensions_are_unsupported():
    assert gemm_rc(M=2 ** 31, K=8, N=8) == tg.TG_ERROR_UNSUPPORTED


def test_unknown_config_id():
    assert tg.tg_gemm_with_config(10 ** 6, PA, PB, None, PC, 8, 8, 8, 8, 8, 8, F32, 0) == \
        tg.TG_ERROR_INVALID_VALUE
    assert tg.tg_gemm_with_config(-1, PA, PB, None, PC, 8, 8, 8, 8, 8, 8, F32, 0) == \
        tg.TG_ERROR_INVALID_VALUE


def test_direct_path_requirements():
    direct = [c["id"] for c in tg.configs() if c["direct_lds"]]
    staged = [c["id"] for c in tg.configs() if not c["direct_lds"]]
    assert direct and staged
    d, s = direct[0], staged[0]
    args = (PA, PB, None, PC, 1024, 1024, 1024, 1024, 1024, 1024, F32)
    assert tg.tg_config_supports(d, *args) == 1
    assert tg.tg_config_supports(s, *args) == 1
    # odd leading dimension / K / unaligned base: only the staged path
    assert tg.tg_config_supports(d, PA, PB, None, PC, 3001, 5003, 1031, 1031, 5003, 5003, F32) == 0
    assert tg.tg_config_supports(s, PA, PB, None, PC, 3001, 5003, 1031, 1031, 5003, 5003, F32) == 1
    assert tg.tg_config_supports(d, PA + 2, *args[1:]) == 0
    assert tg.tg_config_supports(d, PA, PB, None, PC, 64, 64, 64, 72, 64, 64, F32) == 1
    assert tg.tg_config_supports(d, PA, PB, None, PC, 64, 64, 60, 64, 64, 64, F32) == 0
    assert tg.tg_config_supports(d, *args[:4], -1, *args[5:]) == -1


def test_whole_k_configuration_needs_k_in_whole_steps():
    """The schedule-3 kernel (configuration 26, 64-deep K steps) has no test
    for chunks past K in its copies, so it serves only K that is a multiple
    of 64, in every orientation; other K goes to the other kernels."""
    cid = [c["id"] for c in tg.configs() if c["name"] == "pipe_256x256x64_s2_w2x2_mi16_c3"][0]
    for op_a in (0, 1):
        for op_b in (0, 1):
            for K, ok in ((1024, 1), (1088, 1), (1032, 0), (1000, 0), (64, 1), (8, 0)):
                lda = 1024 if op_a else K
                ldb = K if op_b else 1024
                assert tg.tg_config_supports(cid, PA, PB, None, PC, 1024, 1024, K, lda, ldb, 1024,
                                             F32, op_a=op_a, op_b=op_b) == ok, (op_a, op_b, K)
    # the dispatcher still serves such K, on another kernel
    assert tg.tg_select_config(PA, PB, None, PC, 8192, 8192, 8184, 8184, 8192, 8192,
                               tg.TG_DTYPE_F16) != cid
    assert tg.tg_select_config(PA, PB, None, PC, 8192, 8192, 8192, 8192, 8192, 8192,
                               tg.TG_DTYPE_F16) == cid


def test_int8_whole_k_configuration_and_its_table_entry():
    """The int8 schedule-3 kernel (configuration 27, 128-deep K steps) serves
    only K in whole steps; the exact-shape table names it for int8 8192^3 in
    the two orientations it is compiled for, and the other two fall back."""
    cid = [c["id"] for c in tg.configs() if c["name"] == "i8_pipe_256x256x128_s2_w2x2_mi16_c3"][0]
    info = tg.tg_config_info(cid)
    assert info["whole_k"] == 1 and info["elem_bytes"] == 1 and info["block_k"] == 128
    assert info["ops"] == 3
    I32 = tg.TG_DTYPE_I32
    for K, ok in ((1024, 1), (1152, 1), (1088, 0), (1000, 0)):
        assert tg.tg_config_supports(cid, PA, PB, None, PC, 512, 512, K, K, 512, 512, I32) == ok, K
    for op_a in (0, 1):
        for op_b in (0, 1):
            sel = tg.tg_select_config(PA, PB, None, PC, 8192, 8192, 8192, 8192, 8192, 8192, I32,
                                      op_a=op_a, op_b=op_b)
            assert (sel == cid) == (op_a == 0), (op_a, op_b, sel)


@pytest.mark.parametrize("M,N,K,lda,ldb,fused,direct", [
    (256, 256, 256, 256, 256, False, True),
    (1024, 1024, 1024, 1024, 1024, False, True),
    (8192, 8192, 8192, 8192, 8192, False, True),
    (4096, 11008, 4096, 4096, 11008, True, True),
    (3001, 5003, 1031, 1031, 5003, False, False),
])
def test_dispatch_picks_a_supporting_config(M, N, K, lda, ldb, fused, direct):
    bias = PBIAS if fused else None
    cid = tg.tg_select_config(PA, PB, bias, PC, M, N, K, lda, ldb, N, F16)
    assert 0 <= cid < tg.tg_num_configs()
    assert tg.tg_config_supports(cid, PA, PB, bias, PC, M, N, K, lda, ldb, N, F16) == 1
    assert bool(tg.tg_config_info(cid)["direct_lds"]) == direct


def test_gemm_ex_validation_without_gpu():
    T, Nop = tg.TG_OP_T, tg.TG_OP_N
    ex = lambda oa, ob, M, N, K, lda, ldb, ldc, A=PA: tg.tg_gemm_ex(
        oa, ob, A, PB, None, PC, M, N, K, lda, ldb, ldc, F32, 0)
    assert ex(2, Nop, 8, 8, 8, 8, 8, 8) == tg.TG_ERROR_INVALID_VALUE
    assert ex(Nop, -1, 8, 8, 8, 8, 8, 8) == tg.TG_ERROR_INVALID_VALUE
    # stored widths: A^T is K x M (lda >= M), B^T is N x K (ldb >= K)
    assert ex(T, Nop, 16, 8, 4, 8, 8, 8) == tg.TG_ERROR_INVALID_VALUE
    assert ex(Nop, T, 8, 16, 32, 32, 16, 16) == tg.TG_ERROR_INVALID_VALUE
    assert ex(T, T, 0, 16, 32, 1, 32, 16) == tg.TG_SUCCESS        # M = 0: no-op
    assert ex(T, Nop, 8, 8, 8, 8, 8, 8, A=PA + 1) == tg.TG_ERROR_INVALID_VALUE


def test_orientation_support_follows_the_config_table():
    args = (PA, PB, None, PC, 1024, 1024, 1024, 1024, 1024, 1024, F32)
    for c in tg.configs():
        for op_a in (0, 1):
            for op_b in (0, 1):
                want = 1 if c["ops"] & (1 << (2 * op_a + op_b)) and c["elem_bytes"] == 2 else 0
                assert tg.tg_config_supports(c["id"], *args, op_a=op_a, op_b=op_b) == want
    for op_a in (0, 1):
        for op_b in (0, 1):
            cid = tg.tg_select_config(*args, op_a=op_a, op_b=op_b)
            assert tg.tg_config_supports(cid, *args, op_a=op_a, op_b=op_b) == 1
    # direct path with A^T needs M % 8 == 0 (A's stored rows run along M)
    direct_all = [c["id"] for c in tg.configs()
                  if c["direct_lds"] and c["ops"] == 15 and c["elem_bytes"] == 2][0]
    assert tg.tg_config_supports(direct_all, PA, PB, None, PC, 1020, 1024, 1024, 1024, 1024,
                                 1024, F32, op_a=1) == 0
    assert tg.tg_config_supports(direct_all, PA, PB, None, PC, 1024, 1024, 1020, 1024, 1024,
                                 1024, F32, op_a=1) == 1


def test_int8_validation_without_gpu():
    I32 = tg.TG_DTYPE_I32
    ex = lambda bias, K, C=PC, A=PA: tg.tg_gemm_ex(tg.TG_OP_N, tg.TG_OP_N, A, PB, bias, C,
                                                    64, 64, K, K, 64, 64, I32, 0)
    assert ex(PBIAS, 64) == tg.TG_ERROR_INVALID_VALUE          # no bias with int32 C
    assert ex(None, 131072) == tg.TG_ERROR_UNSUPPORTED          # partial sums could leave int32
    assert ex(None, 64, C=PC + 2) == tg.TG_ERROR_INVALID_VALUE  # int32 C needs 4-byte alignment
    args = (PA + 1, PB + 3, None, PC, 1024, 1024, 1024, 1024, 1024, 1024, I32)
    cid = tg.tg_select_config(*args)
    info = tg.tg_config_info(cid)
    assert info["elem_bytes"] == 1 and not info["direct_lds"]  # odd bases: general path
    cid = tg.tg_select_config(PA, PB, None, PC, 8192, 8192, 8192, 8192, 8192, 8192, I32)
    assert tg.tg_config_info(cid)["elem_bytes"] == 1 and tg.tg_config_info(cid)["direct_lds"]
    # fp16 configurations never serve int8 and vice versa
    for c in tg.configs():
        sup = tg.tg_config_supports(c["id"], PA, PB, None, PC, 512, 512, 512, 512, 512, 512, I32)
        assert sup == (1 if c["elem_bytes"] == 1 else 0)


@pytest.mark.parametrize("args", [
    (8, PA, PC, 2, 1), (0, PA, PC, 2, 1),            # unknown MFMA shape
    (128, PA, PC, 2, 1),
    (64, 0, PC, 2, 1), (64, PA, PC, 3, 1),           # the int8 shape: same rules
    (32, 0, PC, 2, 1), (32, PA, 0, 2, 1),            # NULL buffers
    (32, PA, PC, 0, 1), (32, PA, PC, 3, 1),          # iters not even and >= 2
    (16, PA, PC, (1 << 30) + 2, 1),                  # too many iters
    (16, PA, PC, 2, 0), (16, PA, PC, 2, (1 << 20) + 1),   # workgroups out of range
    (32, PA, PC, 1 << 13, (1 << 19) + 1),            # more than 2^32 k-steps in all
])
def test_mfma_ceiling_rejects_bad_arguments(args):
    assert tg.tg_mfma_ceiling(*args) == tg.TG_ERROR_INVALID_VALUE

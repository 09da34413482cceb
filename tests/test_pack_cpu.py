"""The dispatcher's packed-operand plans (operands copied into zero-padded
copies in the caller's workspace before a direct configuration runs), on the
CPU.

tg_select_plan reports what tg_gemm_ws runs without touching a device, so the
rules -- when the dispatcher packs, which operands, which configuration, how
much workspace -- are checked here with stand-in addresses; the packed results
are checked on the GPU (test_gpu_pack.py).
"""
import pytest

import tiled_dense_gemm_08_amd as tg

PA, PB, PC, PW = 0x100000, 0x200000, 0x300000, 0x500000
F16, F32, I32 = tg.TG_DTYPE_F16, tg.TG_DTYPE_F32, tg.TG_DTYPE_I32
MAGIC = "tg-tuning 1"
BIG = 1 << 40


@pytest.fixture(autouse=True)
def empty_cache():
    tg.tg_tuning_clear()
    yield
    tg.tg_tuning_clear()


def lds(M, N, K, op_a, op_b, pad_a=0, pad_b=0):
    return (M if op_a else K) + pad_a, (K if op_b else N) + pad_b


def plan(M, N, K, op_a=0, op_b=0, dtype=F32, pad_a=0, pad_b=0, pa=PA, pb=PB, bias=None, ws=BIG):
    """(configuration, slices, packed mask, workspace used) of tg_gemm_ws(-1, 0, ...)."""
    lda, ldb = lds(M, N, K, op_a, op_b, pad_a, pad_b)
    st, cid, sp, packed, used = tg.tg_select_plan(pa, pb, bias, PC, M, N, K, lda, ldb, N, dtype,
                                                  ws, op_a=op_a, op_b=op_b)
    assert st == tg.TG_SUCCESS
    assert used <= ws
    return cid, sp, packed, used


def direct(cid):
    return tg.tg_config_info(cid)["direct_lds"] == 1


def copy_bytes(rows, cols, es):
    ce = 16 // es
    return rows * (-(-cols // ce) * ce) * es


def round256(n):
    return -(-n // 256) * 256


RAGGED_COPIES = round256(copy_bytes(3001, 1031, 2)) + round256(copy_bytes(1031, 5003, 2))


def test_ragged_workload_packs_both_operands_for_a_direct_kernel():
    # 3001 x 5003 x 1031 with packed (odd) leading dimensions
    cid, sp, packed, used = plan(3001, 5003, 1031)
    assert packed == 3 and direct(cid) and sp == 1
    assert used == RAGGED_COPIES
    # tg_gemm (no workspace) runs a register-staged kernel on it
    lda, ldb = lds(3001, 5003, 1031, 0, 0)
    assert not direct(tg.tg_select_config(PA, PB, None, PC, 3001, 5003, 1031, lda, ldb, 5003,
                                          F32))


def test_the_workspace_bounds_the_plan():
    # too small for the copies: the operands as passed
    cid, sp, packed, used = plan(3001, 5003, 1031, ws=RAGGED_COPIES - 16)
    assert packed == 0 and used == 0 and not direct(cid)
    cid, sp, packed, used = plan(3001, 5003, 1031, ws=0)
    assert (sp, packed, used) == (1, 0, 0)
    # exactly enough
    assert plan(3001, 5003, 1031, ws=RAGGED_COPIES)[2:] == (3, RAGGED_COPIES)


def test_packing_and_slicing_combine():
    # few tiles, long K, padded leading dimension of A: the copy of A, then K
    # slices of the direct kernel on it, partials after the copy
    cid, sp, packed, used = plan(256, 2048, 8192, pad_a=1, dtype=F16)
    assert packed == 1 and sp > 1 and direct(cid)
    assert used == round256(copy_bytes(256, 8192, 2)) + tg.tg_splitk_workspace_bytes(256, 2048, sp)
    # without room for the partials as well, one of the two
    cid, sp, packed, used = plan(256, 2048, 8192, pad_a=1, dtype=F16,
                                 ws=round256(copy_bytes(256, 8192, 2)))
    assert sp == 1 or packed == 0


def test_aligned_operands_are_never_packed():
    for (M, N, K) in [(8192, 8192, 8192), (3000, 5000, 1024), (64, 64, 64)]:
        for op_a in (0, 1):
            for op_b in (0, 1):
                cid, sp, packed, used = plan(M, N, K, op_a, op_b, dtype=F16)
                assert packed == 0, (M, N, K, op_a, op_b)
                assert used == tg.tg_splitk_workspace_bytes(M, N, sp)


def test_small_problems_stay_unpacked():
    for (M, N, K) in [(37, 45, 29), (129, 257, 131), (300, 520, 264)]:
        cid, sp, packed, _ = plan(M, N, K, pad_a=1, pad_b=1)
        assert packed == 0 and not direct(cid)


def test_only_the_operands_that_need_it_are_packed():
    # the auto plan: A padded by one element, B fine: only A
    cid, sp, packed, used = plan(4096, 4096, 2048, pad_a=1)
    assert packed == 1 and direct(cid) and used >= round256(copy_bytes(4096, 2048, 2))
    cid, sp, packed, used = plan(4096, 4096, 2048, pad_b=3)
    assert packed == 2 and used >= round256(copy_bytes(2048, 4096, 2))
    # an unaligned base alone makes the operand need a copy
    assert plan(4096, 4096, 2048, pb=PB + 2)[2] == 2
    # K not a whole chunk: both k-major operands (A.B^T) need their rows padded
    assert plan(4096, 4096, 2001, op_a=0, op_b=1)[2] == 3
    # ... but with A.B only A (B's rows past K read zeros from the copy range)
    assert plan(4096, 4096, 2001)[2] == 1


def test_tuning_cache_hit_is_never_packed(tmp_path):
    lda, ldb = lds(3001, 5003, 1031, 0, 0)
    staged = tg.tg_select_config(PA, PB, None, PC, 3001, 5003, 1031, lda, ldb, 5003, F32)
    f = tmp_path / "t.tgtune"
    f.write_text("%s\n3001 5003 1031 N N f32 0 %d %s 1.0\n"
                 % (MAGIC, staged, tg.tg_config_info(staged)["name"]))
    tg.load_tuning(str(f))
    assert plan(3001, 5003, 1031) == (staged, 1, 0, 0)


def test_named_configuration_plans_reject_what_they_cannot_run():
    lda, ldb = lds(3001, 5003, 1031, 0, 0)
    args = (PA, PB, None, PC, 3001, 5003, 1031, lda, ldb, 5003, F32)
    # a direct configuration on unaligned operands without room for the copies
    assert tg.tg_gemm_ws(6, 1, *args, PW, RAGGED_COPIES - 256) == tg.TG_ERROR_WORKSPACE
    assert tg.tg_gemm_ws(6, 1, *args, None, 0) == tg.TG_ERROR_UNSUPPORTED
    assert tg.tg_gemm_with_config(6, PA, PB, None, PC, 3001, 5003, 1031, lda, ldb, 5003,
                                  F32) == tg.TG_ERROR_UNSUPPORTED
    # a configuration not compiled for the orientation cannot be packed into it
    only_nn = [c["id"] for c in tg.configs() if c["direct_lds"] and c["ops"] == 1
               and c["elem_bytes"] == 2][0]
    st = tg.tg_gemm_ws(only_nn, 1, PA, PB, None, PC, 64, 64, 64, 64, 64, 64, F32, PW, BIG,
                       op_a=1)
    assert st == tg.TG_ERROR_UNSUPPORTED


def test_invalid_arguments_and_empty_problems():
    st, cid, sp, packed, used = tg.tg_select_plan(PA, PB, None, PC, 64, 64, 64, 63, 64, 64, F32)
    assert st == tg.TG_ERROR_INVALID_VALUE
    res = tg.tg_select_plan(PA, PB, None, PC, 0, 64, 64, 64, 64, 64, F32)
    assert res == (tg.TG_SUCCESS, -1, 1, 0, 0)
    import ctypes
    c = ctypes.c_int()
    assert tg.lib.tg_select_plan(0, 0, PA, PB, None, PC, 64, 64, 64, 64, 64, 64, F32, 0,
                                 ctypes.byref(c), ctypes.byref(c), None,
                                 None) == tg.TG_ERROR_INVALID_VALUE


def test_cached_plans_follow_tuning_cache_changes(tmp_path):
    """Plans are cached per host thread; loading or clearing the tuning cache
    must change what the next identical call runs."""
    lda, ldb = lds(2048, 2048, 2048, 0, 0)
    auto = plan(2048, 2048, 2048, dtype=F16)
    assert plan(2048, 2048, 2048, dtype=F16) == auto   # a cache hit gives the same plan
    other = [c for c in tg.configs() if c["direct_lds"] and c["elem_bytes"] == 2
             and c["id"] != auto[0]][0]
    f = tmp_path / "t.tgtune"
    f.write_text("%s\n2048 2048 2048 N N f16 0 %d %s 1.0\n" % (MAGIC, other["id"], other["name"]))
    tg.load_tuning(str(f))
    assert plan(2048, 2048, 2048, dtype=F16) == (other["id"], 1, 0, 0)
    tg.tg_tuning_clear()
    assert plan(2048, 2048, 2048, dtype=F16) == auto
    # the plan follows the operands' alignment, which is part of the key
    assert plan(2048, 2048, 2048, dtype=F16, pa=PA + 2)[2] == 1
    assert plan(2048, 2048, 2048, dtype=F16) == auto

"""The dispatcher's pack plan (operands copied into zero-padded scratch before a
direct configuration runs), on the CPU.

tg_select_plan reports the plan without touching a device, so the rules --
when the dispatcher packs, which operands, which configuration, how much
scratch -- are checked here with stand-in addresses; the packed results are
checked on the GPU (test_gpu_pack.py).
"""
import pytest

import tiled_dense_gemm_08_amd as tg

PA, PB, PC = 0x100000, 0x200000, 0x300000
F16, F32, I32 = tg.TG_DTYPE_F16, tg.TG_DTYPE_F32, tg.TG_DTYPE_I32
MAGIC = "tg-tuning 1"


@pytest.fixture(autouse=True)
def auto_policy():
    tg.tg_tuning_clear()
    prev = tg.tg_set_pack_policy(tg.TG_PACK_AUTO)
    yield
    tg.tg_set_pack_policy(prev)
    tg.tg_tuning_clear()


def lds(M, N, K, op_a, op_b, pad_a=0, pad_b=0):
    return (M if op_a else K) + pad_a, (K if op_b else N) + pad_b


def plan(M, N, K, op_a=0, op_b=0, dtype=F32, pad_a=0, pad_b=0, pa=PA, pb=PB, bias=None):
    lda, ldb = lds(M, N, K, op_a, op_b, pad_a, pad_b)
    st, cid, packed, scratch = tg.tg_select_plan(pa, pb, bias, PC, M, N, K, lda, ldb, N, dtype,
                                                 op_a=op_a, op_b=op_b)
    assert st == tg.TG_SUCCESS
    return cid, packed, scratch


def direct(cid):
    return tg.tg_config_info(cid)["direct_lds"] == 1


def copy_bytes(rows, cols, es):
    ce = 16 // es
    return rows * (-(-cols // ce) * ce) * es


def round256(n):
    return -(-n // 256) * 256


def test_ragged_workload_packs_both_operands_for_a_direct_kernel():
    # 3001 x 5003 x 1031 with packed (odd) leading dimensions
    cid, packed, scratch = plan(3001, 5003, 1031)
    assert packed == 3 and direct(cid)
    assert scratch == round256(copy_bytes(3001, 1031, 2)) + round256(copy_bytes(1031, 5003, 2))
    # the unpacked choice is a register-staged kernel
    lda, ldb = lds(3001, 5003, 1031, 0, 0)
    assert not direct(tg.tg_select_config(PA, PB, None, PC, 3001, 5003, 1031, lda, ldb, 5003,
                                          F32))


def test_aligned_operands_are_never_packed():
    for policy in (tg.TG_PACK_AUTO, tg.TG_PACK_ALWAYS):
        tg.tg_set_pack_policy(policy)
        for (M, N, K) in [(8192, 8192, 8192), (3000, 5000, 1024), (64, 64, 64)]:
            for op_a in (0, 1):
                for op_b in (0, 1):
                    cid, packed, scratch = plan(M, N, K, op_a, op_b, dtype=F16)
                    assert packed == 0 and scratch == 0, (M, N, K, op_a, op_b, policy)


def test_small_problems_stay_unpacked_in_auto():
    for (M, N, K) in [(37, 45, 29), (129, 257, 131), (300, 520, 264)]:
        cid, packed, _ = plan(M, N, K, pad_a=1, pad_b=1)
        assert packed == 0 and not direct(cid)


def test_only_the_operand_that_needs_it_is_packed():
    tg.tg_set_pack_policy(tg.TG_PACK_ALWAYS)
    # A padded by one element, B packed with N a multiple of 8: only A
    cid, packed, scratch = plan(2048, 2048, 2048, pad_a=1)
    assert packed == 1 and direct(cid) and scratch == round256(copy_bytes(2048, 2048, 2))
    cid, packed, scratch = plan(2048, 2048, 2048, pad_b=3)
    assert packed == 2 and scratch == round256(copy_bytes(2048, 2048, 2))
    # an unaligned base alone makes the operand need a copy
    cid, packed, _ = plan(2048, 2048, 2048, pb=PB + 2)
    assert packed == 2
    # K not a whole chunk: both k-major operands (A.B^T) need their rows padded
    cid, packed, _ = plan(1024, 1024, 1001, op_a=0, op_b=1)
    assert packed == 3
    # ... but with A.B only A (B's rows past K read zeros from the copy range)
    cid, packed, _ = plan(1024, 1024, 1001)
    assert packed == 1


def test_policy_never_and_always():
    tg.tg_set_pack_policy(tg.TG_PACK_NEVER)
    assert plan(3001, 5003, 1031)[1] == 0
    tg.tg_set_pack_policy(tg.TG_PACK_ALWAYS)
    for op_a in (0, 1):
        for op_b in (0, 1):
            for dtype in (F16, F32, I32):
                cid, packed, scratch = plan(300, 520, 264, op_a, op_b, dtype=dtype, pad_a=1,
                                            pad_b=1)
                assert packed == 3 and direct(cid) and scratch > 0, (op_a, op_b, dtype)
                assert tg.tg_config_info(cid)["elem_bytes"] == (1 if dtype == I32 else 2)
                assert tg.tg_config_info(cid)["ops"] & (1 << (2 * op_a + op_b))


def test_policy_setter_validates_and_returns_the_previous_policy():
    assert tg.tg_set_pack_policy(tg.TG_PACK_NEVER) == tg.TG_PACK_AUTO
    assert tg.tg_set_pack_policy(3) == -1
    assert tg.tg_set_pack_policy(-2) == -1
    assert tg.tg_set_pack_policy(tg.TG_PACK_ALWAYS) == tg.TG_PACK_NEVER


def test_tuning_cache_hit_is_never_packed(tmp_path):
    lda, ldb = lds(3001, 5003, 1031, 0, 0)
    staged = tg.tg_select_config(PA, PB, None, PC, 3001, 5003, 1031, lda, ldb, 5003, F32)
    f = tmp_path / "t.tgtune"
    f.write_text("%s\n3001 5003 1031 N N f32 0 %d %s 1.0\n"
                 % (MAGIC, staged, tg.tg_config_info(staged)["name"]))
    tg.load_tuning(str(f))
    assert plan(3001, 5003, 1031) == (staged, 0, 0)


def test_invalid_arguments_and_empty_problems():
    st, cid, packed, scratch = tg.tg_select_plan(PA, PB, None, PC, 64, 64, 64, 63, 64, 64, F32)
    assert st == tg.TG_ERROR_INVALID_VALUE
    st, cid, packed, scratch = tg.tg_select_plan(PA, PB, None, PC, 0, 64, 64, 64, 64, 64, F32)
    assert (st, cid, packed, scratch) == (tg.TG_SUCCESS, -1, 0, 0)
    import ctypes
    c = ctypes.c_int()
    assert tg.lib.tg_select_plan(0, 0, PA, PB, None, PC, 64, 64, 64, 64, 64, 64, F32, None,
                                 ctypes.byref(c), None) == tg.TG_ERROR_INVALID_VALUE


def test_no_scratch_is_held_without_a_gpu_call():
    assert tg.tg_scratch_held() == 0
    assert tg.tg_scratch_release() == tg.TG_SUCCESS
    assert tg.tg_scratch_held() == 0

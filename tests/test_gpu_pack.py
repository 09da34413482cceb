"""The packed-operand path on the GPU.

Operands the direct global->LDS copies cannot take (unaligned base, leading
dimension or row length not a multiple of 16 bytes) are copied by the
dispatcher into zero-padded library scratch, and a direct configuration runs
on the copies.  Checked against the CPU oracle (bit-exact on integer inputs)
and, on integer inputs, against the unpacked register-staged run of the same
call; plus the scratch's life cycle: growth, two streams, graph capture.
"""
import sys

import numpy as np
import pytest

import oracle
import parity
import tg_inputs as gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import tiled_dense_gemm_08_amd as tg  # noqa: E402

import test_gpu_int8 as gi  # noqa: E402
import test_gpu_parity as gp  # noqa: E402

F16, F32, I32 = tg.TG_DTYPE_F16, tg.TG_DTYPE_F32, tg.TG_DTYPE_I32
OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]


def log(msg):
    sys.stderr.write("[gpu] %s\n" % msg)
    sys.stderr.flush()


@pytest.fixture(autouse=True)
def pack_always():
    prev = tg.tg_set_pack_policy(tg.TG_PACK_ALWAYS)
    yield
    tg.tg_set_pack_policy(prev)


def plan(M, N, K, op_a, op_b, lda, ldb, ldc, dtype, offs=(0, 0, 0), bias=False, es=2):
    """The dispatcher's plan for stand-in addresses with the same alignment as
    the test's buffers (torch allocations are 256-byte aligned)."""
    cs = 2 if dtype == F16 else 4
    st, cid, packed, scratch = tg.tg_select_plan(
        (1 << 20) + es * offs[0], (2 << 20) + es * offs[1], (3 << 20) if bias else None,
        (4 << 20) + cs * offs[2], M, N, K, lda, ldb, ldc, dtype, op_a=op_a, op_b=op_b)
    assert st == tg.TG_SUCCESS
    return cid, packed


def staged_choice(M, N, K, op_a, op_b, lda, ldb, ldc, dtype, offs=(0, 0, 0), es=2):
    cs = 2 if dtype == F16 else 4
    return tg.tg_select_config((1 << 20) + es * offs[0], (2 << 20) + es * offs[1], None,
                               (4 << 20) + cs * offs[2], M, N, K, lda, ldb, ldc, dtype,
                               op_a=op_a, op_b=op_b)


# (M, N, K, extra lda, extra ldb, offsets of A, B, C in elements)
F16_CASES = [(300, 520, 264, 1, 3, (0, 0, 0)),      # padded leading dimensions
             (129, 257, 131, 3, 5, (1, 3, 1)),      # odd K, unaligned bases
             (77, 45, 29, 0, 0, (0, 0, 0)),         # packed rows, lengths not whole chunks
             (1, 9, 7, 0, 0, (0, 0, 0)),            # rows shorter than a chunk
             (640, 384, 1031, 1, 0, (2, 0, 0))]


@pytest.mark.parametrize("op_a,op_b", OPS)
def test_packed_fp16_matches_oracle_and_staged(op_a, op_b):
    n = 0
    for (M, N, K, pa, pb, offs) in F16_CASES:
        lda = (M if op_a else K) + pa
        ldb = (K if op_b else N) + pb
        for kind, c_dtype, fused in [("uniform", "f32", False), ("int", "f16", True),
                                     ("normal_scaled", "f16", False), ("int", "f32", False)]:
            dtype = F16 if c_dtype == "f16" else F32
            cid, packed = plan(M, N, K, op_a, op_b, lda, ldb, N, dtype, offs, bias=fused)
            assert packed != 0, (M, N, K, op_a, op_b)
            A, B = gen.operands(M, N, K, kind, 5000 + M + N + K)
            As, Bs = gp.stored(A, B, op_a, op_b)
            bias = gen.bias_vector(N, 11, integer=(kind == "int")) if fused else None
            what = "packed %s ops=%d%d %s packed=%d" % (tg.tg_config_info(cid)["name"], op_a,
                                                         op_b, kind, packed)
            out, _ = gp.run(As, Bs, M, N, K, c_dtype, bias=bias, lda=lda, ldb=ldb,
                            a_off=offs[0], b_off=offs[1], c_off=offs[2], op_a=op_a, op_b=op_b,
                            what=what)
            cref = oracle.gemm_ref(As, Bs, M, N, K, bias=bias, op_a=op_a, op_b=op_b)
            parity.check(out, cref, K, c_dtype, kind == "int", what=what)
            if kind == "int":
                # the same call, unpacked, on the register-staged configuration
                sid = staged_choice(M, N, K, op_a, op_b, lda, ldb, N, dtype, offs)
                ref, _ = gp.run(As, Bs, M, N, K, c_dtype, bias=bias, lda=lda, ldb=ldb,
                                a_off=offs[0], b_off=offs[1], c_off=offs[2], op_a=op_a,
                                op_b=op_b, config=sid, what="unpacked")
                assert np.array_equal(out.view(np.uint32) if c_dtype == "f32" else out,
                                      ref.view(np.uint32) if c_dtype == "f32" else ref), what
            n += 1
    assert n > 0


@pytest.mark.parametrize("op_a,op_b", OPS)
def test_packed_int8_is_exact(op_a, op_b):
    for (M, N, K, pa, pb, offs) in [(300, 520, 272, 1, 1, (0, 0, 0)),
                                    (129, 257, 65, 0, 0, (1, 3, 0)),
                                    (100, 70, 1031, 5, 0, (0, 0, 0))]:
        lda = (M if op_a else K) + pa
        ldb = (K if op_b else N) + pb
        cid, packed = plan(M, N, K, op_a, op_b, lda, ldb, N, I32, offs, es=1)
        assert packed != 0
        A, B = gen.operands_i8(M, N, K, 6000 + M + N + K)
        As, Bs = gi.stored(A, B, op_a, op_b)
        out = gi.run(As, Bs, M, N, K, op_a, op_b, lda=lda, ldb=ldb, offs=offs,
                     what="packed int8 packed=%d" % packed)
        gi.check(out, oracle.gemm_i8_ref(As, Bs, M, N, K, op_a=op_a, op_b=op_b),
                 "packed int8 ops=%d%d %dx%dx%d" % (op_a, op_b, M, N, K))


def test_ragged_workload_is_packed_by_default_and_exact_on_integers():
    tg.tg_set_pack_policy(tg.TG_PACK_AUTO)
    w = gen.workload("ragged3001x5003x1031", integer=True)
    M, N, K = w["M"], w["N"], w["K"]
    cid, packed = plan(M, N, K, 0, 0, K, N, N, F32)
    assert packed == 3 and tg.tg_config_info(cid)["direct_lds"] == 1
    out, _ = gp.run(w["A"], w["B"], M, N, K, "f32", what="ragged packed")
    sid = staged_choice(M, N, K, 0, 0, K, N, N, F32)
    ref, _ = gp.run(w["A"], w["B"], M, N, K, "f32", config=sid, what="ragged unpacked")
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    r = np.arange(0, M, 97)
    c = np.arange(0, N, 89)
    rr, cc = np.meshgrid(r, c, indexing="ij")
    cref = oracle.gemm_entries(w["A"], w["B"], rr.ravel(), cc.ravel(), K, K, N)
    parity.check(out[rr.ravel(), cc.ravel()], cref, K, "f32", True, what="ragged sampled")


# --------------------------------------------------------------- scratch --
class Problem:
    """Device operands of one unaligned problem (lda = K + 1) and its oracle."""

    def __init__(self, M, N, K, seed):
        self.M, self.N, self.K = M, N, K
        self.A, self.B = gen.operands(M, N, K, "int", seed)
        self.lda, self.ldb = K + 1, N
        self.ta, self.pa = gp.to_dev(self.A, M, K, self.lda)
        self.tb, self.pb = gp.to_dev(self.B, K, N, self.ldb)
        self.c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        self.cref = oracle.gemm_ref(self.A, self.B, M, N, K)

    def launch(self, stream):
        return tg.tg_gemm(self.pa, self.pb, self.c.data_ptr(), self.M, self.N, self.K,
                          self.lda, self.ldb, self.N, F32, stream.cuda_stream)

    def check(self, what):
        parity.check(self.c.cpu().numpy(), self.cref, self.K, "f32", True, what=what)


def test_scratch_grows_and_is_released():
    assert tg.tg_scratch_release() == tg.TG_SUCCESS
    assert tg.tg_scratch_held() == 0
    s = torch.cuda.current_stream()
    small, big = Problem(200, 300, 100, 1), Problem(900, 1000, 700, 2)
    for p, what in [(small, "small"), (big, "big"), (small, "small again")]:
        p.c.fill_(float("nan"))
        assert p.launch(s) == tg.TG_SUCCESS
        torch.cuda.synchronize()
        p.check(what)
        log("%s: scratch held %d" % (what, tg.tg_scratch_held()))
        assert tg.tg_scratch_held() > 0
    # the big problem's copy of A: 900 rows of K = 700 padded to 704
    assert tg.tg_scratch_held() >= 900 * 704 * 2
    assert tg.tg_scratch_release() == tg.TG_SUCCESS
    assert tg.tg_scratch_held() == 0
    small.c.fill_(float("nan"))
    assert small.launch(s) == tg.TG_SUCCESS
    torch.cuda.synchronize()
    small.check("after release")


def test_two_streams_use_their_own_scratch():
    tg.tg_scratch_release()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    p1, p2 = Problem(512, 768, 333, 3), Problem(700, 300, 555, 4)
    torch.cuda.synchronize()
    for _ in range(3):
        p1.c.fill_(float("nan"))
        p2.c.fill_(float("nan"))
        torch.cuda.synchronize()
        assert p1.launch(s1) == tg.TG_SUCCESS
        assert p2.launch(s2) == tg.TG_SUCCESS
        assert p1.launch(s1) == tg.TG_SUCCESS
        torch.cuda.synchronize()
        p1.check("stream 1")
        p2.check("stream 2")


def test_graph_capture_never_allocates_and_replays_correctly():
    tg.tg_scratch_release()
    side = torch.cuda.Stream()
    p = Problem(600, 520, 300, 5)
    torch.cuda.synchronize()
    # no scratch for this stream yet: the captured call runs unpacked
    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1, stream=side, capture_error_mode="relaxed"):
        assert p.launch(side) == tg.TG_SUCCESS
    assert tg.tg_scratch_held() == 0
    for i in range(3):
        p.c.fill_(float("nan"))
        torch.cuda.synchronize()
        g1.replay()
        torch.cuda.synchronize()
        p.check("unpacked replay %d" % i)
    # an eager call on the stream makes its scratch; a capture then packs
    with torch.cuda.stream(side):
        assert p.launch(side) == tg.TG_SUCCESS
    torch.cuda.synchronize()
    held = tg.tg_scratch_held()
    assert held > 0
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=side, capture_error_mode="relaxed"):
        assert p.launch(side) == tg.TG_SUCCESS
    assert tg.tg_scratch_held() == held
    # a larger eager call on the same stream replaces the buffer; the one the
    # graph refers to is kept
    big = Problem(1200, 1100, 900, 6)
    with torch.cuda.stream(side):
        assert big.launch(side) == tg.TG_SUCCESS
    torch.cuda.synchronize()
    big.check("big eager")
    assert tg.tg_scratch_held() > held
    for i in range(3):
        p.c.fill_(float("nan"))
        torch.cuda.synchronize()
        g2.replay()
        torch.cuda.synchronize()
        p.check("packed replay %d" % i)
    del g1, g2
    torch.cuda.synchronize()
    assert tg.tg_scratch_release() == tg.TG_SUCCESS

"""The packed-operand path and the allocation-free default calls on the GPU.

Operands the direct global->LDS copies cannot take (unaligned base, leading
dimension or row length not a multiple of 16 bytes) are copied by tg_gemm_ws
into zero-padded copies in the caller's workspace, and a direct configuration
runs on the copies.  Checked against the CPU oracle (bit-exact on integer
inputs) and, on integer inputs, against the unpacked register-staged run of
the same call.  The plain calls (tg_gemm, tg_gemm_ex) allocate nothing and
reject buffers that run past their allocation before launching anything.
"""
import sys

import numpy as np
import pytest

import hiputil
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


def staged_choice(M, N, K, op_a, op_b, lda, ldb, ldc, dtype, offs=(0, 0, 0), es=2):
    cs = 2 if dtype == F16 else 4
    return tg.tg_select_config((1 << 20) + es * offs[0], (2 << 20) + es * offs[1], None,
                               (4 << 20) + cs * offs[2], M, N, K, lda, ldb, ldc, dtype,
                               op_a=op_a, op_b=op_b)


def direct_configs(es, op_a, op_b):
    return [c["id"] for c in tg.configs() if c["direct_lds"] and c["elem_bytes"] == es
            and c["ops"] >> (2 * op_a + op_b) & 1]


# (M, N, K, extra lda, extra ldb, offsets of A, B, C in elements)
F16_CASES = [(300, 520, 264, 1, 3, (0, 0, 0)),      # padded leading dimensions
             (129, 257, 131, 3, 5, (1, 3, 1)),      # odd K, unaligned bases
             (77, 45, 29, 0, 0, (0, 0, 0)),         # packed rows, lengths not whole chunks
             (1, 9, 7, 0, 0, (0, 0, 0)),            # rows shorter than a chunk
             (640, 384, 1031, 1, 0, (2, 0, 0)),
             (264, 392, 320, 1, 3, (1, 0, 0))]      # K in whole 64-deep steps


@pytest.mark.parametrize("op_a,op_b", OPS)
def test_packed_fp16_matches_oracle_and_staged(op_a, op_b):
    """Every direct configuration compiled for the orientation, named in
    tg_gemm_ws, on operands it cannot take as passed: packed copies."""
    n = 0
    for cid in direct_configs(2, op_a, op_b):
        info = tg.tg_config_info(cid)
        name = info["name"]
        for (M, N, K, pa, pb, offs) in F16_CASES:
            if info["whole_k"] and K % info["block_k"]:
                continue        # runs only K in whole K steps
            lda = (M if op_a else K) + pa
            ldb = (K if op_b else N) + pb
            for kind, c_dtype, fused in [("uniform", "f32", False), ("int", "f16", True),
                                         ("int", "f32", False)]:
                dtype = F16 if c_dtype == "f16" else F32
                A, B = gen.operands(M, N, K, kind, 5000 + M + N + K)
                As, Bs = gp.stored(A, B, op_a, op_b)
                bias = gen.bias_vector(N, 11, integer=(kind == "int")) if fused else None
                what = "packed %s ops=%d%d %s" % (name, op_a, op_b, kind)
                out, _ = gp.run(As, Bs, M, N, K, c_dtype, bias=bias, lda=lda, ldb=ldb,
                                a_off=offs[0], b_off=offs[1], c_off=offs[2], op_a=op_a,
                                op_b=op_b, config=cid, ws=True, what=what)
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


def run_i8_ws(As, Bs, M, N, K, op_a, op_b, lda, ldb, offs, cid, what):
    """int8 operands through tg_gemm_ws with a named direct configuration."""
    log("%s M=%d N=%d K=%d ops=%d%d lda=%d ldb=%d config=%d offs=%s" % (
        what, M, N, K, op_a, op_b, lda, ldb, cid, offs))
    ta, pa = gi.to_dev(As, As.shape[0], As.shape[1], lda, offs[0])
    tb, pb = gi.to_dev(Bs, Bs.shape[0], Bs.shape[1], ldb, offs[1])
    tc = torch.full((M, N), 2 ** 31 - 1, dtype=torch.int32, device="cuda")
    nws = (As.size + Bs.size + 64 * (As.shape[0] + Bs.shape[0])) * 2 + 4096
    tw = torch.full((nws,), 0x55, dtype=torch.uint8, device="cuda")
    st = tg.tg_gemm_ws(cid, 1, pa, pb, None, tc.data_ptr(), M, N, K, lda, ldb, N, I32,
                       tw.data_ptr(), nws, torch.cuda.current_stream().cuda_stream,
                       op_a=op_a, op_b=op_b)
    assert st == tg.TG_SUCCESS, tg.tg_status_string(st)
    torch.cuda.synchronize()
    return tc.cpu().numpy()


@pytest.mark.parametrize("op_a,op_b", OPS)
def test_packed_int8_is_exact(op_a, op_b):
    for cid in direct_configs(1, op_a, op_b):
        info = tg.tg_config_info(cid)
        for (M, N, K, pa, pb, offs) in [(300, 520, 272, 1, 1, (0, 0)),
                                        (129, 257, 65, 0, 0, (1, 3)),
                                        (100, 70, 1031, 5, 0, (0, 0))]:
            if info["whole_k"] and K % info["block_k"]:
                continue
            lda = (M if op_a else K) + pa
            ldb = (K if op_b else N) + pb
            A, B = gen.operands_i8(M, N, K, 6000 + M + N + K)
            As, Bs = gi.stored(A, B, op_a, op_b)
            out = run_i8_ws(As, Bs, M, N, K, op_a, op_b, lda, ldb, offs, cid, "packed int8")
            gi.check(out, oracle.gemm_i8_ref(As, Bs, M, N, K, op_a=op_a, op_b=op_b),
                     "packed int8 config %d ops=%d%d %dx%dx%d" % (cid, op_a, op_b, M, N, K))


def test_ragged_workload_packed_with_a_workspace_staged_without():
    """The ragged workload: tg_gemm_ws packs both operands into the workspace
    and runs a direct kernel; tg_gemm runs a register-staged kernel on the
    operands as passed.  Bit-identical on integer inputs, every entry checked
    against the oracle."""
    w = gen.workload("ragged3001x5003x1031", integer=True)
    M, N, K = w["M"], w["N"], w["K"]
    P = 1 << 20
    st, cid, sp, packed, used = tg.tg_select_plan(P, 2 * P, None, 4 * P, M, N, K, K, N, N, F32)
    assert st == tg.TG_SUCCESS and packed == 3 and sp == 1
    assert tg.tg_config_info(cid)["direct_lds"] == 1
    out, _ = gp.run(w["A"], w["B"], M, N, K, "f32", ws=True, what="ragged packed")
    ref, _ = gp.run(w["A"], w["B"], M, N, K, "f32", what="ragged tg_gemm (staged)")
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    cref = oracle.gemm_ref(w["A"], w["B"], M, N, K)
    parity.check(out, cref, K, "f32", True, what="ragged packed, whole output")


class Problem:
    """Device operands of one unaligned problem (lda = K + 1), its workspace
    and its oracle."""

    def __init__(self, M, N, K, seed):
        self.M, self.N, self.K = M, N, K
        self.A, self.B = gen.operands(M, N, K, "int", seed)
        self.lda, self.ldb = K + 1, N
        self.ta, self.pa = gp.to_dev(self.A, M, K, self.lda)
        self.tb, self.pb = gp.to_dev(self.B, K, N, self.ldb)
        self.c = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        self.cref = oracle.gemm_ref(self.A, self.B, M, N, K)
        # a named direct configuration: always the packed copy of A (and of B
        # when N is not a multiple of 8)
        self.cid = [c for c in direct_configs(2, 0, 0)
                    if not tg.tg_config_info(c)["whole_k"] or K % tg.tg_config_info(c)["block_k"] == 0][0]
        self.ws = torch.empty(((M + K) * (max(K, N) + 8) * 2 + 4096) // 4, dtype=torch.float32,
                              device="cuda")

    def launch(self, stream):
        return tg.tg_gemm_ws(self.cid, 1, self.pa, self.pb, None, self.c.data_ptr(), self.M,
                             self.N, self.K, self.lda, self.ldb, self.N, F32, self.ws.data_ptr(),
                             self.ws.numel() * 4, stream.cuda_stream)

    def check(self, what):
        parity.check(self.c.cpu().numpy(), self.cref, self.K, "f32", True, what=what)


def test_two_streams_with_their_own_workspaces():
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


def test_graph_capture_of_a_packed_call_replays_correctly():
    """A captured tg_gemm_ws call (pack kernel + GEMM into the caller's
    workspace) replayed several times, with eager work between the replays
    that overwrites the same workspace and C."""
    side = torch.cuda.Stream()
    p = Problem(600, 520, 300, 5)
    other = Problem(600, 520, 300, 6)
    other.ws = p.ws   # the eager calls between replays share the workspace
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side, capture_error_mode="relaxed"):
        assert p.launch(side) == tg.TG_SUCCESS
    for i in range(3):
        p.c.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        p.check("packed replay %d" % i)
        other.c.fill_(float("nan"))
        assert other.launch(torch.cuda.current_stream()) == tg.TG_SUCCESS
        torch.cuda.synchronize()
        other.check("eager between replays %d" % i)
    del g
    torch.cuda.synchronize()


def test_plain_calls_allocate_no_device_memory():
    """tg_gemm and tg_gemm_ex on unaligned and aligned operands, the ragged
    workload included: the device's free memory is unchanged by the calls
    (measured after a first round that loads the kernels' code)."""
    w = gen.workload("ragged3001x5003x1031", integer=True)
    M, N, K = w["M"], w["N"], w["K"]
    ta, pa = gp.to_dev(w["A"], M, K, K)
    tb, pb = gp.to_dev(w["B"], K, N, N)
    tc = torch.empty((M, N), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream

    def calls():
        assert tg.tg_gemm(pa, pb, tc.data_ptr(), M, N, K, K, N, N, F32, s) == tg.TG_SUCCESS
        assert tg.tg_gemm(pa, pb, tc.data_ptr(), 1024, 1024, 1024, K, N, N, F16,
                          s) == tg.TG_SUCCESS
        assert tg.tg_gemm_ex(1, 0, pa, pb, None, tc.data_ptr(), 1000, 1000, 1000, K, N, N,
                             F32, s) == tg.TG_SUCCESS
        torch.cuda.synchronize()

    calls()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        calls()
    free1, _ = torch.cuda.mem_get_info()
    log("free device memory before %d after %d" % (free0, free1))
    assert free1 == free0


def test_buffers_past_their_allocation_are_rejected_before_launch():
    """A leading dimension, a C, a bias or a workspace that runs past the end
    of its allocation: TG_ERROR_INVALID_VALUE, and C is not written."""
    M = N = K = 256
    A, B = gen.operands(M, N, K, "int", 7)
    ta, pa = gp.to_dev(A, M, K, K)
    tb, pb = gp.to_dev(B, K, N, N)
    tc = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    bias = torch.zeros(N, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    # rows this far apart span 0.5 GB (below the 2 GiB limit of the kernels'
    # 32-bit offsets): far past the 2 MB pool blocks that hold these tensors
    huge = 1 << 20
    assert tg.tg_gemm(pa, pb, tc.data_ptr(), M, N, K, huge, N, N, F32, s) == \
        tg.TG_ERROR_INVALID_VALUE
    assert tg.tg_gemm(pa, pb, tc.data_ptr(), M, N, K, K, huge, N, F32, s) == \
        tg.TG_ERROR_INVALID_VALUE
    assert tg.tg_gemm(pa, pb, tc.data_ptr(), M, N, K, K, N, huge, F32, s) == \
        tg.TG_ERROR_INVALID_VALUE
    assert tg.tg_gemm_ex(1, 1, pa, pb, None, tc.data_ptr(), M, N, K, huge, huge, N, F32,
                         s) == tg.TG_ERROR_INVALID_VALUE
    # pointers 64 bytes before the end of their allocations
    for t in (tc, bias, ta):
        base, size = hiputil.alloc_range(t.data_ptr())
        end = base + size - 64
        if t is tc:
            rc = tg.tg_gemm(pa, pb, end, M, N, K, K, N, N, F32, s)
        elif t is bias:
            rc = tg.tg_gemm_bias_relu(pa, pb, end, tc.data_ptr(), M, N, K, K, N, N, F32, s)
        else:
            rc = tg.tg_gemm(end, pb, tc.data_ptr(), M, N, K, K, N, N, F32, s)
        assert rc == tg.TG_ERROR_INVALID_VALUE
    ws = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    base, size = hiputil.alloc_range(ws.data_ptr())
    need = tg.tg_splitk_workspace_bytes(M, N, 4)
    assert tg.tg_gemm_ws(-1, 4, pa, pb, None, tc.data_ptr(), M, N, K, K, N, N, F32,
                         base + size - need // 2, need, s) == tg.TG_ERROR_INVALID_VALUE
    torch.cuda.synchronize()
    assert bool((tc == 7.0).all())
    # the same calls with in-range arguments succeed
    assert tg.tg_gemm(pa, pb, tc.data_ptr(), M, N, K, K, N, N, F32, s) == tg.TG_SUCCESS
    torch.cuda.synchronize()
    parity.check(tc.cpu().numpy(), oracle.gemm_ref(A, B, M, N, K), K, "f32", True, "in range")

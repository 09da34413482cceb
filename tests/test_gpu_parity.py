"""Parity of the HIP path (through the C ABI) with the CPU oracle, on gfx950.

Every workload is compared on every output, the full-size ones (8192^3 and
the fused 4096 x 11008 x 4096) in the launch configuration the bench times
(the dispatcher's plan).  Integer inputs must match bit for bit.
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

import tiled_dense_gemm_08_amd as tg  # noqa: E402  (fails loudly if libtg.so is missing)

F16_NAN = 0x7E00


def log(msg):
    sys.stderr.write("[gpu] %s\n" % msg)
    sys.stderr.flush()


def to_dev(bits_2d, rows, cols, ld, offset_elems=0):
    """fp16 bits (rows x cols) -> device buffer with leading dimension ld and a
    leading offset; returns (tensor, pointer to element (0,0))."""
    n = offset_elems + ((rows - 1) * ld + cols if rows and cols else 0) + 8
    host = np.full(n, F16_NAN, np.uint16)       # NaN padding must never be read
    if rows and cols:
        view = np.lib.stride_tricks.as_strided(host[offset_elems:], shape=(rows, cols),
                                               strides=(ld * 2, 2))
        view[...] = bits_2d
    t = torch.from_numpy(host.view(np.int16)).cuda()
    return t, t.data_ptr() + 2 * offset_elems


def run(A, B, M, N, K, c_dtype, bias=None, lda=None, ldb=None, ldc=None, config=None,
        a_off=0, b_off=0, c_off=0, what="", op_a=0, op_b=0, ws=False):
    """A, B: the stored operands (M x K or, with op_a, K x M; K x N or, with
    op_b, N x K).  ws: run through tg_gemm_ws with a workspace of the size the
    dispatcher's fastest plan uses (with `config`: that configuration,
    unsliced, packing what it cannot take as passed)."""
    ar, ac = (K, M) if op_a else (M, K)
    br, bc = (N, K) if op_b else (K, N)
    lda = ac if lda is None else lda
    ldb = bc if ldb is None else ldb
    ldc = N if ldc is None else ldc
    log("%s M=%d N=%d K=%d ops=%d%d lda=%d ldb=%d ldc=%d %s bias=%s config=%s offs=%d,%d,%d" % (
        what, M, N, K, op_a, op_b, lda, ldb, ldc, c_dtype, bias is not None, config, a_off, b_off,
        c_off))
    ta, pa = to_dev(A, ar, ac, lda, a_off)
    tb, pb = to_dev(B, br, bc, ldb, b_off)
    esz = 2 if c_dtype == "f16" else 4
    nc = c_off + ((M - 1) * ldc + N if M and N else 0) + 8
    if c_dtype == "f16":
        tc = torch.full((nc,), float("nan"), dtype=torch.float16, device="cuda")
    else:
        tc = torch.full((nc,), float("nan"), dtype=torch.float32, device="cuda")
    pc = tc.data_ptr() + esz * c_off
    pbias = None
    if bias is not None:
        tbias = torch.from_numpy(np.ascontiguousarray(bias, np.float32)).cuda()
        pbias = tbias.data_ptr()
    code = tg.TG_DTYPE_F16 if c_dtype == "f16" else tg.TG_DTYPE_F32
    s = torch.cuda.current_stream().cuda_stream
    if ws:
        st, _, _, _, used = tg.tg_select_plan(pa, pb, pbias, pc, M, N, K, lda, ldb, ldc, code,
                                              op_a=op_a, op_b=op_b)
        assert st == tg.TG_SUCCESS
        if config is not None:   # a named configuration's copies: at most both operands
            used = 2 * (ar + br + 2) * (max(ac, bc) + 16) * 2 + 1024
        tw = torch.full((max(used, 16) // 4 + 4,), float("nan"), dtype=torch.float32,
                        device="cuda")
        st = tg.tg_gemm_ws(-1 if config is None else config, 0 if config is None else 1, pa, pb,
                           pbias, pc, M, N, K, lda, ldb, ldc, code, tw.data_ptr(), used, s,
                           op_a=op_a, op_b=op_b)
    elif config is not None:
        st = tg.tg_gemm_with_config(config, pa, pb, pbias, pc, M, N, K, lda, ldb, ldc, code, s,
                                    op_a=op_a, op_b=op_b)
    elif op_a or op_b:
        st = tg.tg_gemm_ex(op_a, op_b, pa, pb, pbias, pc, M, N, K, lda, ldb, ldc, code, s)
    elif bias is not None:
        st = tg.tg_gemm_bias_relu(pa, pb, pbias, pc, M, N, K, lda, ldb, ldc, code, s)
    else:
        st = tg.tg_gemm(pa, pb, pc, M, N, K, lda, ldb, ldc, code, s)
    assert st == tg.TG_SUCCESS, tg.tg_status_string(st)
    torch.cuda.synchronize()
    host = tc.cpu().numpy()
    if c_dtype == "f16":
        host = host.view(np.uint16)
    if not (M and N):
        return np.zeros((M, N), host.dtype), host
    out = np.lib.stride_tricks.as_strided(host[c_off:], shape=(M, N),
                                          strides=(ldc * host.itemsize, host.itemsize)).copy()
    return out, host


def full_check(A, B, M, N, K, c_dtype, integer, bias=None, **kw):
    out, _ = run(A, B, M, N, K, c_dtype, bias=bias, **kw)
    cref = oracle.gemm_ref(A, B, M, N, K, bias=bias, op_a=kw.get("op_a", 0),
                           op_b=kw.get("op_b", 0))
    return parity.check(out, cref, K, c_dtype, integer, what=kw.get("what", ""))


def supports(cid, M, N, K, lda, ldb, ldc, c_dtype, fused, op_a=0, op_b=0):
    # the direct path's alignment checks only look at the pointers' low bits;
    # torch allocations are 256-byte aligned
    code = tg.TG_DTYPE_F16 if c_dtype == "f16" else tg.TG_DTYPE_F32
    return tg.tg_config_supports(cid, 1 << 20, 2 << 20, (3 << 20) if fused else None, 4 << 20,
                                 M, N, K, lda, ldb, ldc, code, op_a=op_a, op_b=op_b) == 1


def stored(A, B, op_a, op_b):
    """Stored forms of logical operands A (M x K) and B (K x N)."""
    return (np.ascontiguousarray(A.T) if op_a else A, np.ascontiguousarray(B.T) if op_b else B)


# ------------------------------------------------------------ small shapes --
SMALL = [(16, 16, 32), (64, 64, 64), (1, 8, 8), (200, 136, 96), (300, 520, 264), (17, 40, 48),
         (256, 256, 256), (130, 260, 136)]
ODD = [(3, 5, 7), (37, 45, 29), (129, 257, 65), (100, 70, 1031)]


F16_CONFIGS = [c["id"] for c in tg.configs() if c["elem_bytes"] == 2]


@pytest.mark.parametrize("cid", F16_CONFIGS)
def test_small_shapes_every_config(cid):
    name = tg.tg_config_info(cid)["name"]
    n = 0
    for (M, N, K) in SMALL + ODD:
        for kind, c_dtype, fused in [("uniform", "f32", False), ("int", "f16", True),
                                     ("normal_scaled", "f16", False), ("int", "f32", False)]:
            if not supports(cid, M, N, K, K, N, N, c_dtype, fused):
                continue
            A, B = gen.operands(M, N, K, kind, 1000 + M + N + K)
            bias = gen.bias_vector(N, 7, integer=(kind == "int")) if fused else None
            full_check(A, B, M, N, K, c_dtype, kind == "int", bias=bias, config=cid,
                       what="%s %s" % (name, kind))
            n += 1
    assert n > 0


# --------------------------------------------------- the five workloads --
def sample_positions(M, N, bm, bn, count, seed):
    rng = np.random.default_rng(seed)
    rows, cols = [], []
    for m0 in range(0, M, bm):
        for n0 in range(0, N, bn):
            m1, n1 = min(M, m0 + bm) - 1, min(N, n0 + bn) - 1
            rows += [m0, m0, m1, m1]
            cols += [n0, n1, n0, n1]
    rows += list(rng.integers(0, M, count))
    cols += list(rng.integers(0, N, count))
    return np.array(rows, np.int64), np.array(cols, np.int64)


@pytest.mark.parametrize("name", ["sq256", "sq1024", "ragged3001x5003x1031"])
@pytest.mark.parametrize("integer", [False, True])
def test_workload_full(name, integer):
    w = gen.workload(name, integer=integer)
    rep = full_check(w["A"], w["B"], w["M"], w["N"], w["K"], w["c_dtype"], integer,
                     bias=w["bias"], what=name)
    log("%s integer=%s %s" % (name, integer, rep))


@pytest.mark.parametrize("name", ["sq8192", "fused4096x11008x4096"])
@pytest.mark.parametrize("integer", [False, True])
def test_workload_full_size_every_output(name, integer):
    """The full-size workloads in the launch configuration the bench times
    (the dispatcher's choice), every output against the oracle: bit-exact on
    integer inputs, within the tolerance otherwise."""
    w = gen.workload(name, integer=integer)
    M, N, K = w["M"], w["N"], w["K"]
    out, _ = run(w["A"], w["B"], M, N, K, w["c_dtype"], bias=w["bias"], ws=True, what=name)
    cref = oracle.gemm_ref(w["A"], w["B"], M, N, K, bias=w["bias"])
    rep = parity.check(out, cref, K, w["c_dtype"], integer, what=name)
    if w["bias"] is not None:
        assert np.all(parity.gpu_values(out, w["c_dtype"]) >= 0)
    log("%s integer=%s every output %s" % (name, integer, rep))


# ------------------------------------------------ cross-config equality --
def test_all_configs_bit_identical_on_integer_inputs():
    M, N, K = 300, 520, 264
    A, B = gen.operands(M, N, K, "int", 55)
    bias = gen.bias_vector(N, 56, integer=True)
    for c_dtype in ("f32", "f16"):
        outs = {}
        for cid in range(tg.tg_num_configs()):
            if supports(cid, M, N, K, K, N, N, c_dtype, True):
                outs[cid], _ = run(A, B, M, N, K, c_dtype, bias=bias, config=cid, what="xcfg")
        ids = sorted(outs)
        assert len(ids) >= 2
        for i in ids[1:]:
            assert np.array_equal(outs[i], outs[ids[0]]), (i, ids[0])


def test_repeated_runs_are_bitwise_identical():
    w = gen.workload("sq1024")
    a, _ = run(w["A"], w["B"], 1024, 1024, 1024, "f32", what="repeat1")
    b, _ = run(w["A"], w["B"], 1024, 1024, 1024, "f32", what="repeat2")
    assert np.array_equal(a, b)


# ---------------------------------------------- layouts and edge cases --
@pytest.mark.parametrize("M,N,K", [(37, 45, 29), (300, 520, 264), (129, 257, 1031)])
@pytest.mark.parametrize("offs", [(0, 0, 0), (1, 3, 1)])
def test_padded_leading_dims_and_unaligned_bases(M, N, K, offs):
    A, B = gen.operands(M, N, K, "uniform", 77)
    bias = gen.bias_vector(N, 78)
    for c_dtype in ("f32", "f16"):
        full_check(A, B, M, N, K, c_dtype, False, bias=bias, lda=K + 3, ldb=N + 5, ldc=N + 7,
                   a_off=offs[0], b_off=offs[1], c_off=offs[2], what="padded")
    Ai, Bi = gen.operands(M, N, K, "int", 79)
    full_check(Ai, Bi, M, N, K, "f16", True, lda=K + 8, ldb=N + 8, ldc=N + 4,
               a_off=offs[0], b_off=offs[1], c_off=offs[2], what="padded-int")


# The epilogue stores C with non-temporal 16-byte stores only where a wave
# tile lies wholly inside C and every row of C starts on a 16-byte boundary;
# elsewhere (misaligned base or leading dimension, edge tiles) chunk by chunk
# with ordinary stores.  Both paths must write the same C.
STORE_PATH_KERNELS = ["pipe_256x256x64_s2_w2x2_mi16_c3", "pipe_256x256x64_s2_w2x4_mi16_c2",
                      "pipe_64x64x64_s4_w2x2_mi16_c0", "pipe_64x64x64_s2_w2x2_mi16_c0"]


@pytest.mark.parametrize("name", STORE_PATH_KERNELS)
def test_streamed_and_plain_c_stores_agree(name):
    cid = [c["id"] for c in tg.configs() if c["name"] == name][0]
    M, N, K = 520, 776, 256   # whole tiles and wave tiles, and ragged edge tiles
    A, B = gen.operands(M, N, K, "int", 81)
    bias = gen.bias_vector(N, 82, integer=True)
    for c_dtype in ("f16", "f32"):
        ref, _ = run(A, B, M, N, K, c_dtype, bias=bias, config=cid, what="%s aligned C" % name)
        parity.check(ref, oracle.gemm_ref(A, B, M, N, K, bias=bias), K, c_dtype, True,
                     what="%s aligned C" % name)
        # misaligned base, misaligned rows, padded aligned rows
        for ldc, c_off in ((N, 1), (N + 1, 0), (N + 8, 0)):
            what = "%s ldc=%d c_off=%d %s" % (name, ldc, c_off, c_dtype)
            assert supports(cid, M, N, K, K, N, ldc, c_dtype, True), what
            out, _ = run(A, B, M, N, K, c_dtype, bias=bias, ldc=ldc, c_off=c_off, config=cid,
                         what=what)
            assert np.array_equal(out, ref), what


def test_K0_writes_zero_or_relu_bias():
    M, N = 70, 90
    A = np.zeros((M, 0), np.uint16)
    B = np.zeros((0, N), np.uint16)
    out, _ = run(A, B, M, N, 0, "f32", what="K0")
    assert np.all(out == 0)
    bias = gen.bias_vector(N, 5)
    out, _ = run(A, B, M, N, 0, "f16", bias=bias, what="K0-bias")
    want = oracle.output_typed(np.broadcast_to(np.maximum(bias.astype(np.float64), 0), (M, N)),
                               "f16")
    assert np.array_equal(np.where(out == 0x8000, 0, out), want)


def test_M0_leaves_C_untouched():
    A = np.zeros((0, 16), np.uint16)
    B = np.zeros((16, 16), np.uint16)
    _, host = run(A, B, 0, 16, 16, "f32", what="M0")
    assert np.all(np.isnan(host))


def test_host_pointer_is_rejected():
    a = np.zeros(64 * 64, np.float16)
    b = torch.zeros(64 * 64, dtype=torch.float16, device="cuda")
    c = torch.zeros(64 * 64, dtype=torch.float32, device="cuda")
    st = tg.tg_gemm(a.ctypes.data, b.data_ptr(), c.data_ptr(), 64, 64, 64, 64, 64, 64,
                    tg.TG_DTYPE_F32, 0)
    assert st == tg.TG_ERROR_NOT_DEVICE_MEMORY
    st = tg.tg_gemm(b.data_ptr(), b.data_ptr(), c.data_ptr(), 64, 64, 64, 64, 64, 64,
                    tg.TG_DTYPE_F32, 0)
    assert st == tg.TG_SUCCESS
    torch.cuda.synchronize()


def test_torch_marshalling_wrapper():
    w = gen.workload("sq256")
    a = torch.from_numpy(w["A"].view(np.float16)).cuda()
    b = torch.from_numpy(w["B"].view(np.float16)).cuda()
    c = tg.gemm(a, b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    cref = oracle.gemm_ref(w["A"], w["B"], 256, 256, 256)
    parity.check(c.cpu().numpy(), cref, 256, "f32", False, what="wrapper")


# ----------------------------------------------- transposed orientations --
OPS = [(0, 1), (1, 0), (1, 1)]


@pytest.mark.parametrize("cid", F16_CONFIGS)
def test_transposed_small_shapes_every_config(cid):
    info = tg.tg_config_info(cid)
    n = 0
    for op_a, op_b in OPS:
        if not info["ops"] & (1 << (2 * op_a + op_b)):
            continue
        for (M, N, K) in SMALL + ODD:
            for kind, c_dtype, fused in [("uniform", "f32", False), ("int", "f16", True)]:
                lda = M if op_a else K
                ldb = K if op_b else N
                if not supports(cid, M, N, K, lda, ldb, N, c_dtype, fused, op_a, op_b):
                    continue
                A, B = gen.operands(M, N, K, kind, 2000 + M + N + K)
                As, Bs = stored(A, B, op_a, op_b)
                bias = gen.bias_vector(N, 9, integer=(kind == "int")) if fused else None
                full_check(As, Bs, M, N, K, c_dtype, kind == "int", bias=bias, config=cid,
                           op_a=op_a, op_b=op_b, what="%s ops=%d%d" % (info["name"], op_a, op_b))
                n += 1
    if info["ops"] != 1:
        assert n > 0


@pytest.mark.parametrize("op_a,op_b", OPS)
def test_transposed_padded_and_unaligned(op_a, op_b):
    M, N, K = 129, 257, 131
    A, B = gen.operands(M, N, K, "uniform", 91)
    As, Bs = stored(A, B, op_a, op_b)
    bias = gen.bias_vector(N, 92)
    ac = M if op_a else K
    bc = K if op_b else N
    full_check(As, Bs, M, N, K, "f16", False, bias=bias, lda=ac + 3, ldb=bc + 5, ldc=N + 1,
               a_off=1, b_off=3, c_off=1, op_a=op_a, op_b=op_b, what="T-padded")
    Ai, Bi = gen.operands(M, N, K, "int", 93)
    Ais, Bis = stored(Ai, Bi, op_a, op_b)
    full_check(Ais, Bis, M, N, K, "f32", True, lda=ac + 8, ldb=bc + 8, op_a=op_a, op_b=op_b,
               what="T-padded-int")


@pytest.mark.parametrize("op_a,op_b", OPS)
@pytest.mark.parametrize("integer", [False, True])
def test_transposed_large_sampled(op_a, op_b, integer):
    # the backward products of the 4096 x 11008 x 4096 layer shape, through
    # the dispatcher: M = N = 4096, K = 11008 (dA = G.B^T-like, dB = A^T.G-like)
    M, N, K = 4096, 4096, 11008
    kind = "int" if integer else "normal_scaled"
    A, B = gen.operands(M, N, K, kind, 95 + 2 * op_a + op_b)
    As, Bs = stored(A, B, op_a, op_b)
    out, _ = run(As, Bs, M, N, K, "f16", op_a=op_a, op_b=op_b, what="T-large")
    cid = tg.tg_select_config(1 << 20, 2 << 20, None, 4 << 20, M, N, K,
                              M if op_a else K, K if op_b else N, N, tg.TG_DTYPE_F16,
                              op_a=op_a, op_b=op_b)
    info = tg.tg_config_info(cid)
    r, c = sample_positions(M, N, info["block_m"], info["block_n"], 3000, 21)
    cref = oracle.gemm_entries(As, Bs, r, c, K, M if op_a else K, K if op_b else N,
                               op_a=op_a, op_b=op_b)
    rep = parity.check(out[r, c], cref, K, "f16", integer, what="T-large")
    assert not np.any(np.isnan(parity.gpu_values(out, "f16")))
    log("T-large ops=%d%d integer=%s config=%s %s" % (op_a, op_b, integer, info["name"], rep))


def test_torch_wrapper_takes_transposed_views():
    M, N, K = 192, 320, 256
    A, B = gen.operands(M, N, K, "uniform", 97)
    a = torch.from_numpy(np.ascontiguousarray(A.T).view(np.float16)).cuda().t()   # (M, K) view
    b = torch.from_numpy(np.ascontiguousarray(B.T).view(np.float16)).cuda().t()   # (K, N) view
    assert a.stride(0) == 1 and b.stride(0) == 1
    c = tg.gemm(a, b, out_dtype=torch.float32)
    torch.cuda.synchronize()
    parity.check(c.cpu().numpy(), oracle.gemm_ref(A, B, M, N, K), K, "f32", False, what="T-view")

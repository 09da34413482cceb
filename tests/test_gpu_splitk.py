"""K-sliced (split-K) GEMM through the C ABI (tg_gemm_ws) on gfx950, against
the oracle.

Integer inputs make every partial sum exact in fp32 (int32 for int8), so the
sliced result must equal the oracle bit for bit whatever the slicing; the
slice boundaries are placed inside K steps and before ragged K tails, for
operands whose rows run along K (k-major) and along M or N (mn-major).
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

CODES = {"f16": tg.TG_DTYPE_F16, "f32": tg.TG_DTYPE_F32, "i32": tg.TG_DTYPE_I32}
F16_NAN = 0x7E00


def log(msg):
    sys.stderr.write("[gpu-splitk] %s\n" % msg)
    sys.stderr.flush()


def stored(M, N, K, op_a, op_b):
    return ((K, M) if op_a else (M, K)), ((N, K) if op_b else (K, N))


def host_operands(M, N, K, op_a, op_b, dtype, seed, kind="int"):
    (ar, ac), (br, bc) = stored(M, N, K, op_a, op_b)
    if dtype == "i32":
        return (gen.ints_i8(seed, ar * ac).reshape(ar, ac),
                gen.ints_i8(seed, br * bc, ar * ac).reshape(br, bc))
    vals = gen.ints_pm4 if kind == "int" else (lambda s, n, st=0: gen.normal(s, n, st) / np.sqrt(K))
    return (gen.to_f16_bits(vals(seed, ar * ac)).reshape(ar, ac),
            gen.to_f16_bits(vals(seed, br * bc, ar * ac)).reshape(br, bc))


def to_dev(a, ld, off_elems):
    """Stored operand -> device buffer with leading dimension ld, offset."""
    rows, cols = a.shape
    es = a.dtype.itemsize
    n = off_elems + ((rows - 1) * ld + cols if rows and cols else 0) + 16
    pad = F16_NAN if es == 2 else 0x55
    host = np.full(n, pad, a.dtype)
    if rows and cols:
        np.lib.stride_tricks.as_strided(host[off_elems:], shape=(rows, cols),
                                        strides=(ld * es, es))[...] = a
    t = torch.from_numpy(host.view(np.int16) if es == 2 else host).cuda()
    return t, t.data_ptr() + es * off_elems


def run(A, B, M, N, K, dtype, op_a=0, op_b=0, bias=None, config=-1, splits=0, lda=None,
        ldb=None, offs=(0, 0), ws_bytes=None, what=""):
    lda = A.shape[1] if lda is None else lda
    ldb = B.shape[1] if ldb is None else ldb
    log("%s M=%d N=%d K=%d %s ops=%d%d config=%d splits=%d ld=%d,%d offs=%s" % (
        what, M, N, K, dtype, op_a, op_b, config, splits, lda, ldb, offs))
    ta, pa = to_dev(A, lda, offs[0])
    tb, pb = to_dev(B, ldb, offs[1])
    cdt = {"f16": torch.float16, "f32": torch.float32, "i32": torch.int32}[dtype]
    tc = torch.full((M, N), 3, dtype=cdt, device="cuda")
    tbias = torch.from_numpy(bias).cuda() if bias is not None else None
    need = tg.tg_splitk_workspace_bytes(M, N, max(splits, 32))
    nbytes = need if ws_bytes is None else ws_bytes
    ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    st = tg.tg_gemm_ws(config, splits, pa, pb, tbias.data_ptr() if tbias is not None else None,
                       tc.data_ptr(), M, N, K, lda, ldb, N, CODES[dtype], ws.data_ptr(),
                       nbytes, torch.cuda.current_stream().cuda_stream, op_a=op_a, op_b=op_b)
    assert st == tg.TG_SUCCESS, tg.tg_status_string(st)
    torch.cuda.synchronize()
    out = tc.cpu().numpy()
    return out.view(np.uint16) if dtype == "f16" else out


def check_exact(out, A, B, M, N, K, dtype, op_a, op_b, bias, what):
    if dtype == "i32":
        want = oracle.gemm_i8_ref(A, B, M, N, K, op_a=op_a, op_b=op_b)
        bad = out.astype(np.int64) != want
        assert not bad.any(), "%s: %d mismatches, first %s" % (what, bad.sum(),
                                                             np.argwhere(bad)[0].tolist())
    else:
        cref = oracle.gemm_ref(A, B, M, N, K, bias=bias, op_a=op_a, op_b=op_b)
        parity.check(out, cref, K, dtype, True, what)


def configs(es, op_a, op_b):
    return [c for c in tg.configs()
            if c["elem_bytes"] == es and c["ops"] >> (2 * op_a + op_b) & 1]


@pytest.mark.parametrize("op_a,op_b", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_every_fp16_config_sliced(op_a, op_b):
    """K = 1000 in 3 slices: slice length a multiple of the K step, a ragged
    last slice; fp32 and fp16 C, with and without bias. A configuration that
    runs only K in whole K steps takes K = 1024 (slices of 6, 6 and 4
    steps) instead."""
    M, N = 200, 264
    bias = gen.bias_vector(N, 72, integer=True)
    for c in configs(2, op_a, op_b):
        K = 1024 if c["whole_k"] else 1000
        A, B = host_operands(M, N, K, op_a, op_b, "f16", 71)
        for dtype, b in (("f32", None), ("f16", bias)):
            what = "config %d %s bias=%s" % (c["id"], dtype, b is not None)
            out = run(A, B, M, N, K, dtype, op_a, op_b, bias=b, config=c["id"], splits=3,
                      what=what)
            check_exact(out, A, B, M, N, K, dtype, op_a, op_b, b, what)


@pytest.mark.parametrize("op_a,op_b", [(0, 0), (1, 0), (0, 1), (1, 1)])
def test_every_int8_config_sliced(op_a, op_b):
    """K = 1040 in 4 slices (K = 1024 for a configuration that runs only K in
    whole K steps)."""
    M, N = 208, 272
    for c in configs(1, op_a, op_b):
        K = 1024 if c["whole_k"] else 1040
        A, B = host_operands(M, N, K, op_a, op_b, "i32", 73)
        what = "int8 config %d" % c["id"]
        out = run(A, B, M, N, K, "i32", op_a, op_b, config=c["id"], splits=4, what=what)
        check_exact(out, A, B, M, N, K, "i32", op_a, op_b, None, what)


@pytest.mark.parametrize("splits", [2, 5, 7, 64])
def test_slice_counts_and_short_k(splits):
    """Uneven slice counts; more slices asked for than K steps exist."""
    M, N, K = 136, 200, 456
    A, B = host_operands(M, N, K, 1, 0, "f16", 74)
    out = run(A, B, M, N, K, "f32", 1, 0, splits=splits, what="splits=%d" % splits)
    check_exact(out, A, B, M, N, K, "f32", 1, 0, None, "splits=%d" % splits)


def test_unaligned_operands_use_the_register_staged_kernels_sliced():
    M, N, K = 150, 230, 777
    A, B = host_operands(M, N, K, 0, 0, "f16", 75)
    bias = gen.bias_vector(N, 76, integer=True)
    for c in configs(2, 0, 0):
        if c["direct_lds"]:
            continue
        out = run(A, B, M, N, K, "f16", bias=bias, config=c["id"], splits=4, lda=K + 3,
                  ldb=N + 1, offs=(1, 3), what="staged %d" % c["id"])
        check_exact(out, A, B, M, N, K, "f16", 0, 0, bias, "staged %d" % c["id"])


def test_auto_choice_slices_small_tile_count_long_k():
    """640 x 640 x 8192: the dispatcher slices K when given a workspace; the
    result is exact on integers and equal to the unsliced call's."""
    M, N, K = 640, 640, 8192
    P = 0x100000
    st, cid, sp, packed, used = tg.tg_select_plan(P, P, None, P, M, N, K, K, N, N,
                                                  tg.TG_DTYPE_F32, 1 << 30)
    assert st == tg.TG_SUCCESS and sp > 1 and packed == 0
    A, B = host_operands(M, N, K, 0, 0, "f16", 77)
    out = run(A, B, M, N, K, "f32", what="auto")
    check_exact(out, A, B, M, N, K, "f32", 0, 0, None, "auto")
    # no workspace: no slicing
    out1 = run(A, B, M, N, K, "f32", ws_bytes=0, what="auto, no workspace")
    assert np.array_equal(out1, out)


def test_sliced_result_is_reproducible_and_within_tolerance():
    M, N, K = 512, 384, 6144
    A, B = host_operands(M, N, K, 0, 1, "f16", 78, kind="normal")
    r1 = run(A, B, M, N, K, "f32", 0, 1, splits=6, what="normal 1")
    r2 = run(A, B, M, N, K, "f32", 0, 1, splits=6, what="normal 2")
    assert np.array_equal(r1, r2)
    cref = oracle.gemm_ref(A, B, M, N, K, op_a=0, op_b=1)
    parity.check(r1, cref, K, "f32", False, "sliced normal")


def test_workspace_errors():
    M, N, K = 256, 256, 4096
    A, B = host_operands(M, N, K, 0, 0, "f16", 79)
    ta, pa = to_dev(A, K, 0)
    tb, pb = to_dev(B, N, 0)
    tc = torch.empty((M, N), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    need = tg.tg_splitk_workspace_bytes(M, N, 4)
    ws = torch.empty(need // 4 + 4, dtype=torch.float32, device="cuda")
    host_ws = np.zeros(need // 4, np.float32)
    args = (pa, pb, None, tc.data_ptr(), M, N, K, K, N, N, tg.TG_DTYPE_F32)
    assert tg.tg_gemm_ws(-1, 4, *args, None, 0, s) == tg.TG_ERROR_WORKSPACE
    assert tg.tg_gemm_ws(-1, 4, *args, ws.data_ptr(), need - 4, s) == tg.TG_ERROR_WORKSPACE
    assert tg.tg_gemm_ws(-1, 4, *args, ws.data_ptr() + 4, need, s) == tg.TG_ERROR_INVALID_VALUE
    assert tg.tg_gemm_ws(-1, 4, *args, host_ws.ctypes.data, need,
                         s) == tg.TG_ERROR_NOT_DEVICE_MEMORY
    assert tg.tg_gemm_ws(-1, 4, *args, ws.data_ptr(), need, s) == tg.TG_SUCCESS
    torch.cuda.synchronize()


def test_large_sampled_normal_data():
    """1536 x 1536 x 8192 with N(0,1)/sqrt(K) data, in the dispatcher's
    sliced configuration, on sampled entries."""
    M, N, K = 1536, 1536, 8192
    A, B = host_operands(M, N, K, 0, 0, "f16", 80, kind="normal")
    out = run(A, B, M, N, K, "f16", what="1536 sampled")
    rng = np.random.default_rng(0)
    rows = rng.integers(0, M, 2000)
    cols = rng.integers(0, N, 2000)
    want = oracle.gemm_entries(A, B, rows, cols, K, K, N)
    got = out[rows, cols].view(np.float16).astype(np.float64)
    tol = parity.tolerance(want, K, "f16")
    assert np.all(np.abs(got - want) <= tol)

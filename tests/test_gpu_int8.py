"""int8 GEMM (int32 C) through the C ABI on gfx950 against the exact oracle.

Every comparison is bit-exact: int8 products summed in int32 are exact for the
K the library accepts, and the oracle sums exactly in int64.
"""
import sys

import numpy as np
import pytest

import oracle
import tg_inputs as gen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import tiled_dense_gemm_08_amd as tg  # noqa: E402

I32 = tg.TG_DTYPE_I32
PAD_I8 = 0x55            # padding byte that must never be read
UNWRITTEN = 0x7FFFFFFF   # no valid int32 result reaches it


def log(msg):
    sys.stderr.write("[gpu-i8] %s\n" % msg)
    sys.stderr.flush()


def to_dev(a, rows, cols, ld, off):
    n = off + ((rows - 1) * ld + cols if rows and cols else 0) + 16
    host = np.full(n, PAD_I8, np.int8)
    if rows and cols:
        view = np.lib.stride_tricks.as_strided(host[off:], shape=(rows, cols), strides=(ld, 1))
        view[...] = a
    t = torch.from_numpy(host).cuda()
    return t, t.data_ptr() + off


def run(As, Bs, M, N, K, op_a=0, op_b=0, lda=None, ldb=None, ldc=None, config=None,
        offs=(0, 0, 0), what=""):
    ar, ac = (K, M) if op_a else (M, K)
    br, bc = (N, K) if op_b else (K, N)
    lda = ac if lda is None else lda
    ldb = bc if ldb is None else ldb
    ldc = N if ldc is None else ldc
    log("%s M=%d N=%d K=%d ops=%d%d ld=%d,%d,%d config=%s offs=%s" % (
        what, M, N, K, op_a, op_b, lda, ldb, ldc, config, offs))
    ta, pa = to_dev(As, ar, ac, lda, offs[0])
    tb, pb = to_dev(Bs, br, bc, ldb, offs[1])
    nc = offs[2] + ((M - 1) * ldc + N if M and N else 0) + 4
    tc = torch.full((nc,), UNWRITTEN, dtype=torch.int32, device="cuda")
    pc = tc.data_ptr() + 4 * offs[2]
    s = torch.cuda.current_stream().cuda_stream
    if config is not None:
        st = tg.tg_gemm_with_config(config, pa, pb, None, pc, M, N, K, lda, ldb, ldc, I32, s,
                                    op_a=op_a, op_b=op_b)
    else:
        st = tg.tg_gemm_ex(op_a, op_b, pa, pb, None, pc, M, N, K, lda, ldb, ldc, I32, s)
    assert st == tg.TG_SUCCESS, tg.tg_status_string(st)
    torch.cuda.synchronize()
    host = tc.cpu().numpy()
    if not (M and N):
        return np.zeros((M, N), np.int32)
    return np.lib.stride_tricks.as_strided(host[offs[2]:], shape=(M, N),
                                           strides=(ldc * 4, 4)).copy()


def stored(A, B, op_a, op_b):
    return (np.ascontiguousarray(A.T) if op_a else A, np.ascontiguousarray(B.T) if op_b else B)


def check(out, want, what):
    bad = out.astype(np.int64) != want
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d mismatches, first at %s: gpu %d ref %d" % (
            what, int(bad.sum()), idx.tolist(), out[tuple(idx[0])], want[tuple(idx[0])]))


def supports(cid, M, N, K, lda, ldb, ldc, op_a, op_b):
    return tg.tg_config_supports(cid, 1 << 20, 2 << 20, None, 4 << 20, M, N, K, lda, ldb, ldc,
                                 I32, op_a=op_a, op_b=op_b) == 1


SHAPES = [(16, 16, 64), (64, 64, 128), (1, 16, 16), (200, 136, 192), (300, 520, 272),
          (17, 40, 48), (256, 256, 256), (130, 260, 144), (3, 5, 7), (37, 45, 29),
          (129, 257, 65), (100, 70, 1031)]
I8_CONFIGS = [c["id"] for c in tg.configs() if c["elem_bytes"] == 1]


@pytest.mark.parametrize("cid", I8_CONFIGS)
def test_int8_every_config_every_orientation(cid):
    info = tg.tg_config_info(cid)
    n = 0
    for op_a in (0, 1):
        for op_b in (0, 1):
            if not info["ops"] & (1 << (2 * op_a + op_b)):
                continue
            for (M, N, K) in SHAPES:
                lda, ldb = (M if op_a else K), (K if op_b else N)
                if not supports(cid, M, N, K, lda, ldb, N, op_a, op_b):
                    continue
                A, B = gen.operands_i8(M, N, K, 3000 + M + N + K)
                As, Bs = stored(A, B, op_a, op_b)
                out = run(As, Bs, M, N, K, op_a, op_b, config=cid, what=info["name"])
                check(out, oracle.gemm_i8_ref(As, Bs, M, N, K, op_a=op_a, op_b=op_b),
                      "%s ops=%d%d %dx%dx%d" % (info["name"], op_a, op_b, M, N, K))
                n += 1
    assert n > 0


@pytest.mark.parametrize("op_a,op_b", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_int8_padded_and_unaligned(op_a, op_b):
    M, N, K = 129, 257, 131
    A, B = gen.operands_i8(M, N, K, 3100)
    As, Bs = stored(A, B, op_a, op_b)
    ac, bc = (M if op_a else K), (K if op_b else N)
    for lda, ldb, offs in [(ac + 3, bc + 5, (1, 3, 1)), (ac + 16, bc + 16, (0, 0, 0))]:
        out = run(As, Bs, M, N, K, op_a, op_b, lda=lda, ldb=ldb, ldc=N + 3, offs=offs,
                  what="i8-padded")
        check(out, oracle.gemm_i8_ref(As, Bs, M, N, K, op_a=op_a, op_b=op_b), "i8-padded")


@pytest.mark.parametrize("name", ["sq8192_i8", "sq8192_i8_nt"])
def test_int8_large_every_output(name):
    """8192^3 int8 through the dispatcher: every int32 output equal to the
    exact oracle."""
    w = gen.workload(name)
    M, N, K = w["M"], w["N"], w["K"]
    out = run(w["A"], w["B"], M, N, K, w["op_a"], w["op_b"], what=name)
    want = oracle.gemm_i8_ref(w["A"], w["B"], M, N, K, lda=w["lda"], ldb=w["ldb"],
                              op_a=w["op_a"], op_b=w["op_b"])
    check(out, want, name)


def test_int8_K0_writes_zero():
    A = np.zeros((70, 0), np.int8)
    B = np.zeros((0, 90), np.int8)
    out = run(A, B, 70, 90, 0, what="i8-K0")
    assert np.all(out == 0)

"""Every configuration on the odd-shape grid M, N, K in {1, 2, 15, 16, 17,
31, 32, 33, 63, 64, 65, 127, 129, 255, 257} (a sample in which every value
occurs twice in every dimension), on integer inputs, bit-exact against the
oracle -- and the same again with the LDS-poison debug build
(libtg_poison.so: LDS filled with NaN before every write of it), which must
give the same bits as the normal library: a read of LDS bytes that the
current K step did not write would show up as NaN or as a different value.

Each configuration is named in tg_gemm_ws, so a direct-copy configuration
runs on packed copies of the operands it cannot take as passed (odd K or N)
and the register-staged and single-stage ones on the operands as passed. The
configurations that serve only K in whole K steps (copy schedule 3) run the
same M and N with K rounded up to a whole number of steps.
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

GRID = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 129, 255, 257]
SHAPES = ([(GRID[i], GRID[(i + 4) % 15], GRID[(i + 9) % 15]) for i in range(15)] +
          [(GRID[i], GRID[(i + 11) % 15], GRID[(i + 2) % 15]) for i in range(15)])
OPS = [(0, 0), (0, 1), (1, 0), (1, 1)]
CONFIGS = tg.configs()
CODES = {"f16": tg.TG_DTYPE_F16, "f32": tg.TG_DTYPE_F32, "i32": tg.TG_DTYPE_I32}


def log(msg):
    sys.stderr.write("[gpu-grid] %s\n" % msg)
    sys.stderr.flush()


def test_grid_sample_covers_every_value_in_every_dimension():
    for d in range(3):
        assert sorted({s[d] for s in SHAPES}) == GRID


def to_dev(a, pad):
    flat = np.ascontiguousarray(a).reshape(-1)
    host = np.concatenate([flat, np.full(16, pad, flat.dtype)])
    t = torch.from_numpy(host.view(np.int16) if host.dtype == np.uint16 else host).cuda()
    return t


def run(L, info, A, B, M, N, K, op_a, op_b, c_dtype, bias):
    """Configuration `info` of library build L on stored operands A, B through
    tg_gemm_ws (one slice); returns C's bits."""
    es = info["elem_bytes"]
    ta = to_dev(A, 0x7E00 if es == 2 else 0x55)
    tb = to_dev(B, 0x7E00 if es == 2 else 0x55)
    cdt = {"f16": torch.float16, "f32": torch.float32, "i32": torch.int32}[c_dtype]
    tc = torch.full((M, N), 3, dtype=cdt, device="cuda")
    if c_dtype != "i32":
        tc.fill_(float("nan"))
    tbias = torch.from_numpy(bias).cuda() if bias is not None else None
    nws = 4 * (A.size + B.size) + 64 * (sum(A.shape) + sum(B.shape)) + 4096
    ws = torch.full((nws // 4,), float("nan"), dtype=torch.float32, device="cuda")
    st = L.tg_gemm_ws(info["id"], 1, op_a, op_b, ta.data_ptr(), tb.data_ptr(),
                      tbias.data_ptr() if tbias is not None else None, tc.data_ptr(), M, N, K,
                      A.shape[1], B.shape[1], N, CODES[c_dtype], ws.data_ptr(), nws,
                      torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_SUCCESS, "%s: %s" % (info["name"], tg.tg_status_string(st))
    torch.cuda.synchronize()
    out = tc.cpu().numpy()
    return out.view(np.uint16) if c_dtype == "f16" else out


def cases(info, shapes):
    """(M, N, K, op_a, op_b, c_dtype, fused) of the configuration's runs:
    orientations rotate over the shapes (as stored when the configuration is
    not compiled for the rotated one); K rounded up to whole K steps for the
    configurations that need them (M and N stay odd)."""
    out = []
    for j, (M, N, K) in enumerate(shapes):
        if info["whole_k"]:
            K = -(-K // info["block_k"]) * info["block_k"]
        op_a, op_b = OPS[j % 4]
        if not info["ops"] >> (2 * op_a + op_b) & 1:
            op_a, op_b = 0, 0
        if info["elem_bytes"] == 1:
            out.append((M, N, K, op_a, op_b, "i32", False))
        else:
            out += [(M, N, K, op_a, op_b, "f32", False), (M, N, K, op_a, op_b, "f16", True)]
    return out


def operands(M, N, K, op_a, op_b, es, seed):
    if es == 1:
        A, B = gen.operands_i8(M, N, K, seed)
    else:
        A, B = gen.operands(M, N, K, "int", seed)
    return (np.ascontiguousarray(A.T) if op_a else A, np.ascontiguousarray(B.T) if op_b else B)


def reference(A, B, M, N, K, op_a, op_b, c_dtype, bias):
    if c_dtype == "i32":
        return oracle.gemm_i8_ref(A, B, M, N, K, op_a=op_a, op_b=op_b).astype(np.int32)
    cref = oracle.gemm_ref(A, B, M, N, K, bias=bias, op_a=op_a, op_b=op_b)
    out = oracle.output_typed(cref, c_dtype)
    return out.view(np.uint32) if c_dtype == "f32" else out


def same(got, want, c_dtype):
    """Bit equality, with +0 and -0 equal."""
    if c_dtype == "f16":
        g, w = np.where(got == 0x8000, 0, got), np.where(want == 0x8000, 0, want)
    elif c_dtype == "f32":
        g, w = got.view(np.uint32), want
        g, w = np.where(g == 0x80000000, 0, g), np.where(w == 0x80000000, 0, w)
    else:
        g, w = got, want
    return np.array_equal(g, w)


@pytest.mark.parametrize("cid", [c["id"] for c in CONFIGS])
def test_odd_shape_grid_every_config(cid):
    info = tg.tg_config_info(cid)
    for (M, N, K, op_a, op_b, c_dtype, fused) in cases(info, SHAPES):
        A, B = operands(M, N, K, op_a, op_b, info["elem_bytes"], 7 * M + 5 * N + 3 * K)
        bias = gen.bias_vector(N, 9, integer=True) if fused else None
        got = run(tg.lib, info, A, B, M, N, K, op_a, op_b, c_dtype, bias)
        want = reference(A, B, M, N, K, op_a, op_b, c_dtype, bias)
        assert same(got, want, c_dtype), "%s %dx%dx%d ops=%d%d %s" % (
            info["name"], M, N, K, op_a, op_b, c_dtype)
    log("%s: %d grid runs exact" % (info["name"], len(cases(info, SHAPES))))


@pytest.fixture(scope="module")
def poison():
    return tg.load_library(tg.POISON_LIB_PATH)


# the poison build on a third of the grid, plus shapes of several K steps
POISON_SHAPES = SHAPES[::3] + [(300, 520, 264), (129, 257, 1031), (640, 384, 520)]


@pytest.mark.parametrize("cid", [c["id"] for c in CONFIGS])
def test_lds_poison_build_gives_the_same_bits(poison, cid):
    info = tg.tg_config_info(cid)
    for (M, N, K, op_a, op_b, c_dtype, fused) in cases(info, POISON_SHAPES):
        A, B = operands(M, N, K, op_a, op_b, info["elem_bytes"], 11 * M + 3 * N + K)
        bias = gen.bias_vector(N, 10, integer=True) if fused else None
        got = run(poison, info, A, B, M, N, K, op_a, op_b, c_dtype, bias)
        ref = run(tg.lib, info, A, B, M, N, K, op_a, op_b, c_dtype, bias)
        what = "%s %dx%dx%d ops=%d%d %s" % (info["name"], M, N, K, op_a, op_b, c_dtype)
        assert np.array_equal(got, ref), "poison build differs: " + what
        assert same(got, reference(A, B, M, N, K, op_a, op_b, c_dtype, bias), c_dtype), what

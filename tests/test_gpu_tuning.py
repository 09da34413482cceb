"""The offline-tune / online-read path on gfx950: the sweep times kernels on
the device, writes a tuning cache, the library loads it, and the dispatcher
then launches the recorded kernel, whose output must match the oracle bit for
bit (integer inputs)."""
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
from tiled_dense_gemm_08_amd import sweep  # noqa: E402

CODES = {"f16": tg.TG_DTYPE_F16, "f32": tg.TG_DTYPE_F32, "i32": tg.TG_DTYPE_I32}


def log(msg):
    sys.stderr.write("[gpu-tune] %s\n" % msg)
    sys.stderr.flush()


@pytest.fixture(autouse=True)
def empty_cache():
    tg.tg_tuning_clear()
    yield
    tg.tg_tuning_clear()


def operands(sh, seed):
    """Stored operands (host) of a shape with integer values."""
    ar, ac = (sh.K, sh.M) if sh.op_a else (sh.M, sh.K)
    br, bc = (sh.N, sh.K) if sh.op_b else (sh.K, sh.N)
    if sh.c_dtype == "i32":
        A = gen.ints_i8(seed, ar * ac).reshape(ar, ac)
        B = gen.ints_i8(seed, br * bc, ar * ac).reshape(br, bc)
    else:
        A = gen.to_f16_bits(gen.ints_pm4(seed, ar * ac)).reshape(ar, ac)
        B = gen.to_f16_bits(gen.ints_pm4(seed, br * bc, ar * ac)).reshape(br, bc)
    return A, B


def run_dispatch(sh, A, B, bias):
    """One call through tg_gemm_ex (the dispatcher), packed operands."""
    ta = torch.from_numpy(A.view(np.int16) if A.dtype == np.uint16 else A).cuda()
    tb = torch.from_numpy(B.view(np.int16) if B.dtype == np.uint16 else B).cuda()
    cdt = {"f16": torch.float16, "f32": torch.float32, "i32": torch.int32}[sh.c_dtype]
    tc = torch.full((sh.M, sh.N), 7, dtype=cdt, device="cuda")
    tbias = torch.from_numpy(bias).cuda() if bias is not None else None
    st = tg.tg_gemm_ex(sh.op_a, sh.op_b, ta.data_ptr(), tb.data_ptr(),
                       tbias.data_ptr() if tbias is not None else None, tc.data_ptr(),
                       sh.M, sh.N, sh.K, A.shape[1], B.shape[1], sh.N, CODES[sh.c_dtype],
                       torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_SUCCESS, tg.tg_status_string(st)
    torch.cuda.synchronize()
    out = tc.cpu().numpy()
    return out.view(np.uint16) if sh.c_dtype == "f16" else out


def check_exact(sh, A, B, bias, out, what):
    if sh.c_dtype == "i32":
        want = oracle.gemm_i8_ref(A, B, sh.M, sh.N, sh.K, op_a=sh.op_a, op_b=sh.op_b)
        assert np.array_equal(out.astype(np.int64), want), what
    else:
        cref = oracle.gemm_ref(A, B, sh.M, sh.N, sh.K, bias=bias, op_a=sh.op_a, op_b=sh.op_b)
        parity.check(out, cref, sh.K, sh.c_dtype, True, what)


def select(sh, A, B, bias):
    P = 0x100000
    return tg.tg_select_config(P, P, P if bias is not None else None, P, sh.M, sh.N, sh.K,
                               A.shape[1], B.shape[1], sh.N, CODES[sh.c_dtype],
                               op_a=sh.op_a, op_b=sh.op_b)


def test_sweep_tune_writes_a_cache_the_dispatcher_follows(tmp_path):
    shapes = [sweep.Shape.parse(s) for s in
              ("640x384x1040:f16", "512x1024x256:f32:bias:nt", "384x640x512:i32:tn")]
    ids = list(range(tg.tg_num_configs()))
    recs = {}
    for sh in shapes:
        log("tune %s" % sh)
        res = sweep.search(sh, ids, reps=3, timing="graph", staged=True)
        w = sweep.winner(res)
        assert w is not None and w["tflops"] > 0
        recs[sh.key()] = (w["config"], w["name"], w["tflops"])
    path = str(tmp_path / "t.tgtune")
    sweep.write_cache(path, recs)
    assert tg.load_tuning(path) == (len(shapes), 0)
    for i, sh in enumerate(shapes):
        A, B = operands(sh, 40 + i)
        bias = (gen.bias_vector(sh.N, 50 + i, integer=True) if sh.fused else None)
        assert select(sh, A, B, bias) == recs[sh.key()][0]
        log("dispatch %s -> config %d" % (sh, recs[sh.key()][0]))
        check_exact(sh, A, B, bias, run_dispatch(sh, A, B, bias), str(sh))


@pytest.mark.parametrize("spec", ["320x448x272:f16", "320x448x272:f32:tt", "320x448x272:i32:nt"])
def test_every_cached_config_is_launched_correctly(tmp_path, spec):
    """A cache record naming any kernel that can run the problem makes the
    dispatcher launch that kernel, with exact results."""
    sh = sweep.Shape.parse(spec)
    A, B = operands(sh, 61)
    want_es = 1 if sh.c_dtype == "i32" else 2
    n = 0
    for c in tg.configs():
        if c["elem_bytes"] != want_es or not c["ops"] >> (2 * sh.op_a + sh.op_b) & 1:
            continue
        if c["whole_k"] and sh.K % c["block_k"]:
            continue
        path = str(tmp_path / ("c%d.tgtune" % c["id"]))
        sweep.write_cache(path, {sh.key(): (c["id"], c["name"], 1.0)})
        assert tg.load_tuning(path) == (1, 0)
        assert select(sh, A, B, None) == c["id"]
        log("%s via cached config %d (%s)" % (spec, c["id"], c["name"]))
        check_exact(sh, A, B, None, run_dispatch(sh, A, B, None), "%s config %d" % (spec, c["id"]))
        n += 1
    assert n >= 2

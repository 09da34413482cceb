"""Fused attention forward through the C ABI on gfx950 against the fp64
oracle (oracle/tgref_attention.c).

Tolerance, from the kernel's arithmetic: the scores and the softmax are fp32
(relative error ~1e-6), the weights are rounded to fp16 before the second
product (each off by at most 2^-11 of itself, or 2^-25 absolute below the
fp16 normal range; they are taken relative to a reference maximum at most
2^8 below the row's, so the largest is in [1, 256] and the sum is at least
1), and O is rounded to fp16 once.  Per element:
    |O - O_ref| <= 2^-10 A + n 2^-24 max|V| + ulp16(O_ref)
with A the softmax-weighted mean |V| the oracle returns and n the number of
visible keys (twice the weight-rounding bound, for the fp32 terms).  The
log-sum-exp is fp32: |lse - lse_ref| <= 2e-5 (1 + |lse_ref|).
"""
import math
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

F16_NAN = 0x7E00


def log(msg):
    sys.stderr.write("[gpu-attn] %s\n" % msg)
    sys.stderr.flush()


def make(B, H, Hkv, Lq, Lk, d, seed, layout="bhld"):
    """Seeded N(0,1) fp16 Q, K, V (bits) in the given layout, with strides."""
    def one(heads, L, s):
        x = gen.to_f16_bits(gen.normal(s, B * heads * L * d))
        if layout == "bhld":
            return x, (heads * L * d, L * d, d)
        # [B, L, heads, d] storage: element (b, h, i, c) at b*L*heads*d + i*heads*d + h*d + c
        x4 = x.reshape(B, heads, L, d).transpose(0, 2, 1, 3).copy()
        return x4.reshape(-1), (L * heads * d, d, heads * d)
    Q, qs = one(H, Lq, seed)
    K, ks = one(Hkv, Lk, seed + 1)
    V, vs = one(Hkv, Lk, seed + 2)
    return (Q, qs), (K, ks), (V, vs)


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()


def run(B, H, Hkv, Lq, Lk, d, causal, seed=0, layout="bhld", scale=None, what=""):
    (Q, qs), (K, ks), (V, vs) = make(B, H, Hkv, Lq, Lk, d, seed, layout)
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    log("%s B=%d H=%d Hkv=%d Lq=%d Lk=%d d=%d causal=%d %s" % (what, B, H, Hkv, Lq, Lk, d,
                                                                causal, layout))
    tq, tk, tv = dev(Q), dev(K), dev(V)
    n_o = max(B * H * Lq * d, 1)
    to = torch.full((n_o,), F16_NAN, dtype=torch.int16, device="cuda")
    tl = torch.full((max(B * H * Lq, 1),), float("nan"), dtype=torch.float32, device="cuda")
    os_ = (H * Lq * d, Lq * d, d)
    st = tg.tg_attention_fwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), to.data_ptr(),
                             tl.data_ptr(), B, H, Hkv, Lq, Lk, d, qs, ks, vs, os_, scale, causal,
                             torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_SUCCESS, tg.tg_status_string(st)
    torch.cuda.synchronize()
    O = to.cpu().numpy().view(np.uint16)[:B * H * Lq * d].reshape(B, H, Lq, d)
    lse = tl.cpu().numpy()[:B * H * Lq].reshape(B, H, Lq)
    return (Q, qs), (K, ks), (V, vs), O, lse, scale


def n_visible(Lq, Lk, causal):
    i = np.arange(Lq)
    return np.clip(i + (Lk - Lq) + 1, 0, Lk) if causal else np.full(Lq, Lk)


def check(O, lse, Oref, lse_ref, A, vmax, nvis, what):
    got = O.view(np.float16).astype(np.float64)
    assert not np.any(np.isnan(got)), what + ": NaN in O"
    tol = 2.0 ** -10 * A + (nvis * 2.0 ** -24 * vmax)[..., None] + parity.ulp16(Oref)
    err = np.abs(got - Oref)
    bad = err > tol
    if bad.any():
        idx = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d of %d outside tolerance, first %s: gpu %r ref %r tol %r" % (
            what, bad.sum(), bad.size, idx, got[idx], Oref[idx], tol[idx]))
    inf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), inf_ref), what + ": -inf rows differ"
    fin = ~inf_ref
    lerr = np.abs(lse[fin] - lse_ref[fin])
    assert np.all(lerr <= 2e-5 * (1 + np.abs(lse_ref[fin]))), (what, lerr.max())


CASES = [
    # B, H, Hkv, Lq, Lk, d, causal
    (1, 2, 2, 128, 128, 64, False),
    (1, 2, 2, 128, 128, 128, True),
    (2, 3, 1, 200, 333, 128, False),     # ragged, grouped K/V heads
    (2, 3, 1, 200, 333, 64, True),
    (1, 4, 2, 300, 100, 128, True),      # more queries than keys: empty rows
    (1, 2, 2, 100, 300, 64, True),       # fewer queries than keys
    (1, 1, 1, 1, 1, 128, False),
    (1, 1, 1, 1, 77, 64, True),
    (1, 2, 1, 257, 64, 128, False),
    (1, 1, 1, 130, 0, 64, False),        # no keys at all
    # causal over several query blocks, odd key-tile counts: the waves skip
    # the tiles past their own diagonal, in both halves of the unrolled loop
    (1, 2, 2, 1000, 1000, 128, True),
    (1, 3, 3, 700, 900, 128, True),
    (1, 2, 1, 900, 700, 64, True),
]


@pytest.mark.parametrize("B,H,Hkv,Lq,Lk,d,causal", CASES)
def test_attention_matches_oracle(B, H, Hkv, Lq, Lk, d, causal):
    (Q, qs), (K, ks), (V, vs), O, lse, scale = run(B, H, Hkv, Lq, Lk, d, causal, seed=7)
    Oref, lref, A = oracle.attention_ref(Q, K, V, B, H, Hkv, Lq, Lk, d, qs, ks, vs, scale, causal)
    vmax = np.abs(oracle.decode(V)).max() if Lk else 0.0
    nv = np.broadcast_to(n_visible(Lq, Lk, causal), (B, H, Lq))
    check(O, lse, Oref, lref, A, vmax, nv, str((B, H, Hkv, Lq, Lk, d, causal)))


@pytest.mark.parametrize("causal", [False, True])
def test_blhd_layout_and_scale(causal):
    B, H, Hkv, Lq, Lk, d = 2, 4, 2, 190, 250, 128
    (Q, qs), (K, ks), (V, vs), O, lse, scale = run(B, H, Hkv, Lq, Lk, d, causal, seed=8,
                                                   layout="blhd", scale=0.2, what="blhd")
    Oref, lref, A = oracle.attention_ref(Q, K, V, B, H, Hkv, Lq, Lk, d, qs, ks, vs, scale, causal)
    vmax = np.abs(oracle.decode(V)).max()
    nv = np.broadcast_to(n_visible(Lq, Lk, causal), (B, H, Lq))
    check(O, lse, Oref, lref, A, vmax, nv, "blhd")


def test_large_sampled_rows():
    """4 x 16 heads x 2048^2 x 128, causal: sampled query rows of every
    query block (first and last row of each block plus random ones)."""
    B, H, Hkv, L, d = 2, 8, 8, 2048, 128
    (Q, qs), (K, ks), (V, vs), O, lse, scale = run(B, H, Hkv, L, L, d, True, seed=9, what="large")
    rng = np.random.default_rng(1)
    rows = []
    for b in range(B):
        for h in range(H):
            for i in list(range(0, L, 128)) + list(range(127, L, 128)) + list(rng.integers(0, L, 8)):
                rows.append((b, h, int(i)))
    rows = np.array(rows)
    Or, lr, Ar = oracle.attention_rows(Q, K, V, B, H, Hkv, L, L, d, qs, ks, vs, scale, True, rows)
    got = O[rows[:, 0], rows[:, 1], rows[:, 2]]
    gl = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    vmax = np.abs(oracle.decode(V)).max()
    nv = n_visible(L, L, True)[rows[:, 2]]
    check(got, gl, Or, lr, Ar, vmax, nv, "large sampled")


def test_torch_wrapper_and_errors():
    B, H, L, d = 1, 2, 96, 64
    q = torch.randn(B, L, H, d, device="cuda").half().transpose(1, 2)   # (B, H, L, d) view
    k = torch.randn(B, L, H, d, device="cuda").half().transpose(1, 2)
    v = torch.randn(B, L, H, d, device="cuda").half().transpose(1, 2)
    out, lse = tg.attention(q, k, v, causal=True, return_lse=True)
    ref = torch.softmax((q.float() @ k.float().transpose(-1, -2)) / math.sqrt(d) +
                        torch.triu(torch.full((L, L), float("-inf"), device="cuda"), 1), -1) @ v.float()
    assert (out.float() - ref).abs().max().item() < 5e-3
    s = torch.cuda.current_stream().cuda_stream
    st = (H * L * d, L * d, d)
    assert tg.tg_attention_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), None,
                               B, H, H, L, L, 96, st, st, st, st, 0.1, 0,
                               s) == tg.TG_ERROR_UNSUPPORTED
    host = np.zeros(B * H * L * d, np.float16)
    assert tg.tg_attention_fwd(host.ctypes.data, k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               None, B, H, H, L, L, d, st, st, st, st, 0.1, 0,
                               s) == tg.TG_ERROR_NOT_DEVICE_MEMORY


def run_values(Qv, Kv, Vv, causal, scale, what):
    """Attention on given float arrays [B, H, L, d] (rounded to fp16)."""
    B, H, Lq, d = Qv.shape
    Hkv, Lk = Kv.shape[1], Kv.shape[2]
    Q, K, V = (np.ascontiguousarray(x, np.float64).astype(np.float16).view(np.uint16).reshape(-1)
               for x in (Qv, Kv, Vv))
    qs, ks = (H * Lq * d, Lq * d, d), (Hkv * Lk * d, Lk * d, d)
    log("%s B=%d H=%d Lq=%d Lk=%d d=%d causal=%d scale=%g" % (what, B, H, Lq, Lk, d, causal, scale))
    tq, tk, tv = dev(Q), dev(K), dev(V)
    to = torch.full((B * H * Lq * d,), F16_NAN, dtype=torch.int16, device="cuda")
    tl = torch.empty(B * H * Lq, dtype=torch.float32, device="cuda")
    st = tg.tg_attention_fwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), to.data_ptr(),
                             tl.data_ptr(), B, H, Hkv, Lq, Lk, d, qs, ks, ks, qs, scale, causal,
                             torch.cuda.current_stream().cuda_stream)
    assert st == tg.TG_SUCCESS, tg.tg_status_string(st)
    torch.cuda.synchronize()
    O = to.cpu().numpy().view(np.uint16).reshape(B, H, Lq, d)
    lse = tl.cpu().numpy().reshape(B, H, Lq)
    Oref, lref, A = oracle.attention_ref(Q, K, V, B, H, Hkv, Lq, Lk, d, qs, ks, ks, scale, causal)
    vmax = np.abs(Vv).max()
    nv = np.broadcast_to(n_visible(Lq, Lk, causal), (B, H, Lq))
    check(O, lse, Oref, lref, A, vmax, nv, what)


@pytest.mark.parametrize("scale", [-0.1, 0.0, 0.7])
def test_scale_sign_and_zero(scale):
    rng = np.random.default_rng(3)
    Qv, Kv, Vv = (rng.standard_normal((1, 2, 160, 64)) for _ in range(3))
    run_values(Qv, Kv, Vv, True, scale, "scale %g" % scale)


@pytest.mark.parametrize("scale", [0.0, -0.0, 1e-35, -1e-35])
def test_zero_scale_gives_exactly_uniform_weights(scale):
    """A zero (or negligible) scale: every visible key weighs the same, so O
    is the mean of the visible V rows and lse = log(visible keys), with no
    NaN from masked keys."""
    B, H, Lq, Lk, d = 1, 2, 160, 96, 64
    rng = np.random.default_rng(6)
    Qv, Kv, Vv = (8.0 * rng.standard_normal((B, H, L, d)) for L in (Lq, Lk, Lk))
    Q, K, V = (np.ascontiguousarray(x).astype(np.float16).view(np.uint16).reshape(-1)
               for x in (Qv, Kv, Vv))
    qs, ks = (H * Lq * d, Lq * d, d), (H * Lk * d, Lk * d, d)
    tq, tk, tv = dev(Q), dev(K), dev(V)
    to = torch.full((B * H * Lq * d,), F16_NAN, dtype=torch.int16, device="cuda")
    tl = torch.empty(B * H * Lq, dtype=torch.float32, device="cuda")
    assert tg.tg_attention_fwd(tq.data_ptr(), tk.data_ptr(), tv.data_ptr(), to.data_ptr(),
                               tl.data_ptr(), B, H, H, Lq, Lk, d, qs, ks, ks, qs, scale, 1,
                               torch.cuda.current_stream().cuda_stream) == tg.TG_SUCCESS
    torch.cuda.synchronize()
    O = to.cpu().numpy().view(np.float16).astype(np.float64).reshape(B, H, Lq, d)
    lse = tl.cpu().numpy().reshape(B, H, Lq)
    nv = np.broadcast_to(n_visible(Lq, Lk, True), (B, H, Lq))
    seen = nv > 0
    assert np.all(np.abs(lse[seen] - np.log(nv[seen])) <= 4e-7 * (1 + np.log(nv[seen])))
    assert np.all(np.isneginf(lse[~seen])) and np.all(O[~seen] == 0)
    V16 = V.view(np.float16).astype(np.float64).reshape(B, H, Lk, d)
    csum = np.cumsum(V16, axis=2)
    for i in range(Lq):
        n = int(nv[0, 0, i])
        if n:
            mean = csum[:, :, n - 1] / n
            # fp16 weights of exactly 1, an fp32 sum of n terms, one division,
            # then the fp16 rounding of O
            tol = n * 2.0 ** -24 * np.abs(V16).max() + 2.0 ** -11 * np.abs(mean) + 2.0 ** -24
            assert np.all(np.abs(O[:, :, i] - mean) <= tol), i


def test_running_maximum_keeps_growing():
    """Scores rise along the keys (0.8 per key for most rows), so the row
    maximum jumps past the reference again and again."""
    L, d = 512, 64
    rng = np.random.default_rng(4)
    Qv = 2.0 + 0.1 * rng.standard_normal((1, 1, L, d))
    Kv = (0.05 * np.arange(L))[None, None, :, None] * np.ones((1, 1, L, d))
    Vv = rng.standard_normal((1, 1, L, d))
    for causal in (False, True):
        run_values(Qv, Kv, Vv, causal, 0.125, "growing max causal=%d" % causal)


def test_score_levels_far_from_zero():
    """All scores near -128 or +120 (natural units): only their differences
    matter."""
    L, d = 300, 64
    rng = np.random.default_rng(5)
    Kv = -2.0 + 0.05 * rng.standard_normal((1, 2, L, d))
    Vv = rng.standard_normal((1, 2, L, d))
    Qv = np.concatenate([np.full((1, 1, L, d), 2.0), np.full((1, 1, L, d), -1.875)], axis=1)
    run_values(Qv, Kv, Vv, True, 0.125, "far score levels")

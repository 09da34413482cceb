"""Pins for the CPU oracle: each check compares it with something other than
itself -- numpy's fp16 conversion, exact rational arithmetic, closed forms and
invariants -- so that a dropped term, a wrong sign or index, a transposed
operand, a bad leading dimension or a rounding slip fails at least one."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import tg_inputs as gen


def f16(vals):
    return np.asarray(vals, dtype=np.float16).view(np.uint16)


def exact(bits):
    """fp16 bits -> exact Fractions through numpy's (independent) decoding."""
    return [[Fraction(float(v)) for v in row] for row in bits.view(np.float16).astype(np.float64)]


# ---------------------------------------------------------------- fp16 codec

def test_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_encode_round_trips_every_finite_value():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    keep = ~np.isnan(vals)
    assert np.array_equal(oracle.encode_f16(vals[keep]), bits[keep])


def test_encode_midpoints_and_neighbours_match_numpy():
    # every pair of adjacent positive fp16 values: the midpoint (a tie) and
    # points just either side of it must round as numpy's direct
    # double -> half conversion rounds them
    pos = np.arange(0, 0x7c00, dtype=np.uint16).view(np.float16).astype(np.float64)
    lo, hi = pos[:-1], pos[1:]
    mid = (lo + hi) / 2
    probe = np.concatenate([mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)])
    probe = np.concatenate([probe, -probe])
    want = probe.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.encode_f16(probe), want)


def test_encode_overflow_underflow_and_random_doubles():
    special = np.array([65504.0, 65519.99, 65520.0, 65536.0, 1e30, 2.0 ** -24,
                        2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -26, 1e-30, 0.0, -0.0])
    special = np.concatenate([special, -special])
    rng = np.random.default_rng(7)
    rand = np.ldexp(rng.random(200000) + 0.5, rng.integers(-30, 18, 200000))
    rand *= np.where(rng.random(200000) < 0.5, -1, 1)
    for x in (special, rand):
        with np.errstate(over="ignore"):
            want = x.astype(np.float16).view(np.uint16)
        assert np.array_equal(oracle.encode_f16(x), want)


def test_f32_rounding_matches_numpy():
    rng = np.random.default_rng(8)
    x = rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000)
    assert np.array_equal(oracle.to_f32(x), x.astype(np.float32))


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("M,K", [(37, 45), (5, 256), (3, 1031)])
def test_identity_B_gives_A(M, K):
    A = gen.to_f16_bits(gen.uniform_pm1(11, M * K)).reshape(M, K)
    B = np.zeros((K, K), np.uint16)
    B[np.arange(K), np.arange(K)] = 0x3C00          # fp16 1.0
    C = oracle.gemm_ref(A, B, M, K, K)
    assert np.array_equal(C, A.view(np.float16).astype(np.float64))


@pytest.mark.parametrize("K", [1, 7, 64, 1031, 4096])
def test_all_ones_gives_K(K):
    M, N = 3, 5
    A = np.full((M, K), 0x3C00, np.uint16)
    B = np.full((K, N), 0x3C00, np.uint16)
    C = oracle.gemm_ref(A, B, M, N, K)
    assert np.all(C == float(K))
    assert np.all(oracle.to_f32(C) == np.float32(K))


def test_K1_is_the_exact_outer_product():
    M, N = 9, 13
    a = gen.to_f16_bits(gen.uniform_pm1(12, M)).reshape(M, 1)
    b = gen.to_f16_bits(gen.uniform_pm1(13, N)).reshape(1, N)
    C = oracle.gemm_ref(a, b, M, N, 1)
    ea, eb = exact(a), exact(b)
    for i in range(M):
        for j in range(N):
            assert Fraction(C[i, j]) == ea[i][0] * eb[0][j]


def test_fused_with_zero_A_is_relu_of_bias():
    M, N, K = 4, 33, 17
    A = np.zeros((M, K), np.uint16)
    B = gen.to_f16_bits(gen.uniform_pm1(14, K * N)).reshape(K, N)
    bias = gen.normal(15, N).astype(np.float32)
    C = oracle.gemm_ref(A, B, M, N, K, bias=bias)
    want = np.maximum(bias.astype(np.float64), 0.0)
    assert np.array_equal(C, np.broadcast_to(want, (M, N)))
    assert not np.any(np.signbit(C))                  # ReLU gives +0, never -0
    assert np.array_equal(oracle.output_typed(C, "f16")[0],
                          want.astype(np.float16).view(np.uint16))


def test_K0_gives_zero_or_relu_bias():
    M, N = 3, 4
    A = np.zeros((M, 0), np.uint16)
    B = np.zeros((0, N), np.uint16)
    assert np.array_equal(oracle.gemm_ref(A, B, M, N, 0), np.zeros((M, N)))
    bias = np.array([-1.5, 0.0, 2.25, -0.0], np.float32)
    C = oracle.gemm_ref(A, B, M, N, 0, bias=bias)
    assert np.array_equal(C[1], [0.0, 0.0, 2.25, 0.0])
    assert not np.any(np.signbit(C))


# ------------------------------------------------- exact rational brute force

def _brute(A, B, M, N, K, bias=None):
    ea, eb = exact(A), exact(B)
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            s = sum((ea[i][k] * eb[k][j] for k in range(K)), Fraction(0))
            if bias is not None:
                s = s + Fraction(float(bias[j]))
                s = max(s, Fraction(0))
            row.append(s)
        out.append(row)
    return out


SHAPES = [(4, 4, 4)] + sorted(set(itertools.permutations((7, 5, 3))))


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("kind", ["uniform", "int", "normal_scaled"])
@pytest.mark.parametrize("fused", [False, True])
def test_brute_force_exact(M, N, K, kind, fused):
    seed = 100 + M * 49 + N * 7 + K
    A, B = gen.operands(M, N, K, kind, seed)
    bias = gen.bias_vector(N, seed + 1, integer=(kind == "int")) if fused else None
    C = oracle.gemm_ref(A, B, M, N, K, bias=bias)
    ex = _brute(A, B, M, N, K, bias)
    for i in range(M):
        for j in range(N):
            # |values| <= 4 and K <= 7: the fp64 sum is exact, so the oracle must
            # equal the exact value rounded once (Python's float(Fraction) is
            # correctly rounded)
            assert C[i, j] == float(ex[i][j]), (i, j)
            if fused:
                assert not np.signbit(C[i, j])
    # output-typed values: one correct rounding of the exact value
    f16_want = np.array([[float(v) for v in row] for row in ex]).astype(np.float16)
    assert np.array_equal(oracle.output_typed(C, "f16"), f16_want.view(np.uint16))


# ---------------------------------------------------------------- invariants

def test_transpose_invariant_bit_exact():
    M, N, K = 23, 31, 57
    A, B = gen.operands(M, N, K, "uniform", 21)
    C = oracle.gemm_ref(A, B, M, N, K)
    Ct = oracle.gemm_ref(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), N, M, K)
    assert np.array_equal(C.T, Ct)


def test_row_and_column_permutations_commute():
    M, N, K = 19, 29, 41
    A, B = gen.operands(M, N, K, "normal_scaled", 22)
    bias = gen.bias_vector(N, 23)
    C = oracle.gemm_ref(A, B, M, N, K, bias=bias)
    rng = np.random.default_rng(3)
    pr, pc = rng.permutation(M), rng.permutation(N)
    Cp = oracle.gemm_ref(A[pr], np.ascontiguousarray(B[:, pc]), M, N, K, bias=bias[pc])
    assert np.array_equal(Cp, C[pr][:, pc])


def test_padded_leading_dimensions_ignore_padding():
    M, N, K = 17, 21, 33
    lda, ldb = K + 5, N + 3
    A, B = gen.operands(M, N, K, "uniform", 24)
    Ap = np.full((M, lda), 0x7E00, np.uint16)      # NaN in the padding
    Bp = np.full((K, ldb), 0x7E00, np.uint16)
    Ap[:, :K] = A
    Bp[:, :N] = B
    C = oracle.gemm_ref(A, B, M, N, K)
    Cp = oracle.gemm_ref(Ap, Bp, M, N, K, lda=lda, ldb=ldb)
    assert np.array_equal(C, Cp)


def test_entries_match_full_product():
    M, N, K = 40, 50, 300
    A, B = gen.operands(M, N, K, "uniform", 25)
    bias = gen.bias_vector(N, 26)
    for b in (None, bias):
        C = oracle.gemm_ref(A, B, M, N, K, bias=b)
        rng = np.random.default_rng(5)
        r, c = rng.integers(0, M, 200), rng.integers(0, N, 200)
        assert np.array_equal(oracle.gemm_entries(A, B, r, c, K, K, N, bias=b), C[r, c])


def test_integer_inputs_are_exact_at_large_K():
    # integer operands in {-4..4}: every partial sum is an integer < 2^24, so the
    # oracle must agree with exact integer arithmetic (numpy int64) bit for bit
    M, N, K = 16, 24, 8192
    A, B = gen.operands(M, N, K, "int", 27)
    C = oracle.gemm_ref(A, B, M, N, K)
    Ai = A.view(np.float16).astype(np.int64)
    Bi = B.view(np.float16).astype(np.int64)
    assert np.array_equal(C, (Ai @ Bi).astype(np.float64))


# ------------------------------------------------------- transposed operands

def _stored(logical, op, pad, seed):
    """Stored array for a logical operand: itself (op 0) or its transpose
    (op 1), by numpy, in rows padded with NaN to width + pad."""
    st = np.ascontiguousarray(logical.T) if op else logical
    rows, cols = st.shape
    out = np.full((rows, cols + pad), 0x7E00, np.uint16)
    out[:, :cols] = st
    return out, cols + pad


def test_transposed_operands_match_numpy_transposes():
    M, N, K = 13, 22, 37
    A, B = gen.operands(M, N, K, "uniform", 40)
    bias = gen.bias_vector(N, 41)
    for op_a, op_b, b in itertools.product((0, 1), (0, 1), (None, bias)):
        As, lda = _stored(A, op_a, 3, 0)
        Bs, ldb = _stored(B, op_b, 5, 0)
        want = oracle.gemm_ref(A, B, M, N, K, bias=b)
        got = oracle.gemm_ref(As, Bs, M, N, K, lda=lda, ldb=ldb, bias=b, op_a=op_a, op_b=op_b)
        assert np.array_equal(got, want), (op_a, op_b)
        r = np.array([0, M - 1, 5, 7])
        c = np.array([0, N - 1, 11, 3])
        ent = oracle.gemm_entries(As, Bs, r, c, K, lda, ldb, bias=b, op_a=op_a, op_b=op_b)
        assert np.array_equal(ent, want[r, c]), (op_a, op_b)


@pytest.mark.parametrize("M,N,K,op_a,op_b", [(5, 3, 7, 1, 0), (5, 3, 7, 0, 1), (5, 3, 7, 1, 1),
                                             (4, 6, 2, 1, 1)])
def test_transposed_brute_force_exact(M, N, K, op_a, op_b):
    # stored operands drawn directly; the logical op(A), op(B) come from numpy
    sa = (K, M) if op_a else (M, K)
    sb = (N, K) if op_b else (K, N)
    As = gen.to_f16_bits(gen.uniform_pm1(60 + M, sa[0] * sa[1])).reshape(sa)
    Bs = gen.to_f16_bits(gen.uniform_pm1(61 + N, sb[0] * sb[1])).reshape(sb)
    A = np.ascontiguousarray(As.T) if op_a else As
    B = np.ascontiguousarray(Bs.T) if op_b else Bs
    C = oracle.gemm_ref(As, Bs, M, N, K, op_a=op_a, op_b=op_b)
    ex = _brute(A, B, M, N, K)
    for i in range(M):
        for j in range(N):
            assert C[i, j] == float(ex[i][j]), (i, j)


def test_transposed_rejects_short_leading_dimensions():
    # a stored K x M operand needs lda >= M, a stored N x K one ldb >= K
    A = np.zeros(64, np.uint16)
    with pytest.raises(ValueError):
        oracle.gemm_ref(A, A, 4, 2, 2, lda=2, ldb=2, op_a=1)
    with pytest.raises(ValueError):
        oracle.gemm_ref(A, A, 2, 4, 3, lda=3, ldb=2, op_b=1)


# ------------------------------------------------------------ int8 operands

def _stored_i8(logical, op):
    return np.ascontiguousarray(logical.T) if op else logical


@pytest.mark.parametrize("M,N,K", [(4, 4, 4), (7, 5, 3), (3, 7, 5)])
def test_int8_brute_force_exact(M, N, K):
    A, B = gen.operands_i8(M, N, K, 70 + M)
    for op_a, op_b in itertools.product((0, 1), (0, 1)):
        C = oracle.gemm_i8_ref(_stored_i8(A, op_a), _stored_i8(B, op_b), M, N, K, op_a=op_a,
                               op_b=op_b)
        for i in range(M):
            for j in range(N):
                want = sum(int(A[i, k]) * int(B[k, j]) for k in range(K))
                assert int(C[i, j]) == want, (op_a, op_b, i, j)


def test_int8_matches_numpy_int64_matmul_all_orientations():
    M, N, K = 67, 45, 300
    A, B = gen.operands_i8(M, N, K, 71)
    want = A.astype(np.int64) @ B.astype(np.int64)
    for op_a, op_b in itertools.product((0, 1), (0, 1)):
        As, Bs = _stored_i8(A, op_a), _stored_i8(B, op_b)
        got = oracle.gemm_i8_ref(As, Bs, M, N, K, op_a=op_a, op_b=op_b)
        assert np.array_equal(got, want), (op_a, op_b)
        r, c = np.array([0, M - 1, 31]), np.array([N - 1, 0, 17])
        ent = oracle.gemm_i8_entries(As, Bs, r, c, K, As.shape[1], Bs.shape[1], op_a=op_a,
                                     op_b=op_b)
        assert np.array_equal(ent, want[r, c])


def test_int8_extremes_and_padding():
    # -128 * -128 summed K times is the largest magnitude; K = 131071 stays
    # below 2^31 (the int32 bound the library enforces)
    K = 131071
    A = np.full((1, K), -128, np.int8)
    B = np.full((K, 2), -128, np.int8)
    B[:, 1] = 127
    C = oracle.gemm_i8_ref(A, B, 1, 2, K)
    assert C[0, 0] == 16384 * K and C[0, 0] < 2 ** 31
    assert C[0, 1] == -16256 * K
    # padded rows are ignored
    M, N, K = 5, 6, 9
    A, B = gen.operands_i8(M, N, K, 72)
    Ap = np.full((M, K + 7), 99, np.int8)
    Ap[:, :K] = A
    Bp = np.full((K, N + 3), -99, np.int8)
    Bp[:, :N] = B
    assert np.array_equal(oracle.gemm_i8_ref(Ap, Bp, M, N, K, lda=K + 7, ldb=N + 3),
                          oracle.gemm_i8_ref(A, B, M, N, K))


def test_int8_generator_range():
    v = gen.ints_i8(3, 100000)
    assert v.dtype == np.int8 and v.min() == -128 and v.max() == 127
    assert abs(float(v.mean()) + 0.5) < 1.0

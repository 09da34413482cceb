"""CPU oracle for the tiled fp16 GEMM (+ fused bias + ReLU).

TEST INFRASTRUCTURE: only the tests, the smoke check and the bench's CPU
baseline may import this package.  It is a plain fp64 implementation of the
definition C = A.B (and C = max(A.B + bias, 0)) written from the TileLang pages
(lqnn.cn walkthrough sections 2.1 and 4.2; codechina.net article section 3.2;
xdnf.cn article section 4.2), in C (tgref.c), bound here with ctypes.  It
shares no code with the HIP library and never imports it.

Every function is pinned by tests/test_oracle.py against closed forms, exact
rational brute force, invariants and numpy's own fp16 conversion.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.tgref_f16_decode.argtypes = [ctypes.c_uint16]
        L.tgref_f16_decode.restype = ctypes.c_double
        L.tgref_f16_encode.argtypes = [ctypes.c_double]
        L.tgref_f16_encode.restype = ctypes.c_uint16
        L.tgref_decode_array.argtypes = [P, P, I64]
        L.tgref_to_f32.argtypes = [P, P, I64]
        L.tgref_to_f16.argtypes = [P, P, I64]
        L.tgref_gemm.argtypes = [P, P, P, P, I64, I64, I64, I64, I64, I64, ctypes.c_int]
        L.tgref_gemm.restype = ctypes.c_int
        L.tgref_gemm_entries.argtypes = [P, P, P, P, P, I64, P, I64, I64, I64]
        L.tgref_gemm_entries.restype = ctypes.c_int
        I = ctypes.c_int
        L.tgref_gemm_ex.argtypes = [I, I, P, P, P, P, I64, I64, I64, I64, I64, I64, I]
        L.tgref_gemm_ex.restype = I
        L.tgref_gemm_entries_ex.argtypes = [I, I, P, P, P, P, P, I64, P, I64, I64, I64]
        L.tgref_gemm_entries_ex.restype = I
        L.tgref_gemm_i8_ex.argtypes = [I, I, P, P, P, I64, I64, I64, I64, I64, I64, I]
        L.tgref_gemm_i8_ex.restype = I
        L.tgref_gemm_i8_entries_ex.argtypes = [I, I, P, P, P, P, I64, P, I64, I64, I64]
        L.tgref_gemm_i8_entries_ex.restype = I
        D = ctypes.c_double
        L.tgref_attention.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, P, P, P, D, I,
                                      P, P, P, I]
        L.tgref_attention.restype = I
        L.tgref_attention_rows.argtypes = [P, P, P, I64, I64, I64, I64, I64, I64, P, P, P, D,
                                           I, P, I64, P, P, P, I]
        L.tgref_attention_rows.restype = I
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float16:
        a = a.view(np.uint16)
    assert a.dtype == np.uint16, a.dtype
    return a


def default_threads():
    """Threads for the oracle: the CPUs this process may run on, or fewer when
    OMP_NUM_THREADS declares a smaller share of the host."""
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    if share.isdigit() and int(share) > 0:
        n = min(n, int(share))
    return max(1, n)


def cpu_model():
    """The host CPU's model name (lscpu's 'Model name'), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def decode(bits):
    """fp16 bit patterns (uint16) -> exact float64 values."""
    bits = _u16(bits)
    out = np.empty(bits.shape, np.float64)
    lib().tgref_decode_array(_ptr(bits), _ptr(out), bits.size)
    return out


def encode_f16(x):
    """float64 -> fp16 bit patterns by direct round-to-nearest-even."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().tgref_to_f16(_ptr(x), _ptr(out), x.size)
    return out


def to_f32(x):
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.float32)
    lib().tgref_to_f32(_ptr(x), _ptr(out), x.size)
    return out


def gemm_ref(A, B, M, N, K, lda=None, ldb=None, bias=None, nthreads=None, op_a=0, op_b=0):
    """Unrounded fp64 reference C (M x N, dense) of op(A).op(B) for fp16-bit
    operands.

    A: uint16 bits, row-major with leading dim lda: M x K (op_a = 0) or stored
       K x M (op_a = 1).
    B: uint16 bits: K x N (op_b = 0) or stored N x K (op_b = 1).
    bias: None (plain GEMM) or float32[N] (fused bias + ReLU).
    """
    ar, ac = (K, M) if op_a else (M, K)
    br, bc = (N, K) if op_b else (K, N)
    lda = ac if lda is None else lda
    ldb = bc if ldb is None else ldb
    A = _u16(A).reshape(-1)
    B = _u16(B).reshape(-1)
    if ar > 0 and ac > 0:
        assert A.size >= (ar - 1) * lda + ac
    if br > 0 and bc > 0:
        assert B.size >= (br - 1) * ldb + bc
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.size >= N
    C = np.zeros((M, N), np.float64)
    rc = lib().tgref_gemm_ex(op_a, op_b, _ptr(A), _ptr(B), _ptr(bias), _ptr(C), M, N, K, lda,
                             ldb, N, nthreads or default_threads())
    if rc != 0:
        raise ValueError("tgref_gemm_ex rejected its arguments")
    return C


def gemm_entries(A, B, rows, cols, K, lda, ldb, bias=None, op_a=0, op_b=0):
    """Unrounded fp64 reference values of op(A).op(B) at the listed (row, col)
    positions."""
    A = _u16(A).reshape(-1)
    B = _u16(B).reshape(-1)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
    out = np.empty(rows.shape, np.float64)
    rc = lib().tgref_gemm_entries_ex(op_a, op_b, _ptr(A), _ptr(B), _ptr(bias), _ptr(rows),
                                     _ptr(cols), rows.size, _ptr(out), K, lda, ldb)
    if rc != 0:
        raise ValueError("tgref_gemm_entries_ex rejected its arguments")
    return out


def _i8(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.int8, a.dtype
    return a.reshape(-1)


def gemm_i8_ref(A, B, M, N, K, lda=None, ldb=None, nthreads=None, op_a=0, op_b=0):
    """Exact int64 C (M x N) of op(A).op(B) for int8 operands (stored as for
    gemm_ref: M x K or, with op_a, K x M; K x N or, with op_b, N x K)."""
    lda = (M if op_a else K) if lda is None else lda
    ldb = (K if op_b else N) if ldb is None else ldb
    C = np.zeros((M, N), np.int64)
    rc = lib().tgref_gemm_i8_ex(op_a, op_b, _ptr(_i8(A)), _ptr(_i8(B)), _ptr(C), M, N, K, lda,
                                ldb, N, nthreads or default_threads())
    if rc != 0:
        raise ValueError("tgref_gemm_i8_ex rejected its arguments")
    return C


def gemm_i8_entries(A, B, rows, cols, K, lda, ldb, op_a=0, op_b=0):
    """Exact int64 values of op(A).op(B) at the listed (row, col) positions."""
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    out = np.empty(rows.shape, np.int64)
    rc = lib().tgref_gemm_i8_entries_ex(op_a, op_b, _ptr(_i8(A)), _ptr(_i8(B)), _ptr(rows),
                                        _ptr(cols), rows.size, _ptr(out), K, lda, ldb)
    if rc != 0:
        raise ValueError("tgref_gemm_i8_entries_ex rejected its arguments")
    return out


def output_typed(cref, c_dtype):
    """Round the fp64 reference to the output type: 'f32' -> float32 (RNE),
    'f16' -> fp16 bit patterns (direct RNE from double)."""
    if c_dtype == "f32":
        return to_f32(cref)
    if c_dtype == "f16":
        return encode_f16(cref)
    raise ValueError(c_dtype)


# ------------------------------------------------------------ attention --
def _strides(st):
    st = np.ascontiguousarray(st, dtype=np.int64)
    assert st.shape == (3,)
    return st


def attention_ref(Q, K, V, B, H, Hkv, Lq, Lk, d, q_strides, k_strides, v_strides, scale,
                  causal=False, nthreads=None):
    """fp64 reference of scaled dot-product attention (tgref_attention.c):
    returns O [B, H, Lq, d], lse [B, H, Lq] and the softmax-weighted mean
    magnitude A [B, H, Lq, d] of V (for the error bound).

    Q, K, V: flat fp16 bit arrays (uint16) holding element (b, h, i, c) at
    b*s[0] + h*s[1] + i*s[2] + c with s the given {batch, head, row} strides;
    K and V have Hkv heads, query head h reading head h // (H // Hkv)."""
    Q, K, V = (np.ascontiguousarray(_u16(x)).reshape(-1) for x in (Q, K, V))
    qs, ks, vs = _strides(q_strides), _strides(k_strides), _strides(v_strides)
    O = np.zeros((B, H, Lq, d))
    lse = np.zeros((B, H, Lq))
    A = np.zeros((B, H, Lq, d))
    rc = lib().tgref_attention(_ptr(Q), _ptr(K), _ptr(V), B, H, Hkv, Lq, Lk, d, _ptr(qs),
                               _ptr(ks), _ptr(vs), float(scale), int(bool(causal)), _ptr(O),
                               _ptr(lse), _ptr(A), nthreads or default_threads())
    if rc != 0:
        raise ValueError("tgref_attention rejected its arguments (%d)" % rc)
    return O, lse, A


def attention_rows(Q, K, V, B, H, Hkv, Lq, Lk, d, q_strides, k_strides, v_strides, scale,
                   causal, rows, nthreads=None):
    """As attention_ref for the listed (b, h, i) query rows only; returns
    O [n, d], lse [n], A [n, d]."""
    Q, K, V = (np.ascontiguousarray(_u16(x)).reshape(-1) for x in (Q, K, V))
    qs, ks, vs = _strides(q_strides), _strides(k_strides), _strides(v_strides)
    rows = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1, 3)
    n = rows.shape[0]
    O = np.zeros((n, d))
    lse = np.zeros(n)
    A = np.zeros((n, d))
    rc = lib().tgref_attention_rows(_ptr(Q), _ptr(K), _ptr(V), B, H, Hkv, Lq, Lk, d, _ptr(qs),
                                    _ptr(ks), _ptr(vs), float(scale), int(bool(causal)),
                                    _ptr(rows), n, _ptr(O), _ptr(lse), _ptr(A),
                                    nthreads or default_threads())
    if rc != 0:
        raise ValueError("tgref_attention_rows rejected its arguments (%d)" % rc)
    return O, lse, A

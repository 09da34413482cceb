"""Seeded synthetic inputs for the tiled fp16 GEMM workloads.

Shared by the tests, the bench and the smoke check; it holds none of the
GEMM's arithmetic (no products, sums, bias or ReLU), only random numbers and
their conversion to the operand formats.  Both the HIP path and the CPU oracle
consume the same fp16 bytes produced here, so parity never depends on the
generator's details.

Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; the 64-bit finaliser constants are the ones
published with Java's SplittableRandom).  Draw t (t = 0, 1, ...) of the stream
with seed s is mix64(s + (t + 1) * 0x9E3779B97F4A7C15), which is what the
sequential generator returns on its (t+1)-th call, so it vectorises.

* uniform u in [0, 1): (x >> 11) * 2^-53
* uniform[-1, 1): 2u - 1
* normal: Box-Muller on the pair (1 - u1, u2): r = sqrt(-2 ln(1 - u1)),
  z0 = r cos(2 pi u2), z1 = r sin(2 pi u2); both outputs are used, in order
* integer in {-4..4}: floor(9u) - 4

For each workload, A (row-major, M x K) takes the first draws of the stream,
then B (row-major, K x N) the next ones.  The bias vector has its own stream.
Every operand value is rounded to fp16 (round to nearest even, numpy's
float64 -> float16 conversion); the bias is rounded to fp32.
"""
import math

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_CHUNK = 1 << 22


def splitmix64(seed, n, start=0):
    """Draws start .. start+n-1 of the SplitMix64 stream with this seed."""
    out = np.empty(n, np.uint64)
    s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF)
    with np.errstate(over="ignore"):
        for b in range(0, n, _CHUNK):
            e = min(n, b + _CHUNK)
            z = np.arange(start + b + 1, start + e + 1, dtype=np.uint64) * GAMMA + s
            z ^= z >> np.uint64(30)
            z *= _M1
            z ^= z >> np.uint64(27)
            z *= _M2
            z ^= z >> np.uint64(31)
            out[b:e] = z
    return out


def uniform01(seed, n, start=0):
    return (splitmix64(seed, n, start) >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)


def uniform_pm1(seed, n, start=0):
    return 2.0 * uniform01(seed, n, start) - 1.0


def normal(seed, n, start=0):
    """Normal values start .. start+n-1 of the Box-Muller stream (pairs of draws)."""
    p0 = start // 2
    p1 = (start + n + 1) // 2
    u = uniform01(seed, 2 * (p1 - p0), 2 * p0)
    u1 = u[0::2]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log1p(-u1))
    z = np.empty(2 * (p1 - p0), np.float64)
    z[0::2] = r * np.cos(2.0 * math.pi * u2)
    z[1::2] = r * np.sin(2.0 * math.pi * u2)
    off = start - 2 * p0
    return z[off:off + n]


def ints_pm4(seed, n, start=0):
    return np.floor(9.0 * uniform01(seed, n, start)) - 4.0


def to_f16_bits(x):
    """float64 values -> fp16 bit patterns (uint16), round to nearest even."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


# The five workloads: (name, M, N, K, value kind, seed, fused, output dtype).
WORKLOADS = {
    "sq256": dict(M=256, N=256, K=256, kind="uniform", seed=0, fused=False, c_dtype="f32"),
    "sq1024": dict(M=1024, N=1024, K=1024, kind="uniform", seed=1, fused=False, c_dtype="f32"),
    "sq8192": dict(M=8192, N=8192, K=8192, kind="normal_scaled", seed=2, fused=False,
                   c_dtype="f16"),
    "fused4096x11008x4096": dict(M=4096, N=11008, K=4096, kind="uniform", seed=3, fused=True,
                                 c_dtype="f16", bias_seed=4),
    "ragged3001x5003x1031": dict(M=3001, N=5003, K=1031, kind="uniform", seed=5, fused=False,
                                 c_dtype="f32"),
    # the 8192^3 problem with transposed operands (the backward products of a
    # linear layer); the stored operand is the transpose of the same values
    "sq8192_nt": dict(M=8192, N=8192, K=8192, kind="normal_scaled", seed=2, fused=False,
                      c_dtype="f16", op_b=1),
    "sq8192_tn": dict(M=8192, N=8192, K=8192, kind="normal_scaled", seed=2, fused=False,
                      c_dtype="f16", op_a=1),
    # int8 operands uniform over [-128, 127], exact int32 C
    "sq8192_i8": dict(M=8192, N=8192, K=8192, kind="i8", seed=6, fused=False, c_dtype="i32"),
    "sq8192_i8_nt": dict(M=8192, N=8192, K=8192, kind="i8", seed=6, fused=False,
                         c_dtype="i32", op_b=1),
}


def _values(kind, seed, n, start, K):
    if kind == "uniform":
        return uniform_pm1(seed, n, start)
    if kind == "normal_scaled":
        return normal(seed, n, start) / math.sqrt(K)
    if kind == "int":
        return ints_pm4(seed, n, start)
    raise ValueError(kind)


def operands(M, N, K, kind, seed):
    """fp16 bits of A (M x K) then B (K x N) from one stream."""
    A = to_f16_bits(_values(kind, seed, M * K, 0, K)).reshape(M, K)
    B = to_f16_bits(_values(kind, seed, K * N, M * K, K)).reshape(K, N)
    return A, B


def ints_i8(seed, n, start=0):
    """int8 values uniform over [-128, 127]: floor(256 u) - 128."""
    return (np.floor(256.0 * uniform01(seed, n, start)) - 128.0).astype(np.int8)


def operands_i8(M, N, K, seed):
    """int8 A (M x K) then B (K x N) from one stream."""
    A = ints_i8(seed, M * K, 0).reshape(M, K)
    B = ints_i8(seed, K * N, M * K).reshape(K, N)
    return A, B


def bias_vector(N, seed, integer=False):
    if integer:
        return ints_pm4(seed, N).astype(np.float32)
    return normal(seed, N).astype(np.float32)


def workload(name, integer=False):
    """Inputs of a named workload; integer=True draws A, B (and the bias) from
    {-4..4} with the same seeds, for the bit-exact check.  A and B are the
    stored arrays (transposed for workloads with op_a / op_b set)."""
    w = dict(WORKLOADS[name])
    kind = "int" if integer else w["kind"]
    if w["kind"] == "i8":
        A, B = operands_i8(w["M"], w["N"], w["K"], w["seed"])
    else:
        A, B = operands(w["M"], w["N"], w["K"], kind, w["seed"])
    op_a, op_b = w.get("op_a", 0), w.get("op_b", 0)
    if op_a:
        A = np.ascontiguousarray(A.T)   # stored K x M
    if op_b:
        B = np.ascontiguousarray(B.T)   # stored N x K
    bias = None
    if w["fused"]:
        bias = bias_vector(w["N"], w["bias_seed"], integer=integer)
    return dict(name=name, M=w["M"], N=w["N"], K=w["K"], A=A, B=B, bias=bias,
                c_dtype=w["c_dtype"], integer=integer, op_a=op_a, op_b=op_b,
                lda=A.shape[1], ldb=B.shape[1])


# Fused-attention workloads: Q, K, V with N(0,1) values rounded to fp16, one
# stream each (seeds seed, seed + 1, seed + 2), stored [B, H, L, d] dense.
ATTN_WORKLOADS = {
    "attn_b2h16l4096d128": dict(B=2, H=16, Hkv=16, Lq=4096, Lk=4096, d=128, causal=False,
                                seed=10),
    "attn_b2h16l4096d128_causal": dict(B=2, H=16, Hkv=16, Lq=4096, Lk=4096, d=128, causal=True,
                                       seed=10),
    "attn_b4h16l2048d64": dict(B=4, H=16, Hkv=16, Lq=2048, Lk=2048, d=64, causal=False,
                               seed=13),
}


def attention_workload(name):
    """fp16 bits of Q [B, H, Lq, d], K and V [B, Hkv, Lk, d] of a named
    attention workload, with the {batch, head, row} strides."""
    w = dict(ATTN_WORKLOADS[name])
    B, H, Hkv, Lq, Lk, d = w["B"], w["H"], w["Hkv"], w["Lq"], w["Lk"], w["d"]
    Q = to_f16_bits(normal(w["seed"], B * H * Lq * d))
    K = to_f16_bits(normal(w["seed"] + 1, B * Hkv * Lk * d))
    V = to_f16_bits(normal(w["seed"] + 2, B * Hkv * Lk * d))
    w.update(name=name, Q=Q, K=K, V=V, qs=(H * Lq * d, Lq * d, d), ks=(Hkv * Lk * d, Lk * d, d),
             vs=(Hkv * Lk * d, Lk * d, d), os=(H * Lq * d, Lq * d, d))
    return w

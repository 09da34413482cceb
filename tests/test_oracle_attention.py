"""Pins of the attention oracle (oracle/tgref_attention.c) against closed
forms and invariants of softmax attention, none of which re-types its
formula:

* Q = 0 (or scale = 0): uniform weights, O = mean of the visible V rows,
  lse = log(number of visible keys);
* one key: O = V[0], lse = the one score;
* two keys: the weights are the logistic function of the score difference;
* a dominant key (score gap > 60): O = that key's V row;
* causal, Lq == Lk: row i equals the unmasked result over keys 0..i, and
  row 0 is V[0]; Lq > Lk: the first Lq - Lk rows see nothing (O = 0,
  lse = -inf);
* adding the same vector w to every key shifts every score of row i by
  scale * q_i . w: O unchanged, lse + scale * q_i . w;
* V -> a V + b gives O -> a O + b; permuting keys (unmasked) changes nothing;
* grouped K/V heads equal the same heads repeated; the {batch, head, row}
  strides of two layouts give the same result;
* A (the weighted mean |V|) equals O for non-negative V.
Values are small integers or fp16-exact so that the inputs the invariants
build are exact in fp16."""
import math

import numpy as np
import pytest

import oracle
import tg_inputs as gen


def f16(x):
    return np.asarray(x, np.float64).astype(np.float16).view(np.uint16)


def dense(B, H, L, d):
    """{batch, head, row} strides of a dense [B, H, L, d] array."""
    return (H * L * d, L * d, d)


def run(Q, K, V, B, H, Hkv, Lq, Lk, d, scale=None, causal=False):
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    return oracle.attention_ref(f16(Q), f16(K), f16(V), B, H, Hkv, Lq, Lk, d,
                                dense(B, H, Lq, d), dense(B, Hkv, Lk, d), dense(B, Hkv, Lk, d),
                                scale, causal)


def ints(seed, shape, lo=-4, hi=4):
    return np.random.default_rng(seed).integers(lo, hi + 1, size=shape).astype(np.float64)


def test_zero_queries_give_the_mean_of_v():
    B, H, Lq, Lk, d = 2, 3, 5, 7, 8
    Q = np.zeros((B, H, Lq, d))
    K = ints(1, (B, H, Lk, d))
    V = ints(2, (B, H, Lk, d))
    O, lse, A = run(Q, K, V, B, H, H, Lq, Lk, d)
    want = V.mean(axis=2)[:, :, None, :]
    assert np.allclose(O, np.broadcast_to(want, O.shape), rtol=0, atol=1e-14)
    assert np.allclose(lse, math.log(Lk), rtol=0, atol=1e-14)
    assert np.allclose(A, np.broadcast_to(np.abs(V).mean(axis=2)[:, :, None, :], A.shape),
                       rtol=0, atol=1e-14)
    # scale 0 is the same as zero queries
    O0, lse0, _ = run(ints(3, (B, H, Lq, d)), K, V, B, H, H, Lq, Lk, d, scale=0.0)
    assert np.array_equal(O0, O) and np.array_equal(lse0, lse)


def test_causal_zero_queries_average_the_visible_prefix():
    B, H, L, d = 1, 2, 6, 4
    V = ints(4, (B, H, L, d))
    O, lse, _ = run(np.zeros((B, H, L, d)), ints(5, (B, H, L, d)), V, B, H, H, L, L, d,
                    causal=True)
    for i in range(L):
        assert np.allclose(O[:, :, i], V[:, :, :i + 1].mean(axis=2), rtol=0, atol=1e-14)
        assert lse[0, 0, i] == pytest.approx(math.log(i + 1), abs=1e-14)


def test_single_key():
    B, H, Lq, d = 1, 2, 3, 16
    Q, K, V = ints(6, (B, H, Lq, d)), ints(7, (B, H, 1, d)), ints(8, (B, H, 1, d))
    O, lse, _ = run(Q, K, V, B, H, H, Lq, 1, d, scale=0.25)
    assert np.array_equal(O, np.broadcast_to(V, O.shape))
    want = 0.25 * np.einsum("bhic,bhc->bhi", Q, K[:, :, 0])
    assert np.allclose(lse, want, rtol=0, atol=1e-13)


def test_two_keys_follow_the_logistic_function():
    d = 4
    Q = np.array([[[[1, 0, 2, 0], [0, 0, 0, 1]]]], np.float64)     # B=H=1, Lq=2
    K = np.array([[[[1, 1, 0, 0], [0, 2, 1, 3]]]], np.float64)
    V = np.array([[[[1, 2, 3, 4], [-5, 6, -7, 8]]]], np.float64)
    O, lse, _ = run(Q, K, V, 1, 1, 1, 2, 2, d, scale=0.5)
    for i in range(2):
        s0, s1 = 0.5 * Q[0, 0, i] @ K[0, 0, 0], 0.5 * Q[0, 0, i] @ K[0, 0, 1]
        w1 = 1.0 / (1.0 + math.exp(s0 - s1))
        want = (1 - w1) * V[0, 0, 0] + w1 * V[0, 0, 1]
        assert np.allclose(O[0, 0, i], want, rtol=0, atol=1e-14)
        assert lse[0, 0, i] == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))),
                                             abs=1e-14)


def test_dominant_key_selects_its_value_row():
    B, H, Lk, d = 1, 1, 9, 8
    K = np.zeros((B, H, Lk, d))
    for j in range(Lk):
        K[0, 0, j, j % d] = 1.0
    K[0, 0, 5] = 0
    K[0, 0, 5, 3] = 8.0
    Q = np.zeros((B, H, 1, d))
    Q[0, 0, 0, 3] = 8.0                   # scores 64 for key 5, <= 8 otherwise
    V = ints(9, (B, H, Lk, d))
    O, lse, _ = run(Q, K, V, B, H, H, 1, Lk, d, scale=1.0)
    assert np.allclose(O[0, 0, 0], V[0, 0, 5], rtol=0, atol=1e-20)
    assert lse[0, 0, 0] == pytest.approx(64.0, abs=1e-20)


def test_causal_rows_equal_unmasked_prefixes():
    B, H, L, d = 2, 2, 9, 16
    Q, K, V = (gen.normal(s, B * H * L * d).reshape(B, H, L, d) for s in (11, 12, 13))
    Q, K, V = (np.asarray(f16(x)).view(np.float16).astype(np.float64) for x in (Q, K, V))
    O, lse, _ = run(Q, K, V, B, H, H, L, L, d, causal=True)
    assert np.array_equal(O[:, :, 0], V[:, :, 0])
    for i in range(L):
        Oi, lsei, _ = run(Q[:, :, i:i + 1], K[:, :, :i + 1], V[:, :, :i + 1], B, H, H, 1, i + 1, d)
        assert np.allclose(O[:, :, i], Oi[:, :, 0], rtol=0, atol=1e-14)
        assert np.allclose(lse[:, :, i], lsei[:, :, 0], rtol=0, atol=1e-14)


def test_causal_with_more_queries_than_keys():
    B, H, Lq, Lk, d = 1, 1, 6, 4, 8
    Q, K, V = ints(14, (B, H, Lq, d)), ints(15, (B, H, Lk, d)), ints(16, (B, H, Lk, d))
    O, lse, A = run(Q, K, V, B, H, H, Lq, Lk, d, causal=True)
    # the mask ends at the bottom right: query i sees keys j <= i - 2
    assert np.all(O[0, 0, :2] == 0) and np.all(np.isneginf(lse[0, 0, :2]))
    assert np.all(A[0, 0, :2] == 0)
    assert np.array_equal(O[0, 0, 2], V[0, 0, 0])
    full, lse_full, _ = run(Q, K, V, B, H, H, Lq, Lk, d)
    assert np.array_equal(O[0, 0, -1], full[0, 0, -1])
    assert lse[0, 0, -1] == lse_full[0, 0, -1]
    # fewer queries than keys: the first query already sees Lk - Lq + 1 keys
    O2, _, _ = run(Q[:, :, :2], K, V, B, H, H, 2, Lk, d, causal=True)
    sub, _, _ = run(Q[:, :, :1], K[:, :, :3], V[:, :, :3], B, H, H, 1, 3, d)
    assert np.allclose(O2[0, 0, 0], sub[0, 0, 0], rtol=0, atol=1e-14)


def test_shifting_every_key_by_a_vector():
    B, H, Lq, Lk, d = 1, 2, 4, 6, 8
    Q, K, V = ints(17, (B, H, Lq, d)), ints(18, (B, H, Lk, d)), ints(19, (B, H, Lk, d))
    w = ints(20, (d,), -2, 2)
    scale = 0.125
    O, lse, _ = run(Q, K, V, B, H, H, Lq, Lk, d, scale=scale)
    O2, lse2, _ = run(Q, K + w, V, B, H, H, Lq, Lk, d, scale=scale)
    assert np.allclose(O2, O, rtol=0, atol=1e-12)
    assert np.allclose(lse2, lse + scale * (Q @ w), rtol=0, atol=1e-12)


def test_affine_map_of_v_and_key_permutation():
    B, H, Lq, Lk, d = 1, 1, 5, 7, 8
    Q, K, V = ints(21, (B, H, Lq, d)), ints(22, (B, H, Lk, d)), ints(23, (B, H, Lk, d))
    O, lse, _ = run(Q, K, V, B, H, H, Lq, Lk, d, scale=0.3)
    O2, lse2, _ = run(Q, K, 2 * V + 1, B, H, H, Lq, Lk, d, scale=0.3)
    assert np.allclose(O2, 2 * O + 1, rtol=0, atol=1e-12)
    assert np.array_equal(lse2, lse)
    perm = np.random.default_rng(0).permutation(Lk)
    O3, lse3, _ = run(Q, K[:, :, perm], V[:, :, perm], B, H, H, Lq, Lk, d, scale=0.3)
    assert np.allclose(O3, O, rtol=0, atol=1e-12)
    assert np.allclose(lse3, lse, rtol=0, atol=1e-12)


def test_weighted_magnitude():
    B, H, Lq, Lk, d = 1, 1, 3, 5, 8
    Q, K = ints(24, (B, H, Lq, d)), ints(25, (B, H, Lk, d))
    V = ints(26, (B, H, Lk, d), 0, 4)
    O, _, A = run(Q, K, V, B, H, H, Lq, Lk, d, scale=0.2)
    assert np.allclose(A, O, rtol=0, atol=1e-13)
    _, _, A2 = run(Q, K, -V, B, H, H, Lq, Lk, d, scale=0.2)
    assert np.allclose(A2, A, rtol=0, atol=1e-13)


def test_grouped_heads_equal_repeated_heads():
    B, H, Hkv, Lq, Lk, d = 2, 4, 2, 3, 5, 8
    Q, K, V = ints(27, (B, H, Lq, d)), ints(28, (B, Hkv, Lk, d)), ints(29, (B, Hkv, Lk, d))
    O, lse, _ = run(Q, K, V, B, H, Hkv, Lq, Lk, d, causal=True)
    Kr, Vr = np.repeat(K, H // Hkv, axis=1), np.repeat(V, H // Hkv, axis=1)
    O2, lse2, _ = run(Q, Kr, Vr, B, H, H, Lq, Lk, d, causal=True)
    assert np.array_equal(O, O2) and np.array_equal(lse, lse2)


def test_strided_layouts_agree():
    """[B, H, L, d] and [B, L, H, d] storage of the same tensors."""
    B, H, L, d = 2, 3, 4, 8
    Q, K, V = ints(30, (B, H, L, d)), ints(31, (B, H, L, d)), ints(32, (B, H, L, d))
    O, lse, _ = run(Q, K, V, B, H, H, L, L, d, causal=True)
    blhd = [f16(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (Q, K, V)]
    st = (L * H * d, d, H * d)
    O2, lse2, _ = oracle.attention_ref(*blhd, B, H, H, L, L, d, st, st, st, 1 / math.sqrt(d),
                                       True)
    assert np.array_equal(O, O2) and np.array_equal(lse, lse2)


def test_selected_rows_match_the_full_computation():
    B, H, Hkv, Lq, Lk, d = 2, 4, 2, 7, 9, 16
    Q, K, V = ints(33, (B, H, Lq, d)), ints(34, (B, Hkv, Lk, d)), ints(35, (B, Hkv, Lk, d))
    O, lse, A = run(Q, K, V, B, H, Hkv, Lq, Lk, d, causal=True)
    rows = [(1, 3, 6), (0, 0, 0), (1, 2, 4), (0, 1, 2)]
    Or, lr, Ar = oracle.attention_rows(f16(Q), f16(K), f16(V), B, H, Hkv, Lq, Lk, d,
                                       dense(B, H, Lq, d), dense(B, Hkv, Lk, d),
                                       dense(B, Hkv, Lk, d), 1 / math.sqrt(d), True, rows)
    for r, (b, h, i) in enumerate(rows):
        assert np.array_equal(Or[r], O[b, h, i]) and lr[r] == lse[b, h, i]
        assert np.array_equal(Ar[r], A[b, h, i])
    with pytest.raises(ValueError):
        oracle.attention_rows(f16(Q), f16(K), f16(V), B, H, Hkv, Lq, Lk, d, dense(B, H, Lq, d),
                              dense(B, Hkv, Lk, d), dense(B, Hkv, Lk, d), 1.0, True, [(2, 0, 0)])


def test_invalid_sizes_rejected():
    z = np.zeros(64, np.uint16)
    st = (0, 0, 0)
    with pytest.raises(ValueError):
        oracle.attention_ref(z, z, z, 1, 3, 2, 1, 1, 4, st, st, st, 1.0)   # H % Hkv != 0
    with pytest.raises(ValueError):
        oracle.attention_ref(z, z, z, 1, 1, 1, 1, 1, 0, st, st, st, 1.0)   # d = 0


def test_large_scores_stay_finite():
    """Scores near 1000 (exp would overflow double without the row maximum
    taken out first)."""
    B, H, Lq, Lk, d = 1, 1, 2, 3, 4
    Q = np.array([[[[30, 0, 0, 0], [0, 30, 0, 0]]]], np.float64)
    K = np.array([[[[32, 0, 0, 0], [31, 1, 0, 0], [0, 33, 0, 0]]]], np.float64)
    V = ints(36, (B, H, Lk, d))
    O, lse, _ = run(Q, K, V, B, H, H, Lq, Lk, d, scale=1.0)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(lse))
    # row 0: scores 960, 930, 0 -> key 0 (weight 1 - e^-30); row 1: 0, 30, 990 -> key 2
    assert np.allclose(O[0, 0, 0], V[0, 0, 0], rtol=0, atol=1e-11)
    assert np.allclose(O[0, 0, 1], V[0, 0, 2], rtol=0, atol=1e-11)
    assert lse[0, 0, 0] == pytest.approx(960 + math.log1p(math.exp(-30)), abs=1e-10)

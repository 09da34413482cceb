"""Pins for the seeded input generator."""
import numpy as np

import tg_inputs as gen


def _sequential_splitmix(seed, n):
    out, s = [], seed
    for _ in range(n):
        s = (s + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
        z = s
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        out.append(z ^ (z >> 31))
    return out


def test_splitmix64_published_vectors():
    # first outputs of the reference SplitMix64 with state 0
    assert [int(x) for x in gen.splitmix64(0, 3)] == [
        0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_splitmix64_matches_sequential_and_offsets():
    for seed in (0, 1, 5, 2 ** 63 + 11):
        want = _sequential_splitmix(seed, 50)
        assert [int(x) for x in gen.splitmix64(seed, 50)] == want
        assert [int(x) for x in gen.splitmix64(seed, 20, start=30)] == want[30:]


def test_distributions():
    u = gen.uniform_pm1(3, 200000)
    assert u.min() >= -1 and u.max() < 1 and abs(u.mean()) < 0.01
    z = gen.normal(4, 200001)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert np.array_equal(gen.normal(4, 10, start=7), z[7:17])
    i = gen.ints_pm4(5, 90000)
    assert set(np.unique(i)) == set(range(-4, 5))
    assert np.all(np.abs(np.bincount((i + 4).astype(int)) - 10000) < 500)


def test_workload_shapes_and_streams():
    w = gen.workload("sq256")
    assert w["A"].shape == (256, 256) and w["B"].shape == (256, 256)
    A2, B2 = gen.operands(256, 256, 256, "uniform", 0)
    assert np.array_equal(w["A"], A2) and np.array_equal(w["B"], B2)
    # B continues the stream after A
    flat = gen.to_f16_bits(gen.uniform_pm1(0, 2 * 256 * 256))
    assert np.array_equal(flat[256 * 256:], w["B"].reshape(-1))
    wi = gen.workload("sq256", integer=True)
    vals = wi["A"].view(np.float16).astype(np.float64)
    assert np.all(vals == np.round(vals)) and vals.min() >= -4 and vals.max() <= 4

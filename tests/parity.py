"""Comparison rules between the HIP path's output and the CPU oracle.

* integer inputs ({-4..4}, integer bias): bit-exact against the oracle's
  output-typed value (+0 and -0 compare equal); every product and partial sum
  is an integer below 2^24, exact in fp32 in any order, so both sides round the
  same exact value once.
* otherwise, element-wise |C_gpu - C_ref| <= 1e-3 * sqrt(K), plus one fp16 ulp
  of |C_ref| when C is fp16, with C_ref the unrounded fp64 oracle value.
"""
import numpy as np

import oracle


def ulp16(x):
    """Spacing of fp16 values at |x|: 2^(floor(log2|x|) - 10), or 2^-24 below 2^-14."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return np.where(a < 2.0 ** -14, 2.0 ** -24, 2.0 ** (e - 10))


def tolerance(cref, K, c_dtype):
    tol = 1e-3 * np.sqrt(max(K, 0)) * np.ones_like(cref)
    if c_dtype == "f16":
        tol = tol + ulp16(cref)
    return tol


def gpu_values(c, c_dtype):
    """GPU output array -> float64 values."""
    c = np.asarray(c)
    if c_dtype == "f16":
        return c.view(np.float16).astype(np.float64) if c.dtype == np.uint16 else c.astype(np.float64)
    return c.astype(np.float64)


def check(c_gpu, cref, K, c_dtype, integer, what=""):
    """Assert the parity rule; returns a small report dict."""
    c_gpu = np.asarray(c_gpu)
    cref = np.asarray(cref, np.float64)
    assert c_gpu.shape == cref.shape, (c_gpu.shape, cref.shape)
    vals = gpu_values(c_gpu, c_dtype)
    assert not np.any(np.isnan(vals)), what + ": NaN in GPU output"
    err = np.abs(vals - cref)
    rep = {"max_abs_err": float(err.max()) if err.size else 0.0, "n": int(err.size)}
    if integer:
        want = oracle.output_typed(cref, c_dtype)
        if c_dtype == "f16":
            got = c_gpu.view(np.uint16) if c_gpu.dtype != np.uint16 else c_gpu
            got = np.where(got == 0x8000, 0, got)
            want = np.where(want == 0x8000, 0, want)
            bad = got != want
        else:
            bad = vals != want.astype(np.float64)
        nbad = int(bad.sum())
        if nbad:
            idx = np.argwhere(bad)[:5]
            raise AssertionError("%s: %d integer-input mismatches, first at %s: gpu %s ref %s"
                                 % (what, nbad, idx.tolist(), vals[tuple(idx[0])],
                                    cref[tuple(idx[0])]))
        rep["bit_exact"] = True
        return rep
    tol = tolerance(cref, K, c_dtype)
    bad = err > tol
    nbad = int(bad.sum())
    if nbad:
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d elements outside tolerance, first at %s: gpu %r ref %r tol %r"
                             % (what, nbad, idx.tolist(), vals[tuple(idx[0])],
                                cref[tuple(idx[0])], tol[tuple(idx[0])]))
    rep["allclose_1e-2"] = bool(np.all(err <= 1e-2 + 1e-2 * np.abs(cref)))
    if c_dtype == "f16":
        rep["max_err_ulp16"] = float((err / ulp16(cref)).max()) if err.size else 0.0
    return rep

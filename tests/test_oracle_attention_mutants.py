"""The attention oracle's pins must catch plausible mistakes: each case plants
one mistake in a copy of oracle/tgref_attention.c (on the CPU, in a temp
dir), builds it with the unchanged fp16 codec, loads it in place of the real
oracle and checks that at least one pin fails."""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_attention as pins

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "tgref_attention.c")
CODEC = os.path.join(HERE, "tgref.c")

MUTANTS = {
    "scale_dropped": ("s[j] = J->scale * acc;", "s[j] = acc;"),
    "max_not_subtracted": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j]);"),
    "causal_off_by_one": ("int64_t n = i + (J->Lk - J->Lq) + 1;",
                          "int64_t n = i + (J->Lk - J->Lq);"),
    "causal_top_left": ("int64_t n = i + (J->Lk - J->Lq) + 1;", "int64_t n = i + 1;"),
    "grouped_heads_interleaved": ("const int64_t hk = h / (J->H / J->Hkv);",
                                  "const int64_t hk = h % J->Hkv;"),
    "values_read_from_keys": ("const uint16_t *vrow = vbase + j * J->vs[2];",
                              "const uint16_t *vrow = kbase + j * J->ks[2];"),
    "not_normalised": ("out_O[c] /= l;", "out_O[c] /= 1.0;"),
    "lse_without_max": ("*out_lse = m + log(l);", "*out_lse = log(l);"),
    "key_row_stride_ignored": ("const uint16_t *krow = kbase + j * J->ks[2];",
                               "const uint16_t *krow = kbase + j * J->d;"),
    "magnitude_signed": ("out_A[c] += s[j] * fabs(v);", "out_A[c] += s[j] * v;"),
    "last_key_dropped": ("for (int64_t j = 0; j < n; j++) {\n        const uint16_t *krow",
                         "for (int64_t j = 0; j + 1 < n; j++) {\n        const uint16_t *krow"),
}


def _pins():
    return [getattr(pins, n) for n in dir(pins) if n.startswith("test_")]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site not found: " + name
    c = tmp_path / "attn_mut.c"
    so = tmp_path / "libtgref_attn_mut.so"
    c.write_text(src.replace(old, new))
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
                    "-ffp-contract=off", "-o", str(so), CODEC, str(c), "-lm"], check=True)
    real = oracle.lib()
    mut = ctypes.CDLL(str(so))
    for fn in ("tgref_attention", "tgref_attention_rows"):
        getattr(mut, fn).argtypes = getattr(real, fn).argtypes
        getattr(mut, fn).restype = getattr(real, fn).restype

    class Proxy:
        def __getattr__(self, fn):
            return getattr(mut if fn.startswith("tgref_attention") else real, fn)

    caught = []
    saved = oracle._lib
    oracle._lib = Proxy()
    try:
        for pin in _pins():
            try:
                pin()
            except (AssertionError, ValueError):
                caught.append(pin.__name__)
    finally:
        oracle._lib = saved
    assert caught, "no pin caught mutant " + name

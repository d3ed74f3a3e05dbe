"""Plant plausible mistakes in copies of the oracle and check that the pins catch each.

Each mutant is a copy of oracle/ref_attn.c with one textual change, built with
gcc into a temporary directory.  The test passes only if at least one pin in
``oracle_pins.ALL_PINS`` fails on every mutant, which shows that the pins are
sharp enough to reject a dropped term, a wrong sign, an off-by-one in the mask,
a transposed operand or a wrong GQA index.  CPU only.
"""
import os

import pytest

import oracle_pins
from oracle import Oracle
from oracle import build as oracle_build

MUTANTS = {
    "scale dropped from scores": [("      s *= scale;\n", "")],
    "no max subtraction": [("Pi[j] = exp(Pi[j] - m);", "Pi[j] = exp(Pi[j]);"),
                           ("lse[i] = m + log(l);", "lse[i] = log(l);")],
    "mask hides the diagonal in P.V": [("for (int j = 0; j <= i; ++j) acc += Pi[j] * v",
                                        "for (int j = 0; j < i; ++j) acc += Pi[j] * v")],
    "rows not normalised": [("for (int j = 0; j <= i; ++j) Pi[j] /= l;", "")],
    "LSE in log2": [("lse[i] = m + log(l);", "lse[i] = m + log2(l);")],
    "O reads K instead of V": [("acc += Pi[j] * v[(size_t)j * hd + d];", "acc += Pi[j] * k[(size_t)j * hd + d];")],
    "dS sign flipped": [("dSi[j] = Pi[j] * (dPi[j] - rd);", "dSi[j] = Pi[j] * (dPi[j] + rd);")],
    "dS row term dropped": [("dSi[j] = Pi[j] * (dPi[j] - rd);", "dSi[j] = Pi[j] * dPi[j];")],
    "dP reads K instead of V": [("acc += dO[(size_t)i * hd + d] * v[(size_t)j * hd + d];",
                                 "acc += dO[(size_t)i * hd + d] * k[(size_t)j * hd + d];")],
    "dQ scale dropped": [("dq[(size_t)i * hd + d] = scale * acc;", "dq[(size_t)i * hd + d] = acc;")],
    "dK scale dropped": [("dk[(size_t)j * hd + d] = scale * acc;", "dk[(size_t)j * hd + d] = acc;")],
    "dK transposed dS": [("acc += dS[(size_t)i * S + j] * q[(size_t)i * hd + d];",
                          "acc += dS[(size_t)j * S + i] * q[(size_t)i * hd + d];")],
    "dK skips the diagonal": [("for (int i = j; i < S; ++i) acc += dS[", "for (int i = j + 1; i < S; ++i) acc += dS[")],
    "dV uses dS instead of P": [("acc += P[(size_t)i * S + j] * dO[(size_t)i * hd + d];",
                                 "acc += dS[(size_t)i * S + j] * dO[(size_t)i * hd + d];")],
    "dQ sums past the diagonal": [("for (int j = 0; j <= i; ++j) acc += dS[(size_t)i * S + j] * k",
                                   "for (int j = 0; j <= i && j + 1 < S; ++j) acc += dS[(size_t)i * S + j + 1] * k")],
    "GQA kv head interleaved (h mod Hkv)": [("memcpy(dst + (size_t)(kvh * group + r) * head",
                                             "memcpy(dst + (size_t)(r * Hkv + kvh) * head")],
    "group sum keeps only r = 0": [("for (int r = 0; r < group; ++r) acc += dk_rep",
                                    "for (int r = 0; r < 1; ++r) acc += dk_rep"),
                                   ("for (int r = 0; r < group; ++r) acc += dv_rep",
                                    "for (int r = 0; r < 1; ++r) acc += dv_rep")],
}


@pytest.fixture(scope="module")
def source():
    with open(oracle_build.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source, tmp_path):
    src = source
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, f"mutation anchor not unique in ref_attn.c: {old!r}"
        src = src.replace(old, new)
    path = tmp_path / "mutant.c"
    path.write_text(src)
    lib = oracle_build.build(str(path), str(tmp_path / "libmutant.so"))
    mutant = Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception:  # AssertionError, or the mutant's NaNs tripping a check
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the mutant {name!r}"
    print(f"{name}: caught by {', '.join(caught)}")


def test_real_oracle_builds_from_unmodified_source(source):
    assert os.path.exists(oracle_build.SRC) and "xattn_ref_run" in source

"""The decode-attention oracle against its pins, and planted mistakes against
the pins (each mutant is a copy of oracle/ref_decode.c with one textual change,
built with gcc into a temporary directory; at least one pin must fail on each).
CPU only."""
import pytest

import decode_pins
from oracle import DecodeOracle, default_decode
from oracle import build as oracle_build


@pytest.mark.parametrize("pin", decode_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(default_decode())


# (old, new, which occurrence) -- occurrence 0 is the first in the file
MUTANTS = {
    "scale dropped": [("s *= scale;", "", 0)],
    "scale applied twice": [("exp(scale * s - m)", "exp(scale * scale * s - m)", 0)],
    "no max subtraction": [("exp(scale * s - m)", "exp(scale * s)", 0),
                           ("= m + log(l);", "= log(l);", 0)],
    "lse drops the max": [("= m + log(l);", "= log(l);", 0)],
    "weights not normalised": [("for (int d = 0; d < hd; ++d) oh[d] /= l;", "", 0)],
    "values read from K": [("oh[d] += p * vg[", "oh[d] += p * kg[", 0)],
    "reads one past the length": [("for (int j = 0; j < n; ++j) {", "for (int j = 0; j <= n && j < T; ++j) {", 0),
                                  ("for (int j = 0; j < n; ++j) {", "for (int j = 0; j <= n && j < T; ++j) {", 0)],
    "last position skipped": [("for (int j = 0; j < n; ++j) {", "for (int j = 0; j + 1 < n; ++j) {", 0),
                              ("for (int j = 0; j < n; ++j) {", "for (int j = 0; j + 1 < n; ++j) {", 0)],
    "kv head interleaved (h mod Hkv)": [("const int g = h / group;", "const int g = h % Hkv;", 0)],
    "empty sequence not special-cased": [("if (n == 0) {", "if (0) {", 0)],
    "length ignored": [("const int n = len ? len[b] : T;", "const int n = T;", 1)],
}


def _nth(src, old, n):
    i = -1
    for _ in range(n + 1):
        i = src.index(old, i + 1)
    return i


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    with open(oracle_build.SRC_DEC) as f:
        src = f.read()
    for old, new, n in MUTANTS[name]:
        i = _nth(src, old, n)  # counted in the text as edited so far
        src = src[:i] + new + src[i + len(old):]
    path = tmp_path / "mutant.c"
    path.write_text(src)
    lib = oracle_build.build(str(path), str(tmp_path / "libmutant_decode.so"))
    o = DecodeOracle(lib)
    caught = []
    for pin in decode_pins.ALL_PINS:
        try:
            pin(o)
        except Exception as e:  # AssertionError, or the mutant's NaNs/errors tripping a check
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"mutant '{name}' passed every pin"

"""The QK-norm + RoPE oracle against its pins, and planted mistakes against the
pins (each mutant is a copy of oracle/ref_qknorm_rope.c with one textual change,
built with gcc into a temporary directory; at least one pin must fail on each).
CPU only."""
import pytest

import norm_pins
from oracle import NormOracle, default_norm
from oracle import build as oracle_build


@pytest.mark.parametrize("pin", norm_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(default_norm())


# (old, new, which occurrence) -- occurrence 0 is the first in the file
MUTANTS = {
    "rotation sign flipped": [("o[i] = y1 * cos(th) - y2 * sin(th);", "o[i] = y1 * cos(th) + y2 * sin(th);", 0)],
    "eps dropped": [("const double r = sqrt(ss / hd + eps);", "const double r = sqrt(ss / hd);", 0)],
    "sum instead of mean": [("const double r = sqrt(ss / hd + eps);", "const double r = sqrt(ss + eps);", 0)],
    "frequency exponent halved": [("pow(base, -2.0 * (double)i / (double)hd)", "pow(base, -1.0 * (double)i / (double)hd)", 0)],
    "weight ignored": [("const double y1 = w[i] * (x[i] / r), y2 = w[i + half] * (x[i + half] / r);",
                        "const double y1 = (x[i] / r), y2 = (x[i + half] / r);", 0)],
    "interleaved pairing": [("const double y1 = w[i] * (x[i] / r), y2 = w[i + half] * (x[i + half] / r);",
                             "const double y1 = w[2 * i] * (x[2 * i] / r), y2 = w[2 * i + 1] * (x[2 * i + 1] / r);", 0)],
    "position off by one": [("const double th = angle(s, i, hd, base);", "const double th = angle(s + 1, i, hd, base);", 0)],
    "token-major output": [("double* o = Out + (((size_t)b * H + h) * S + s) * hd;",
                            "double* o = Out + (((size_t)b * S + s) * H + h) * hd;", 0)],
    "backward rotation not transposed": [("gy[i] = G[i] * cos(th) + G[i + half] * sin(th);",
                                          "gy[i] = G[i] * cos(th) - G[i + half] * sin(th);", 0),
                                         ("gy[i + half] = -G[i] * sin(th) + G[i + half] * cos(th);",
                                          "gy[i + half] = G[i] * sin(th) + G[i + half] * cos(th);", 0)],
    "Jacobian sign": [("- x[d] * x[k] / (hd * r * r * r)", "+ x[d] * x[k] / (hd * r * r * r)", 0)],
    "Jacobian missing 1/hd": [("- x[d] * x[k] / (hd * r * r * r)", "- x[d] * x[k] / (r * r * r)", 0)],
    "dx ignores the weight": [("for (int d = 0; d < hd; ++d) gxh[d] = w[d] * gy[d];",
                               "for (int d = 0; d < hd; ++d) gxh[d] = gy[d];", 0)],
    "dw from the weighted output": [("dw[d] += (x[d] / r) * gy[d];", "dw[d] += w[d] * (x[d] / r) * gy[d];", 0)],
    "dw from the unnormalised input": [("dw[d] += (x[d] / r) * gy[d];", "dw[d] += x[d] * gy[d];", 0)],
}


def _nth(src, old, n):
    i = -1
    for _ in range(n + 1):
        i = src.index(old, i + 1)
    return i


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    with open(oracle_build.SRC_NORM) as f:
        src = f.read()
    for old, new, n in MUTANTS[name]:
        i = _nth(src, old, n)
        src = src[:i] + new + src[i + len(old):]
    path = tmp_path / "mutant.c"
    path.write_text(src)
    lib = oracle_build.build(str(path), str(tmp_path / "libmutant_norm.so"))
    o = NormOracle(lib)
    caught = []
    for pin in norm_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError as e:
            caught.append(f"{pin.__name__}: {e}")
    assert caught, f"mutant '{name}' passed every pin"

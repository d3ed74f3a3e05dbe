"""The right-padded-batch oracle against its pins, and planted mistakes in it
(subclasses of the oracle with one change each) against the pins.  CPU only."""
import numpy as np
import pytest

import ragged_pins
from oracle import Oracle, default


@pytest.mark.parametrize("pin", ragged_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(default())


class _Shorter(Oracle):  # each sequence loses its last row
    def run_ragged(self, q, k, v, lens, dO=None, scale=None, backward=True):
        return super().run_ragged(q, k, v, [max(0, n - 1) for n in lens], dO, scale, backward)


class _PadZeroLse(Oracle):  # padding rows get lse = 0
    def run_ragged(self, *a, **kw):
        r = super().run_ragged(*a, **kw)
        r["lse"][np.isneginf(r["lse"])] = 0.0
        return r


class _Unmasked(Oracle):  # ignores the lengths: plain run over the padding
    def run_ragged(self, q, k, v, lens, dO=None, scale=None, backward=True):
        return self.run(q, k, v, dO, scale=scale, backward=backward)


class _OffByOneRows(Oracle):  # rows shifted: prefix of length n+1 written to n rows
    def run_ragged(self, q, k, v, lens, dO=None, scale=None, backward=True):
        S = np.asarray(q).shape[2]
        r = super().run_ragged(q, k, v, [min(S, n + 1) if 0 < n < S else n for n in lens], dO,
                               scale, backward)
        return r


@pytest.mark.parametrize("cls", [_Shorter, _PadZeroLse, _Unmasked, _OffByOneRows],
                         ids=lambda c: c.__name__)
def test_mutant_is_caught(cls):
    m = cls()
    caught = []
    for pin in ragged_pins.ALL_PINS:
        try:
            pin(m)
        except Exception as e:
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"mutant {cls.__name__} passed every pin"

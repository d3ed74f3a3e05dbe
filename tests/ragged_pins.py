"""Pins for the oracle of right-padded batches (``Oracle.run_ragged``).

``run_ragged`` composes the causal-attention oracle over each sequence's
prefix.  These pins check it against what the pages fix about right padding
("xtrain evolution overview", post-training stage, milestone M2d): under the
causal mask a real row never sees a later (padding) position, so

* the real rows of a plain causal run over the padded batch (any finite
  padding) equal the ragged result, for o and lse;
* with the loss masked on the padding rows (their upstream gradient zero), the
  padded run's dq, dk and dv on real rows equal the ragged result too;
* padding rows come back as o = 0, lse = -inf and zero gradients, padding
  inputs (NaN here) are never read, and a batch with every length S is the
  plain run.
Every pin raises ``AssertionError`` on a mismatch.
"""
import numpy as np

B, S, H, Hkv, hd = 4, 11, 4, 2, 8
LENS = [11, 6, 1, 0]


def _inputs(seed, pad):
    r = np.random.default_rng(seed)
    q, k, v, dO = (r.standard_normal((B, h, S, hd)) for h in (H, Hkv, Hkv, H))
    for b, n in enumerate(LENS):
        for x in (q, k, v, dO):
            x[b, :, n:] = pad
    return q, k, v, dO


def _close(a, b, tol, what):
    a, b = np.asarray(a), np.asarray(b)
    assert np.all(np.isfinite(a)) and np.all(np.isfinite(b)), f"{what}: non-finite"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    den = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= tol * den, f"{what}: max|err| {err:.3e} > {tol:g} * {den:.3e}"


def pin_real_rows_equal_padded_forward(o):
    q, k, v, dO = _inputs(1, pad=3.0)
    rag = o.run_ragged(q, k, v, LENS, backward=False)
    pad = o.run(q, k, v, backward=False)
    for b, n in enumerate(LENS):
        _close(rag["o"][b, :, :n], pad["o"][b, :, :n], 1e-13, f"o, length {n}")
        _close(rag["lse"][b, :, :n], pad["lse"][b, :, :n], 1e-13, f"lse, length {n}")


def pin_masked_padded_backward(o):
    q, k, v, dO = _inputs(2, pad=-2.0)
    for b, n in enumerate(LENS):
        dO[b, :, n:] = 0.0  # the loss is masked on padding rows
    rag = o.run_ragged(q, k, v, LENS, dO)
    pad = o.run(q, k, v, dO)
    for b, n in enumerate(LENS):
        for name in ("dq", "dk", "dv"):
            _close(rag[name][b, :, :n], pad[name][b, :, :n], 1e-12, f"{name}, length {n}")


def pin_padding_outputs_and_nan_inputs(o):
    q, k, v, dO = _inputs(3, pad=np.nan)
    r = o.run_ragged(q, k, v, LENS, dO)
    for b, n in enumerate(LENS):
        assert np.all(r["o"][b, :, n:] == 0.0), f"o padding rows, length {n}"
        assert np.all(np.isneginf(r["lse"][b, :, n:])), f"lse padding rows, length {n}"
        for name in ("dq", "dk", "dv"):
            assert np.all(r[name][b, :, n:] == 0.0), f"{name} padding rows, length {n}"
        for name in ("o", "lse", "dq", "dk", "dv"):
            assert np.all(np.isfinite(r[name][b, :, :n])), f"{name} real rows, length {n}"


def pin_full_lengths_are_the_plain_run(o):
    q, k, v, dO = _inputs(4, pad=0.5)
    rag = o.run_ragged(q, k, v, [S] * B, dO)
    pl = o.run(q, k, v, dO)
    for name in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(rag[name], pl[name]), f"{name}: all lengths S differs from run"


ALL_PINS = [pin_real_rows_equal_padded_forward, pin_masked_padded_backward,
            pin_padding_outputs_and_nan_inputs, pin_full_lengths_are_the_plain_run]

"""Pins for the fp64 CPU oracle of decode attention (``oracle/ref_decode.c``).

Every pin takes a ``DecodeOracle`` and raises ``AssertionError`` when the oracle
disagrees with the fact it checks.  ``test_decode_oracle.py`` runs them on the
real oracle and on deliberately broken copies of it.

What pins what (decode attention is one query per (sequence, head) against the
cached keys and values, and must equal the last row of full causal attention:
"xtrain evolution overview", post-training stage, milestones M2a-M2c):

* the last row of the causal-attention oracle (itself pinned on its own) on
  every shape, with GQA, for the full cache and for each ragged length
* ragged lengths: positions past a sequence's length are never read (they hold
  NaN and huge values here); an empty sequence gives o = 0 and lse = -inf
* closed forms: one cached position gives o = v_0 and lse = scale q.k_0; zero
  keys give the mean of the values and lse = ln n; constant values give o = c
* key-shift invariance with scores far beyond exp() overflow
* the GQA mapping: query head h reads kv head floor(h / group)
* the library cross-check: torch fp64 scaled_dot_product_attention of one query
"""
import math

import numpy as np

from oracle import default as default_attention


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    den = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * den, f"{what}: max|err| {err:.3e} > {tol:g} * {den:.3e}"


def _last_row(qfull, k, v, n, scale):
    """Row n-1 of full causal attention over the first n positions."""
    r = default_attention().run(qfull[:, :, :n], k[:, :, :n], v[:, :, :n], scale=scale,
                                backward=False)
    return r["o"][:, :, n - 1], r["lse"][:, :, n - 1]


SHAPES = [(2, 9, 4, 2, 8), (1, 1, 2, 1, 4), (3, 17, 3, 3, 16), (1, 40, 8, 2, 16)]


def pin_last_row_of_causal(o):
    for i, (B, T, H, Hkv, hd) in enumerate(SHAPES):
        qf, k, v = _rand((B, H, T, hd), 10 + i), _rand((B, Hkv, T, hd), 20 + i), _rand((B, Hkv, T, hd), 30 + i)
        scale = 0.7 / math.sqrt(hd)
        r = o.decode(qf[:, :, T - 1], k, v, scale=scale)
        ro, rl = _last_row(qf, k, v, T, scale)
        _close(r["o"], ro, 1e-12, f"o vs last causal row {B, T, H, Hkv, hd}")
        _close(r["lse"], rl, 1e-12, f"lse vs last causal row {B, T, H, Hkv, hd}")


def pin_ragged_lengths(o):
    B, T, H, Hkv, hd = 5, 12, 4, 2, 8
    lens = [12, 5, 1, 0, 9]
    qf, k, v = _rand((B, H, T, hd), 40), _rand((B, Hkv, T, hd), 41), _rand((B, Hkv, T, hd), 42)
    for b, n in enumerate(lens):  # positions past the length must never be read
        k[b, :, n:] = np.nan
        v[b, :, n:] = 1e300
    q = np.stack([qf[b, :, max(n, 1) - 1] for b, n in enumerate(lens)])
    r = o.decode(q, k, v, lens=lens)
    for b, n in enumerate(lens):
        if n == 0:
            assert np.all(r["o"][b] == 0.0), "empty sequence: o must be 0"
            assert np.all(np.isneginf(r["lse"][b])), "empty sequence: lse must be -inf"
            continue
        ro, rl = _last_row(qf[b:b + 1], k[b:b + 1], v[b:b + 1], n, 1.0 / math.sqrt(hd))
        _close(r["o"][b], ro[0], 1e-12, f"ragged o, length {n}")
        _close(r["lse"][b], rl[0], 1e-12, f"ragged lse, length {n}")


def pin_closed_forms(o):
    B, T, H, Hkv, hd = 2, 6, 4, 2, 8
    q, k, v = _rand((B, H, hd), 50), _rand((B, Hkv, T, hd), 51), _rand((B, Hkv, T, hd), 52)
    scale = 0.3
    g = np.arange(H) // (H // Hkv)
    # one cached position
    r = o.decode(q, k, v, lens=[1, 1], scale=scale)
    _close(r["o"], v[:, g, 0], 1e-14, "one position: o = v_0")
    _close(r["lse"], scale * np.einsum("bhd,bhd->bh", q, k[:, g, 0]), 1e-14, "one position: lse")
    # zero keys: uniform weights
    r = o.decode(q, np.zeros_like(k), v, lens=[6, 4], scale=scale)
    _close(r["o"][0], v[0, g, :6].mean(axis=1), 1e-13, "zero keys: mean of v (n=6)")
    _close(r["o"][1], v[1, g, :4].mean(axis=1), 1e-13, "zero keys: mean of v (n=4)")
    _close(r["lse"], np.log([[6.0] * H, [4.0] * H]), 1e-14, "zero keys: lse = ln n")
    # constant values
    c = _rand(hd, 53)
    r = o.decode(q, k, np.broadcast_to(c, v.shape), scale=scale)
    _close(r["o"], np.broadcast_to(c, (B, H, hd)), 1e-13, "constant values")


def pin_key_shift(o):
    B, T, H, Hkv, hd = 1, 10, 2, 1, 8
    q, k, v = 4.0 * _rand((B, H, hd), 60), _rand((B, Hkv, T, hd), 61), _rand((B, Hkv, T, hd), 62)
    u = 300.0 * np.abs(_rand(hd, 63)) * np.sign(q[0, 0])  # scores of order 1e3: exp() overflows
    a, b = o.decode(q, k, v, scale=0.5), o.decode(q, k + u, v, scale=0.5)
    _close(b["o"], a["o"], 1e-12, "key shift: o unchanged")
    _close(b["lse"], a["lse"] + 0.5 * np.einsum("bhd,d->bh", q, u), 1e-12,
           "key shift: lse moves by scale q.u")


def pin_gqa_mapping(o):
    B, T, H, Hkv, hd = 1, 5, 6, 2, 4
    q, k = _rand((B, H, hd), 70), _rand((B, Hkv, T, hd), 71)
    c = np.array([[1.0, 2.0, 3.0, 4.0], [-5.0, -6.0, -7.0, -8.0]])
    v = np.broadcast_to(c[None, :, None, :], (B, Hkv, T, hd)).copy()
    r = o.decode(q, k, v)
    for h in range(H):
        _close(r["o"][0, h], c[h // 3], 1e-14, f"query head {h} reads kv head {h // 3}")


def pin_torch_sdpa(o):
    import torch
    import torch.nn.functional as F
    B, T, H, Hkv, hd = 2, 13, 6, 3, 8
    q, k, v = _rand((B, H, hd), 80), _rand((B, Hkv, T, hd), 81), _rand((B, Hkv, T, hd), 82)
    scale = 0.4
    group = H // Hkv
    kt = torch.tensor(k).repeat_interleave(group, dim=1)
    vt = torch.tensor(v).repeat_interleave(group, dim=1)
    ref = F.scaled_dot_product_attention(torch.tensor(q)[:, :, None, :], kt, vt, scale=scale)[:, :, 0]
    lse = torch.logsumexp(scale * torch.einsum("bhd,bhtd->bht", torch.tensor(q), kt), dim=-1)
    r = o.decode(q, k, v, scale=scale)
    _close(r["o"], ref.numpy(), 1e-12, "torch sdpa o")
    _close(r["lse"], lse.numpy(), 1e-12, "torch logsumexp")


ALL_PINS = [pin_last_row_of_causal, pin_ragged_lengths, pin_closed_forms, pin_key_shift,
            pin_gqa_mapping, pin_torch_sdpa]

"""Pins for the fp64 CPU oracle of the per-head RMS QK-norm + RoPE step.

Every pin takes a ``NormOracle`` and raises ``AssertionError`` when the oracle
disagrees with the fact it checks.  ``test_norm_oracle.py`` runs them on the
real oracle and on deliberately broken copies of it.

What pins what (the oracle computes RMSNorm over each head's hd values with a
weight per dimension, then the half-split rotary embedding at the token's
position in its sequence, as in the "xtrain evolution overview" rows T5, T9,
T10 and the KI-1 fix of "xtrain -- Known Issues & Perf Backlog"):

* hand-derived outputs for unit basis vectors (tests/golden): the norm's scale,
  the pairing of dimension i with i + hd/2, each pair's frequency, the sign of
  the rotation and the position used
* position 0 rotates nothing: the output is w * x / r there
* the rotation preserves the length of each pair; with unit weight the squared
  length of a row is hd * m / (m + eps), m the mean square of the input
* scale invariance with eps = 0: out(a x) = out(x) for a > 0, hence
  sum_k x_k dx_k = 0 for every row
* the relative-position property of the rotary embedding: dot products of a
  rotated q and k depend on their positions only through the difference
* the output is head-major: a token's heads land in [b, h, s, :]
* central finite differences of L = sum(Out * G) against the analytic backward
  (dx and dw)
* the library cross-check: torch fp64 ``rms_norm`` + the rotation, autograd
"""
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    den = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol * den, f"{what}: max|err| {err:.3e} > {tol:g} * {den:.3e}"


def pin_golden_unit_vectors(o):
    with open(os.path.join(GOLDEN, "qknorm_rope_unit_vectors.json")) as f:
        g = json.load(f)
    hd = g["hd"]
    S = 1 + max(c["s"] for c in g["cases"])
    for c in g["cases"]:
        x = np.zeros((1, S, 1, hd))
        x[0, c["s"], 0, :] = c["x"]
        x[0, [t for t in range(S) if t != c["s"]], 0, 0] = 1.0  # other rows: anything finite
        out = o.fwd(x, np.ones(hd), eps=g["eps"], base=g["base"])
        _close(out[0, 0, c["s"]], c["out"], 1e-13, f"unit vector {c['x']} at s={c['s']}")


def pin_position_zero_is_identity(o):
    B, S, H, hd = 2, 3, 3, 8
    x, w = _rand((B, S, H, hd), 1), _rand(hd, 2)
    eps = 1e-6
    out = o.fwd(x, w, eps=eps)
    r = np.sqrt(np.mean(x[:, 0] ** 2, axis=-1, keepdims=True) + eps)
    _close(out[:, :, 0, :], w * x[:, 0] / r, 1e-13, "position 0")


def pin_pair_lengths_and_row_norm(o):
    B, S, H, hd = 1, 7, 2, 16
    x, eps = 3.0 * _rand((B, S, H, hd), 3), 1e-2
    w = _rand(hd, 4)
    out = o.fwd(x, w, eps=eps)
    r = np.sqrt(np.mean(x ** 2, axis=-1, keepdims=True) + eps)
    y = np.transpose(w * x / r, (0, 2, 1, 3))  # [B, H, S, hd]
    h = hd // 2
    _close(out[..., :h] ** 2 + out[..., h:] ** 2, y[..., :h] ** 2 + y[..., h:] ** 2, 1e-12,
           "pair lengths")
    out1 = o.fwd(x, np.ones(hd), eps=eps)
    m = np.transpose(np.mean(x ** 2, axis=-1), (0, 2, 1))
    _close(np.sum(out1 ** 2, axis=-1), hd * m / (m + eps), 1e-12, "row norm with unit weight")


def pin_scale_invariance(o):
    B, S, H, hd = 1, 4, 2, 8
    x, w, G = _rand((B, S, H, hd), 5), _rand(hd, 6), _rand((B, H, S, hd), 7)
    _close(o.fwd(2.5 * x, w, eps=0.0), o.fwd(x, w, eps=0.0), 1e-13, "scale invariance")
    dx, _ = o.bwd(x, w, G, eps=0.0)
    _close(np.sum(x * dx, axis=-1), np.zeros((B, S, H)), 1e-12, "sum_k x_k dx_k")


def pin_relative_position(o):
    hd, S = 16, 12
    q, k = _rand(hd, 8), _rand(hd, 9)
    w = np.ones(hd)

    def dot(m, n):
        x = np.zeros((1, S, 2, hd))
        x[0, :, 0, 0] = 1.0
        x[0, :, 1, 0] = 1.0
        x[0, m, 0, :] = q
        x[0, n, 1, :] = k
        out = o.fwd(x, w, eps=0.0)
        return float(out[0, 0, m] @ out[0, 1, n])

    for m, n, t in ((3, 1, 4), (5, 5, 6), (2, 7, 3)):
        a, b = dot(m, n), dot(m + t, n + t)
        assert abs(a - b) <= 1e-12 * max(1.0, abs(a)), f"relative position ({m},{n})+{t}: {a} vs {b}"
    assert abs(dot(3, 1) - dot(4, 1)) > 1e-6, "rotation does not depend on position"


def pin_head_major_layout(o):
    B, S, H, hd = 2, 3, 4, 4
    x, w = _rand((B, S, H, hd), 10), _rand(hd, 11)
    out = o.fwd(x, w)
    for h in range(H):
        one = o.fwd(x[:, :, h:h + 1, :], w)
        _close(out[:, h:h + 1], one, 0.0, f"head {h} on its own")


def pin_finite_differences(o):
    eps_fd = 1e-5
    for (B, S, H, hd, eps, seed) in ((1, 3, 2, 4, 1e-6, 20), (2, 2, 3, 8, 1e-1, 21)):
        x, w, G = _rand((B, S, H, hd), seed), _rand(hd, seed + 1), _rand((B, H, S, hd), seed + 2)
        dx, dw = o.bwd(x, w, G, eps=eps)

        def L(xx, ww):
            return float(np.sum(o.fwd(xx, ww, eps=eps) * G))

        fdx = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps_fd
            xm[idx] -= eps_fd
            fdx[idx] = (L(xp, w) - L(xm, w)) / (2 * eps_fd)
        fdw = np.zeros(hd)
        for d in range(hd):
            wp, wm = w.copy(), w.copy()
            wp[d] += eps_fd
            wm[d] -= eps_fd
            fdw[d] = (L(x, wp) - L(x, wm)) / (2 * eps_fd)
        _close(dx, fdx, 1e-6, f"FD dx {x.shape}")
        _close(dw, fdw, 1e-6, f"FD dw {x.shape}")


def pin_torch_cross_check(o):
    import torch
    import torch.nn.functional as F
    B, S, H, hd, eps, base = 2, 5, 3, 8, 1e-6, 10000.0
    x, w, G = _rand((B, S, H, hd), 30), _rand(hd, 31), _rand((B, H, S, hd), 32)
    xt = torch.tensor(x, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    y = F.rms_norm(xt, (hd,), weight=wt, eps=eps)            # [B, S, H, hd]
    half = hd // 2
    inv = base ** (-2.0 * torch.arange(half, dtype=torch.float64) / hd)
    ang = torch.arange(S, dtype=torch.float64)[:, None] * inv[None, :]   # [S, half]
    c, s = torch.cos(ang)[None, :, None, :], torch.sin(ang)[None, :, None, :]
    y1, y2 = y[..., :half], y[..., half:]
    out = torch.cat([y1 * c - y2 * s, y2 * c + y1 * s], dim=-1).permute(0, 2, 1, 3)
    (out * torch.tensor(G)).sum().backward()
    _close(o.fwd(x, w, eps=eps), out.detach().numpy(), 1e-12, "torch forward")
    dx, dw = o.bwd(x, w, G, eps=eps)
    _close(dx, xt.grad.numpy(), 1e-11, "torch dx")
    _close(dw, wt.grad.numpy(), 1e-11, "torch dw")


ALL_PINS = [pin_golden_unit_vectors, pin_position_zero_is_identity, pin_pair_lengths_and_row_norm,
            pin_scale_invariance, pin_relative_position, pin_head_major_layout,
            pin_finite_differences, pin_torch_cross_check]

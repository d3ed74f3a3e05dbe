"""Pins for the fp64 CPU oracle: checks against facts fixed by the mathematics.

Every pin takes an ``Oracle`` instance and raises ``AssertionError`` when the
oracle disagrees with the fact it checks.  ``test_oracle_pins.py`` runs them on
the real oracle; ``test_oracle_mutants.py`` runs them on deliberately broken
copies of it to show that plausible mistakes are caught.

What pins what (the oracle computes causal softmax attention and its backward,
as in the "xtrain evolution overview" infra table, rows T14/T15, and the KI-1
fix of "xtrain -- Known Issues & Perf Backlog"):

* hand-worked example with exact values derived on paper (tests/golden)
* closed forms: first row, zero keys (uniform weights), constant values, S = 1
* softmax rows sum to one; weights above the diagonal are exactly zero
* key-shift invariance with scores far beyond exp() overflow
* causality: future inputs leave earlier O/LSE/dQ rows bitwise unchanged
* GQA with group 1 equals per-head MHA exactly; GQA equals MHA on repeated K/V
* finite differences of L = sum(O * dO) against the analytic backward
* the library cross-check: torch fp64 scaled_dot_product_attention + autograd
* exact identities: row sums of dS vanish, D = rowsum(dO*O) equals sum(P*dP),
  column sum of dV, and sum_i q_i.dQ_i = sum_j k_j.dK_j
* batch independence and thread-count independence (bitwise)
"""
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(shape, seed):
    return _rng(seed).standard_normal(shape)


def _rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    den = max(1e-300, float(np.max(np.abs(b))) if b.size else 1.0)
    return float(np.max(np.abs(a - b))) / den if a.size else 0.0


def _close(a, b, tol, what):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    assert err <= tol * scale, f"{what}: max|err| {err:.3e} > {tol:.1e} * {scale:.3e}"


def _inputs(B, S, H, Hkv, hd, seed):
    r = _rng(seed)
    return (r.standard_normal((B, H, S, hd)), r.standard_normal((B, Hkv, S, hd)),
            r.standard_normal((B, Hkv, S, hd)), r.standard_normal((B, H, S, hd)))


# --------------------------------------------------------------------------
def pin_hand_worked(oracle):
    """Exact values derived by hand for a two-token, one-dimensional example
    with two query heads sharing one kv head (tests/golden/hand_worked_gqa.json)."""
    with open(os.path.join(GOLDEN, "hand_worked_gqa.json")) as f:
        g = json.load(f)
    q, k, v, dO = (np.array(g["inputs"][n], dtype=np.float64) for n in ("q", "k", "v", "dO"))
    out = oracle.run(q, k, v, dO, scale=g["scale"])
    for n in ("o", "lse", "dq", "dk", "dv"):
        _close(out[n], np.array(g["expected"][n], dtype=np.float64), 1e-14, f"hand-worked {n}")


def pin_rows_sum_to_one(oracle):
    S, hd = 13, 8
    q, k, v = _rand((S, hd), 1), _rand((S, hd), 2), _rand((S, hd), 3)
    P = oracle.head(q, k, v, want=("P",))["P"]
    assert np.all(np.abs(P.sum(axis=1) - 1.0) <= 1e-12), "softmax rows do not sum to 1"
    upper = np.triu(np.ones((S, S), dtype=bool), k=1)
    assert np.all(P[upper] == 0.0), "weights above the diagonal are not exactly zero"
    assert np.all(P[~upper] > 0.0), "a visible key has zero weight"


def pin_first_row(oracle):
    S, hd = 9, 16
    q, k, v = _rand((S, hd), 4), _rand((S, hd), 5), _rand((S, hd), 6)
    scale = 0.3
    out = oracle.head(q, k, v, scale=scale, want=("o", "lse"))
    _close(out["o"][0], v[0], 1e-15, "O_0 = V_0")
    _close(out["lse"][0], scale * float(q[0] @ k[0]), 1e-14, "LSE_0 = scale q0.k0")


def pin_zero_keys(oracle):
    """K = 0: uniform weights 1/(i+1) over the prefix."""
    S, hd = 11, 8
    q, v, dO = _rand((S, hd), 7), _rand((S, hd), 8), _rand((S, hd), 9)
    k = np.zeros((S, hd))
    out = oracle.head(q, k, v, dO, want=("P", "o", "lse", "dq", "dv"))
    i = np.arange(S)
    P_exp = np.tril(np.ones((S, S))) / (i + 1.0)[:, None]
    _close(out["P"], P_exp, 1e-15, "P = 1/(i+1)")
    _close(out["o"], np.cumsum(v, axis=0) / (i + 1.0)[:, None], 1e-14, "O = prefix mean")
    _close(out["lse"], np.log(i + 1.0), 1e-14, "LSE = ln(i+1)")
    assert np.all(out["dq"] == 0.0), "dQ must vanish when K = 0"
    w = dO / (i + 1.0)[:, None]
    dv_exp = np.cumsum(w[::-1], axis=0)[::-1]
    _close(out["dv"], dv_exp, 1e-14, "dV_j = sum_{i>=j} dO_i/(i+1)")


def pin_constant_values(oracle):
    """V_j = c for every j: O_i = c, and dQ = dK = 0."""
    S, hd = 10, 8
    q, k, dO = _rand((S, hd), 10), _rand((S, hd), 11), _rand((S, hd), 12)
    c = _rand((hd,), 13)
    v = np.tile(c, (S, 1))
    out = oracle.head(q, k, v, dO, want=("o", "dq", "dk", "dv"))
    _close(out["o"], v, 1e-14, "O = c")
    _close(out["dq"], np.zeros_like(q), 1e-13, "dQ = 0")
    _close(out["dk"], np.zeros_like(k), 1e-13, "dK = 0")
    assert np.max(np.abs(out["dv"])) > 0.1


def pin_single_token(oracle):
    hd = 16
    q, k, v, dO = (_rand((1, hd), s) for s in (14, 15, 16, 17))
    scale = 0.25
    out = oracle.head(q, k, v, dO, scale=scale, want=("o", "lse", "dq", "dk", "dv"))
    _close(out["o"], v, 1e-15, "S=1: O = V")
    _close(out["lse"], [scale * float(q[0] @ k[0])], 1e-15, "S=1: LSE")
    _close(out["dv"], dO, 1e-15, "S=1: dV = dO")
    assert np.all(out["dq"] == 0.0) and np.all(out["dk"] == 0.0), "S=1: dQ = dK = 0"


def pin_key_shift(oracle):
    """K_j -> K_j + u leaves O, dQ, dK, dV unchanged and shifts LSE_i by
    scale q_i.u.  The shift pushes every score to ~ +1000, far past where
    exp() overflows in double, so a softmax without max subtraction fails."""
    B, S, H, Hkv, hd = 1, 12, 2, 2, 8
    q, k, v, dO = _inputs(B, S, H, Hkv, hd, 18)
    q[..., 0] = 1.0 + 0.1 * np.abs(q[..., 0])
    scale = 1.0 / math.sqrt(hd)
    u = np.zeros(hd)
    u[0] = 1000.0 / scale
    base = oracle.run(q, k, v, dO, scale=scale)
    shifted = oracle.run(q, k + u, v, dO, scale=scale)
    _close(shifted["o"], base["o"], 1e-9, "shift: O")
    _close(shifted["lse"] - scale * np.einsum("bhsd,d->bhs", q, u), base["lse"], 1e-9, "shift: LSE")
    for n in ("dq", "dk", "dv"):
        _close(shifted[n], base[n], 1e-8, f"shift: {n}")


def pin_causality(oracle):
    """Perturbing inputs at positions >= t leaves O, LSE and dQ rows < t bitwise equal."""
    B, S, H, Hkv, hd, t = 2, 12, 2, 1, 8, 5
    q, k, v, dO = _inputs(B, S, H, Hkv, hd, 19)
    base = oracle.run(q, k, v, dO)
    r = _rng(20)
    q2, k2, v2, dO2 = (a.copy() for a in (q, k, v, dO))
    for a in (q2, k2, v2, dO2):
        a[:, :, t:, :] += r.standard_normal(a[:, :, t:, :].shape)
    pert = oracle.run(q2, k2, v2, dO2)
    for n in ("o", "dq"):
        assert np.array_equal(pert[n][:, :, :t], base[n][:, :, :t]), f"causality: {n} rows < t changed"
        assert not np.array_equal(pert[n][:, :, t:], base[n][:, :, t:])
    assert np.array_equal(pert["lse"][:, :, :t], base["lse"][:, :, :t]), "causality: LSE rows < t changed"


def pin_group1_is_mha(oracle):
    """GQA with group = 1 equals per-head multi-head attention exactly."""
    B, S, H, hd = 2, 9, 3, 8
    q, k, v, dO = _inputs(B, S, H, H, hd, 21)
    out = oracle.run(q, k, v, dO)
    for b in range(B):
        for h in range(H):
            ref = oracle.head(q[b, h], k[b, h], v[b, h], dO[b, h], want=("o", "lse", "dq", "dk", "dv"))
            for n in ref:
                assert np.array_equal(out[n][b, h], ref[n]), f"group 1 != MHA for {n} at b={b} h={h}"


def pin_gqa_is_repeated_mha(oracle):
    """GQA (query head h reads kv head h // group) equals MHA on repeated K/V,
    with dK/dV of the repeated heads summed over the group."""
    B, S, H, Hkv, hd = 2, 10, 6, 2, 8
    group = H // Hkv
    q, k, v, dO = _inputs(B, S, H, Hkv, hd, 22)
    gqa = oracle.run(q, k, v, dO)
    krep, vrep = np.repeat(k, group, axis=1), np.repeat(v, group, axis=1)
    mha = oracle.run(q, krep, vrep, dO)
    for n in ("o", "lse", "dq"):
        assert np.array_equal(gqa[n], mha[n]), f"GQA != repeated MHA for {n}"
    for n in ("dk", "dv"):
        summed = np.zeros_like(gqa[n])
        for r in range(group):
            summed += mha[n][:, [g * group + r for g in range(Hkv)]]
        _close(gqa[n], summed, 1e-15, f"GQA {n} = group sum of repeated MHA")


def pin_finite_differences(oracle):
    """Central differences of L = sum(O * dO) match the analytic dQ, dK, dV."""
    for (B, S, H, Hkv, hd, seed) in [(1, 16, 2, 2, 16, 23), (1, 8, 4, 2, 8, 24)]:
        q, k, v, dO = _inputs(B, S, H, Hkv, hd, seed)
        scale = 1.0 / math.sqrt(hd)
        ana = oracle.run(q, k, v, dO, scale=scale)
        eps = 1e-5

        def loss(qq, kk, vv):
            return float(np.sum(oracle.run(qq, kk, vv, None, scale=scale, backward=False)["o"] * dO))

        for name, idx in (("dq", 0), ("dk", 1), ("dv", 2)):
            args = [q, k, v]
            base = args[idx]
            fd = np.zeros_like(base)
            it = np.nditer(base, flags=["multi_index"])
            for _ in it:
                mi = it.multi_index
                plus, minus = base.copy(), base.copy()
                plus[mi] += eps
                minus[mi] -= eps
                a_p = list(args); a_p[idx] = plus
                a_m = list(args); a_m[idx] = minus
                fd[mi] = (loss(*a_p) - loss(*a_m)) / (2 * eps)
            _close(ana[name], fd, 1e-6, f"finite differences {name} (B{B} S{S} H{H} Hkv{Hkv} hd{hd})")


def pin_torch_sdpa(oracle):
    """Library cross-check: torch fp64 CPU scaled_dot_product_attention (causal,
    GQA) with autograd, and torch.logsumexp of the masked scores."""
    import torch
    import torch.nn.functional as F
    B, S, H, Hkv, hd = 2, 37, 4, 2, 16
    q, k, v, dO = _inputs(B, S, H, Hkv, hd, 25)
    scale = 0.2
    out = oracle.run(q, k, v, dO, scale=scale)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale, enable_gqa=True)
    o.backward(torch.tensor(dO))
    _close(out["o"], o.detach().numpy(), 1e-12, "torch SDPA: O")
    _close(out["dq"], tq.grad.numpy(), 1e-12, "torch SDPA: dQ")
    _close(out["dk"], tk.grad.numpy(), 1e-12, "torch SDPA: dK")
    _close(out["dv"], tv.grad.numpy(), 1e-12, "torch SDPA: dV")
    krep = torch.tensor(np.repeat(k, H // Hkv, axis=1))
    s = torch.matmul(torch.tensor(q), krep.transpose(-1, -2)) * scale
    mask = torch.ones(S, S, dtype=torch.bool).triu(1)
    lse = torch.logsumexp(s.masked_fill(mask, float("-inf")), dim=-1)
    _close(out["lse"], lse.numpy(), 1e-12, "torch logsumexp: LSE")


def pin_identities(oracle):
    """sum_j dS_ij = 0; D_i = sum_d dO_id O_id = sum_j P_ij dP_ij;
    sum_j dV_j = sum_{h in g} sum_i dO_i; sum_i q_i.dQ_i = sum_j k_j.dK_j."""
    S, hd = 15, 8
    q, k, v, dO = (_rand((S, hd), s) for s in (26, 27, 28, 29))
    h = oracle.head(q, k, v, dO, want=("dS", "rowdot", "o"))
    assert np.max(np.abs(h["dS"].sum(axis=1))) <= 1e-13, "rows of dS must sum to zero"
    _close(h["rowdot"], np.sum(dO * h["o"], axis=1), 1e-13, "D = rowsum(dO*O)")

    B, S, H, Hkv, hd = 2, 14, 4, 2, 8
    group = H // Hkv
    q, k, v, dO = _inputs(B, S, H, Hkv, hd, 30)
    out = oracle.run(q, k, v, dO)
    for b in range(B):
        for g in range(Hkv):
            heads = range(g * group, (g + 1) * group)
            _close(out["dv"][b, g].sum(axis=0), sum(dO[b, hh].sum(axis=0) for hh in heads), 1e-13,
                   "sum_j dV_j = sum_i dO_i")
            lhs = sum(float(np.sum(q[b, hh] * out["dq"][b, hh])) for hh in heads)
            rhs = float(np.sum(k[b, g] * out["dk"][b, g]))
            assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(rhs)), f"q.dQ {lhs} != k.dK {rhs}"


def pin_batch_independence(oracle):
    B, S, H, Hkv, hd = 3, 11, 2, 1, 8
    q, k, v, dO = _inputs(B, S, H, Hkv, hd, 31)
    full = oracle.run(q, k, v, dO)
    for b in range(B):
        one = oracle.run(q[b:b + 1], k[b:b + 1], v[b:b + 1], dO[b:b + 1])
        for n in one:
            assert np.array_equal(full[n][b:b + 1], one[n]), f"batch entry {b} differs for {n}"


def pin_thread_independence(oracle):
    B, S, H, Hkv, hd = 2, 20, 4, 2, 8
    q, k, v, dO = _inputs(B, S, H, Hkv, hd, 32)
    oracle.set_threads(1)
    one = oracle.run(q, k, v, dO)
    oracle.set_threads(0)
    many = oracle.run(q, k, v, dO)
    for n in one:
        assert np.array_equal(one[n], many[n]), f"thread count changes {n}"


def pin_unit_restriction(oracle):
    """Computing a subset of (b, kv head) units gives the same values as the full run."""
    B, S, H, Hkv, hd = 2, 9, 4, 2, 8
    q, k, v, dO = _inputs(B, S, H, Hkv, hd, 33)
    full = oracle.run(q, k, v, dO)
    part = oracle.run(q, k, v, dO, units=(1, 3))
    group = H // Hkv
    for u in (1, 2):
        b, g = divmod(u, Hkv)
        hs = slice(g * group, (g + 1) * group)
        for n in ("o", "lse", "dq"):
            assert np.array_equal(part[n][b, hs], full[n][b, hs])
        for n in ("dk", "dv"):
            assert np.array_equal(part[n][b, g], full[n][b, g])
    assert np.all(np.isnan(part["o"][0, 0:group]))


ALL_PINS = [
    pin_hand_worked, pin_rows_sum_to_one, pin_first_row, pin_zero_keys, pin_constant_values,
    pin_single_token, pin_key_shift, pin_causality, pin_group1_is_mha, pin_gqa_is_repeated_mha,
    pin_finite_differences, pin_torch_sdpa, pin_identities, pin_batch_independence,
    pin_thread_independence, pin_unit_restriction,
]

"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI
binding, run the oracle on the same seeded inputs, compare.

Tolerance (per output tensor X in {o, lse, dq, dk, dv}):
    max |X_gpu - X_ref| <= tau * max(max |X_ref|, 1e-3 * T_X)
with tau = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs, X_ref the fp64 oracle
on the same (already rounded) inputs.  T_X is the size of one term of the sum
that defines X (e.g. scale*|dO||v||k| for dq); it only matters when X_ref is
identically zero by cancellation (a single token gives dq = dk = 0 exactly),
where the max-normalised bound alone would demand bit-exact zeros.
"""
import sys

import numpy as np

from bwd_head_rms_amd import inputs

TAU = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("o", "lse", "dq", "dk", "dv")


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(arrs, dtype):
    return {n: inputs.to_torch(a, dtype, "cuda") for n, a in arrs.items()}


def gpu_run(arrs, dtype, scale=None, backward=True):
    """HIP fwd (+ bwd) on numpy float32 inputs; returns float64 numpy outputs."""
    import torch
    from bwd_head_rms_amd import api
    t = to_dev(arrs, dtype)
    o, lse = api.fwd(t["q"], t["k"], t["v"], scale)
    out = {"o": o, "lse": lse}
    if backward:
        dq, dk, dv = api.bwd(t["q"], t["k"], t["v"], o, lse, t["dO"], scale)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: x.float().cpu().numpy().astype(np.float64) for n, x in out.items()}


def unit_slices(u, Hkv, group):
    """(b, query-head slice, kv head) of flattened (b, kv head) unit u."""
    b, g = divmod(u, Hkv)
    return b, slice(g * group, (g + 1) * group), g


def term_sizes(arrs, scale):
    """Size of one summand of each output's defining sum (see module doc)."""
    m = {n: float(np.max(np.abs(a))) for n, a in arrs.items()}
    return {"o": m["v"], "lse": 1.0, "dq": scale * m["dO"] * m["v"] * m["k"],
            "dk": scale * m["dO"] * m["v"] * m["q"], "dv": m["dO"]}


BF16_UNIT_ROUNDOFF = 2.0 ** -8  # nearest-even rounding to bf16's 8-bit significand


def bf16_backward_allowance(arrs, ref, o_used, scale):
    """Per-element bound on what the bf16 backward's own roundings may move
    dq, dk and dv by, to first order.  Each term is the rigorous bound of one
    rounding that the bf16 path performs by design:

    * D_i = sum_d dO_id o_id is taken from the o the backward is given (bf16),
      not the exact o*: with dD_i = sum_d dO_id (o_id - o*_id), dS_ij moves by
      exactly -P_ij dD_i, hence dq_i by -scale dD_i sum_j P_ij k_j and dk_j by
      -scale sum_i P_ij dD_i q_i;
    * dS is rounded to bf16 (relative error <= u = 2^-8) before the products
      dq = scale dS.K and dk = scale dS^T.Q: at most scale u sum_j |dS_ij||k_j|
      and scale u sum_i |dS_ij||q_i|;
    * P is rounded to bf16 before dv = P^T.dO: at most u sum_i P_ij |dO_i|.

    Absolute values are taken inside every sum, and dk, dv sum over the query
    heads of the group.  P, dP and dS are the exact ones, from the oracle's lse:
    P_ij = exp(scale q_i.k_j - lse_i) for j <= i, dP_ij = dO_i.v_j,
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik).  These bounds only matter where
    the sums cancel, as on rows that put nearly all weight on one key."""
    u = BF16_UNIT_ROUNDOFF
    q, k, v, dO = (np.asarray(arrs[n], np.float64) for n in ("q", "k", "v", "dO"))
    B, Hq, S, hd = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    dD = np.abs(np.sum(dO * (np.asarray(o_used, np.float64) - ref["o"]), axis=-1))  # [B,H,S]
    mask = np.tril(np.ones((S, S), bool))
    bq = np.zeros_like(q)
    bk = np.zeros_like(k)
    bv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kv, vv = k[b, h // group], v[b, h // group]
            P = np.where(mask, np.exp(scale * (q[b, h] @ kv.T) - ref["lse"][b, h][:, None]), 0.0)
            dP = dO[b, h] @ vv.T
            dS = np.abs(P * (dP - np.sum(P * dP, axis=1, keepdims=True)))
            bq[b, h] = scale * (dD[b, h][:, None] * (P @ np.abs(kv)) + u * (dS @ np.abs(kv)))
            bk[b, h // group] += scale * ((P * dD[b, h][:, None] + u * dS).T @ np.abs(q[b, h]))
            bv[b, h // group] += u * (P.T @ np.abs(dO[b, h]))
    return {"dq": bq, "dk": bk, "dv": bv}


def compare(gpu, ref, dtype, what, names=NAMES, units=None, Hkv=None, group=None, terms=None,
            allow=None):
    """Assert the tolerance for every output; with ``units`` only those
    (b, kv head) units are compared.  ``allow`` ({name: array shaped like the
    output}) adds a per-element allowance to the bound.  Returns
    {name: err/max|ref|}."""
    tau = TAU[dtype]
    ratios = {}
    for n in names:
        g_, r_ = gpu[n], ref[n]
        if allow is not None and n in allow:
            den0 = float(np.max(np.abs(r_)))
            if terms is not None:
                den0 = max(den0, 1e-3 * terms[n])
            excess = np.abs(g_ - r_) - allow[n]
            err = float(np.max(excess))
            ratios[n] = err / den0 if den0 > 0 else err
            assert np.all(np.isfinite(g_)), f"{what}: {n} has non-finite values"
            assert err <= tau * den0, (f"{what}: {n} max(|err| - allowance) {err:.3e} > "
                                       f"{tau:g} * {den0:.3e}")
            continue
        if units is not None:
            gs, rs = [], []
            for u in units:
                b, hs, kv = unit_slices(u, Hkv, group)
                idx = (b, kv) if n in ("dk", "dv") else (b, hs)
                gs.append(g_[idx].ravel())
                rs.append(r_[idx].ravel())
            g_, r_ = np.concatenate(gs), np.concatenate(rs)
        assert np.all(np.isfinite(g_)), f"{what}: {n} has non-finite values"
        err = float(np.max(np.abs(g_ - r_)))
        den = float(np.max(np.abs(r_)))
        if terms is not None:
            den = max(den, 1e-3 * terms[n])
        ratios[n] = err / den if den > 0 else err
        assert err <= tau * den, f"{what}: {n} max|err| {err:.3e} > {tau:g} * {den:.3e}"
    log(f"{what}: " + " ".join(f"{n}={ratios[n]:.2e}" for n in names))
    return ratios

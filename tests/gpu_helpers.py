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


def compare(gpu, ref, dtype, what, names=NAMES, units=None, Hkv=None, group=None, terms=None):
    """Assert the tolerance for every output; with ``units`` only those
    (b, kv head) units are compared.  Returns {name: err/max|ref|}."""
    tau = TAU[dtype]
    ratios = {}
    for n in names:
        g_, r_ = gpu[n], ref[n]
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

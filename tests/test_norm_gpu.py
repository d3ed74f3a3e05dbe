"""GPU parity of the per-head RMS QK-norm + RoPE step (xattn_qknorm_rope_fwd /
_bwd through the C ABI) against its fp64 oracle on the same seeded inputs.

Tolerance per output tensor X in {out, dx, dw}: max|X_gpu - X_ref| <= tau *
max|X_ref| with tau = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs (the same
bar as the attention path).  Shapes: the q and k inputs of every attention
workload at full size (x = [B, S, heads, hd] as the projection writes it), a
ragged set spanning several workgroups and partial ones, every head dimension,
S = 1, positions far beyond the workloads' (angle reduction), other eps and
base values; dw is also checked bitwise run to run.
"""
import zlib

import numpy as np
import pytest

import gpu_helpers as H
from bwd_head_rms_amd import inputs
from oracle import default_norm

pytestmark = pytest.mark.gpu


def _inputs(B, S, Hh, hd, dtype, seed):
    rng = np.random.default_rng(seed)
    x = (2.0 * rng.standard_normal((B, S, Hh, hd))).astype(np.float32)
    w = (1.0 + 0.25 * rng.standard_normal(hd)).astype(np.float32)
    g = rng.standard_normal((B, Hh, S, hd)).astype(np.float32)
    if dtype == "bf16":
        x = inputs.bf16_round(x)
    return x, w, g


def _gpu(x, w, g, dtype, eps, base):
    import torch
    from bwd_head_rms_amd import api
    tx = inputs.to_torch(x, dtype, "cuda")
    tw = torch.from_numpy(w).cuda()
    tg = torch.from_numpy(g).cuda()
    out = api.qknorm_rope_fwd(tx, tw, eps=eps, rope_base=base)
    dx, dw = api.qknorm_rope_bwd(tx, tw, tg, eps=eps, rope_base=base)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)  # noqa: E731
    return f(out), f(dx), f(dw)


def _check(B, S, Hh, hd, dtype, seed, eps=1e-6, base=10000.0, what=""):
    H.log(f"qknorm_rope {what} B={B} S={S} H={Hh} hd={hd} {dtype} eps={eps} base={base}")
    x, w, g = _inputs(B, S, Hh, hd, dtype, seed)
    out, dx, dw = _gpu(x, w, g, dtype, eps, base)
    o = default_norm()
    ref_out = o.fwd(x, w, eps=eps, base=base)
    ref_dx, ref_dw = o.bwd(x, w, g, eps=eps, base=base)
    tau = H.TAU[dtype]
    msg = []
    for n, a, r in (("out", out, ref_out), ("dx", dx, ref_dx), ("dw", dw, ref_dw)):
        assert np.all(np.isfinite(a)), f"{what}: {n} non-finite"
        err = float(np.max(np.abs(a - r)))
        den = float(np.max(np.abs(r)))
        msg.append(f"{n}={err / den:.2e}")
        assert err <= tau * den, f"{what} {dtype}: {n} max|err| {err:.3e} > {tau:g} * {den:.3e}"
    H.log("  " + " ".join(msg))


# the q and k inputs of every attention workload, at full size
WORKLOAD_INPUTS = []
for name, wl in inputs.WORKLOADS.items():
    WORKLOAD_INPUTS.append((f"{name}:q", wl.B, wl.S, wl.H, wl.hd, wl.dtype))
    if wl.Hkv != wl.H:
        WORKLOAD_INPUTS.append((f"{name}:k", wl.B, wl.S, wl.Hkv, wl.hd, wl.dtype))


@pytest.mark.parametrize("case", WORKLOAD_INPUTS, ids=lambda c: c[0])
def test_workload_shapes(case):
    name, B, S, Hh, hd, dtype = case
    _check(B, S, Hh, hd, dtype, seed=zlib.crc32(name.encode()) % 1000, what=name)


EDGE = [(1, 1, 1, 16), (1, 1, 3, 64), (3, 7, 5, 16), (2, 33, 3, 32), (1, 130, 7, 64),
        (5, 3, 1, 32), (2, 1000, 9, 64)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", EDGE, ids=lambda s: "B{}_S{}_H{}_hd{}".format(*s))
def test_edge_shapes(shape, dtype):
    _check(*shape, dtype, seed=sum(shape), what="edge")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_other_eps_and_base(dtype):
    _check(2, 50, 3, 32, dtype, seed=7, eps=0.5, base=500.0, what="eps 0.5 base 500")
    _check(1, 20, 2, 64, dtype, seed=8, eps=0.0, base=1e6, what="eps 0 base 1e6")


def test_far_positions_f32():
    """Positions up to 70000: angles of ~7e4 rad must be reduced without losing
    fp32 accuracy."""
    _check(1, 70000, 1, 64, "f32", seed=9, what="long")


def test_dw_bitwise_run_to_run():
    x, w, g = _inputs(3, 257, 6, 64, "bf16", 10)
    a = _gpu(x, w, g, "bf16", 1e-6, 10000.0)
    b = _gpu(x, w, g, "bf16", 1e-6, 10000.0)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)

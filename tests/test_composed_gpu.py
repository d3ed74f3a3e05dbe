"""GPU parity of the composed path (xattn_composed_fwd / _bwd through the C ABI:
scores, causal softmax and products through S x S fp32 buffers) against the
fp64 attention oracle, and A/B against the fused path on the same inputs.

* Every named workload at full size: o, lse, dq, dk, dv against the oracle
  (all units where it finishes in seconds, else sampled units, as the fused
  parity tests), tolerance 1e-4 (fp32) / 2e-2 (bf16) of max|ref|.
* The probabilities the forward keeps: lower triangle against the oracle's P,
  rows summing to one, zeros past the diagonal to the end of the 128 tile.
* Edge shapes: S not a multiple of 4 or of the tile, S = 1, GQA, every head
  dimension, both dtypes.
* A/B: composed and fused outputs agree within twice the tolerance (each is
  within it of the oracle).
"""
import numpy as np
import pytest

import gpu_helpers as H
from bwd_head_rms_amd import inputs
from oracle import default

pytestmark = pytest.mark.gpu

SAMPLED = {
    "tiny_b1_s16_h2_hd16_f32": None,
    "dim384_b16_s256_h12_hd32_f32": None,
    "dim384_b32_s256_h12_hd32_bf16": None,
    "gqa_b16_s1024_h8_kv2_hd64_f32": [0, 31],
    "gqa_b16_s1024_h8_kv2_hd64_bf16": [0, 31],
    "long_b4_s2048_h16_hd64_bf16": [0, 63],
}


def composed_run(arrs, dtype, scale=None, keep_p=False):
    import torch
    from bwd_head_rms_amd import api
    t = H.to_dev(arrs, dtype)
    o, lse, p = api.composed_fwd(t["q"], t["k"], t["v"], scale)
    dq, dk, dv = api.composed_bwd(t["q"], t["k"], t["v"], p, t["dO"], scale)
    torch.cuda.synchronize()
    out = {n: x.float().cpu().numpy().astype(np.float64)
           for n, x in dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv).items()}
    if keep_p:
        out["p"] = p.cpu().numpy().astype(np.float64)
    del p
    return out


def _oracle(arrs, scale, units):
    ref = default()
    if units is None:
        return ref.run(arrs["q"], arrs["k"], arrs["v"], arrs["dO"], scale=scale)
    outs = [ref.run(arrs["q"], arrs["k"], arrs["v"], arrs["dO"], scale=scale, units=(u, u + 1))
            for u in units]
    merged = {n: np.where(np.isnan(outs[0][n]), 0.0, outs[0][n]) for n in H.NAMES}
    for o in outs[1:]:
        for n in H.NAMES:
            merged[n] = np.where(np.isnan(o[n]), merged[n], o[n])
    return merged


@pytest.mark.parametrize("name", list(inputs.WORKLOADS))
def test_workload_parity(name):
    w = inputs.WORKLOADS[name]
    H.log(f"composed parity {w.describe()}")
    arrs = inputs.generate_workload(w)
    gpu = composed_run(arrs, w.dtype, w.scale)
    units = SAMPLED[name]
    r = _oracle(arrs, w.scale, units)
    if units is None:
        H.compare(gpu, r, w.dtype, f"composed {name}")
    else:
        H.compare(gpu, r, w.dtype, f"composed {name}", units=units, Hkv=w.Hkv, group=w.group)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_probabilities(dtype):
    B, S, Hh, Hkv, hd = 2, 200, 3, 1, 32
    arrs = inputs.generate(B, S, Hh, Hkv, hd, seed=61, dtype=dtype)
    gpu = composed_run(arrs, dtype, keep_p=True)
    P = gpu["p"]
    tau = H.TAU[dtype] if dtype == "bf16" else 1e-5
    for b in range(B):
        for h in range(Hh):
            ref = default().head(arrs["q"][b, h], arrs["k"][b, 0], arrs["v"][b, 0], want=("P",))["P"]
            low = np.tril(np.ones((S, S), dtype=bool))
            assert np.max(np.abs(P[b, h][low] - ref[low])) <= tau, "P against the oracle"
            assert np.allclose(np.where(low, P[b, h], 0.0).sum(axis=1), 1.0, atol=1e-5)
            for i in range(S):
                end = min(S, (i // 128 + 1) * 128)
                assert np.all(P[b, h, i, i + 1:end] == 0.0), f"row {i}: nonzero past the diagonal"


EDGE = [(1, 1, 2, 1, 16), (2, 7, 2, 2, 32), (1, 33, 4, 2, 64), (2, 130, 3, 3, 16),
        (1, 129, 8, 2, 64), (3, 257, 2, 1, 32)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", EDGE, ids=lambda s: "B{}_S{}_H{}_kv{}_hd{}".format(*s))
def test_edge_shapes(shape, dtype):
    B, S, Hh, Hkv, hd = shape
    arrs = inputs.generate(B, S, Hh, Hkv, hd, seed=sum(shape), dtype=dtype)
    gpu = composed_run(arrs, dtype)
    r = default().run(arrs["q"], arrs["k"], arrs["v"], arrs["dO"])
    terms = H.term_sizes(arrs, 1.0 / np.sqrt(hd))
    H.compare(gpu, r, dtype, f"composed edge {shape} {dtype}", terms=terms)


@pytest.mark.parametrize("name", ["dim384_b16_s256_h12_hd32_f32", "gqa_b16_s1024_h8_kv2_hd64_bf16"])
def test_composed_equals_fused(name):
    w = inputs.WORKLOADS[name]
    arrs = inputs.generate_workload(w)
    a = composed_run(arrs, w.dtype, w.scale)
    b = H.gpu_run(arrs, w.dtype, w.scale)
    tau = 2 * H.TAU[w.dtype]
    msg = []
    for n in H.NAMES:
        err, den = float(np.max(np.abs(a[n] - b[n]))), float(np.max(np.abs(b[n])))
        msg.append(f"{n}={err / den:.2e}")
        assert err <= tau * den, f"{name}: composed vs fused {n}: {err:.3e} > {tau} * {den:.3e}"
    H.log(f"  composed vs fused {name}: " + " ".join(msg))

"""GPU parity of right-padded batches with per-sequence lengths
(xattn_fwd_ragged / xattn_bwd_ragged through the C ABI).

* Against the oracle (``Oracle.run_ragged``: each sequence's prefix through the
  causal-attention oracle) on real rows, every output, with the attention
  path's tolerance (fp32 1e-4, bf16 2e-2 of max|ref|; dq, dk, dv floors as in
  the plain parity tests); padding rows must be exactly o = 0, lse = -inf and
  zero gradients, with NaN in every padding input (never read).
* Batched == looped, bitwise: a ragged batch equals the plain kernels run on
  each sequence alone (S = its length), for every output.
* Right padding is free under the causal mask, bitwise: the real rows of the
  plain forward over the padded batch equal the ragged forward.
* Lengths outside [0, S] are clamped.
* The benchmark's length mix (8 x 2048, bf16): bitwise against the plain runs
  of its shortest and longest sequences, and one head against the oracle.
"""
import numpy as np
import pytest

import gpu_helpers as Hh
from bwd_head_rms_amd import inputs
from oracle import default

pytestmark = pytest.mark.gpu

NAMES = ("o", "lse", "dq", "dk", "dv")


def _draw(B, S, H, Hkv, hd, dtype, seed, lens, pad):
    a = inputs.generate(B, S, H, Hkv, hd, seed, shaped=True, dtype=dtype)
    for b, n in enumerate(lens):
        n = min(max(n, 0), S)
        for x in a.values():
            x[b, :, n:] = pad
    return a


def _gpu(a, dtype, lens=None, backward=True):
    import torch
    from bwd_head_rms_amd import api
    t = Hh.to_dev(a, dtype)
    tl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = api.fwd(t["q"], t["k"], t["v"], lens=tl)
    out = {"o": o, "lse": lse}
    if backward:
        out["dq"], out["dk"], out["dv"] = api.bwd(t["q"], t["k"], t["v"], o, lse, t["dO"], lens=tl)
    torch.cuda.synchronize()
    return {n: x.float().cpu().numpy().astype(np.float64) for n, x in out.items()}


def _check_oracle(B, S, H, Hkv, hd, dtype, lens, seed):
    a = _draw(B, S, H, Hkv, hd, dtype, seed, lens, pad=np.nan)
    g = _gpu(a, dtype, lens)
    clamped = [min(max(n, 0), S) for n in lens]
    ref = default().run_ragged(a["q"], a["k"], a["v"], clamped, a["dO"])
    terms = Hh.term_sizes({n: np.nan_to_num(x) for n, x in a.items()}, 1.0 / np.sqrt(hd))
    tau = Hh.TAU[dtype]
    msg = []
    for name in NAMES:
        gx, rx = g[name], ref[name]
        real = np.zeros(gx.shape, dtype=bool)
        for b, n in enumerate(clamped):
            real[b, :, :n] = True
        pad = ~real
        if name == "lse":
            assert np.all(np.isneginf(gx[pad])), f"{name}: padding rows must be -inf"
        else:
            assert np.all(gx[pad] == 0.0), f"{name}: padding rows must be 0"
        if not real.any():
            continue
        gr, rr = gx[real], rx[real]
        assert np.all(np.isfinite(gr)), f"{name}: real rows non-finite"
        err = float(np.max(np.abs(gr - rr)))
        den = max(float(np.max(np.abs(rr))), 1e-3 * terms[name])
        msg.append(f"{name}={err / den:.2e}")
        assert err <= tau * den, f"{name} {dtype}: max|err| {err:.3e} > {tau:g} * {den:.3e}"
    Hh.log(f"  ragged B{B} S{S} H{H}/{Hkv} hd{hd} {dtype} lens={lens}: " + " ".join(msg))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hd", [16, 32, 64])
def test_against_oracle(hd, dtype):
    _check_oracle(5, 300, 4, 2, hd, dtype, [300, 1, 0, 129, 256], seed=hd + 7)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gqa_group4_against_oracle(dtype):
    _check_oracle(3, 1024, 8, 2, 64, dtype, [1024, 555, 64], seed=44)


def test_lengths_are_clamped():
    _check_oracle(3, 70, 2, 1, 32, "f32", [-5, 1000, 33], seed=45)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_batched_equals_looped_bitwise(dtype):
    B, S, H, Hkv, hd = 4, 640, 4, 2, 64
    lens = [640, 513, 128, 77]
    a = _draw(B, S, H, Hkv, hd, dtype, 46, lens, pad=np.nan)
    g = _gpu(a, dtype, lens)
    for b, n in enumerate(lens):
        one = _gpu({k: np.ascontiguousarray(x[b:b + 1, :, :n]) for k, x in a.items()}, dtype)
        for name in NAMES:
            assert np.array_equal(g[name][b:b + 1, :, :n], one[name]), \
                f"{dtype} sequence {b} (length {n}): {name} differs from its own run"
    Hh.log(f"  batched == looped bitwise ({dtype}, lens {lens})")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_right_padding_is_free_forward_bitwise(dtype):
    B, S, H, Hkv, hd = 3, 1000, 4, 4, 64
    lens = [1000, 700, 31]
    a = _draw(B, S, H, Hkv, hd, dtype, 47, lens, pad=0.25)  # finite padding
    rag = _gpu(a, dtype, lens, backward=False)
    plain = _gpu(a, dtype, None, backward=False)
    for b, n in enumerate(lens):
        for name in ("o", "lse"):
            assert np.array_equal(rag[name][b, :, :n], plain[name][b, :, :n]), \
                f"{dtype} length {n}: {name} of real rows differs from the padded run"
    Hh.log(f"  right padding free, forward bitwise ({dtype})")


def test_bench_workload():
    """The length mix the benchmark times (8 x 2048, 16 heads of 64, bf16): the
    shortest and longest sequences equal their own plain runs bitwise, and one
    head of the shortest matches the oracle."""
    rw = inputs.RAGGED_BENCH
    lens = rw.lens()
    a = inputs.generate(rw.B, rw.S, rw.H, rw.Hkv, rw.hd, rw.seed, shaped=True, dtype=rw.dtype)
    Hh.log(f"ragged bench workload {rw.name} lens={lens}")
    g = _gpu(a, rw.dtype, lens)
    for b in (int(np.argmin(lens)), int(np.argmax(lens))):
        n = lens[b]
        one = _gpu({k: np.ascontiguousarray(x[b:b + 1, :, :n]) for k, x in a.items()}, rw.dtype)
        for name in NAMES:
            assert np.array_equal(g[name][b:b + 1, :, :n], one[name]), f"length {n}: {name}"
        for name in ("o", "dq"):
            assert np.all(g[name][b, :, n:] == 0.0)
    b = int(np.argmin(lens))
    n = lens[b]
    ref = default().run(a["q"][b:b + 1, :1, :n], a["k"][b:b + 1, :1, :n], a["v"][b:b + 1, :1, :n],
                        a["dO"][b:b + 1, :1, :n])
    tau = Hh.TAU[rw.dtype]
    for name in NAMES:
        gx = g[name][b:b + 1, :1, :n]
        err, den = float(np.max(np.abs(gx - ref[name]))), float(np.max(np.abs(ref[name])))
        assert err <= tau * den, f"{name}: {err:.3e} > {tau} * {den:.3e}"

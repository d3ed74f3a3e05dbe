"""The per-element bf16 allowance of the GPU parity tests (gpu_helpers.
bf16_backward_allowance) is neither too small nor vacuous: on the rising-score
inputs, a float64 replay of the bf16 backward's roundings (D from the bf16 o,
dS and P rounded to bf16 before their products) falls inside it, while
plausible kernel mistakes do not.  CPU only."""
import numpy as np
import pytest

import gpu_helpers as H
from bwd_head_rms_amd import inputs
from oracle import default
from test_parity_gpu import rising_scores_inputs


def bf16_replay(arrs, ref, scale):
    """dq, dk, dv with the bf16 path's roundings applied to exact values."""
    q, k, v, dO = (arrs[n].astype(np.float64) for n in ("q", "k", "v", "dO"))
    r16 = lambda x: inputs.bf16_round(np.asarray(x, np.float32)).astype(np.float64)
    o16 = r16(ref["o"])
    B, Hq, S, hd = q.shape
    group = Hq // k.shape[1]
    mask = np.tril(np.ones((S, S), bool))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(Hq):
            kv, vv = k[b, h // group], v[b, h // group]
            P = np.where(mask, np.exp(scale * (q[b, h] @ kv.T) - ref["lse"][b, h][:, None]), 0.0)
            D = np.sum(dO[b, h] * o16[b, h], axis=1)
            dS = r16(P * (dO[b, h] @ vv.T - D[:, None]))
            dq[b, h] = scale * dS @ kv
            dk[b, h // group] += scale * dS.T @ q[b, h]
            dv[b, h // group] += r16(P).T @ dO[b, h]
    return {"dq": dq, "dk": dk, "dv": dv}, o16


@pytest.fixture(scope="module")
def case():
    arrs, scale = rising_scores_inputs("bf16")
    ref = default().run(arrs["q"], arrs["k"], arrs["v"], arrs["dO"], scale=scale)
    sim, o16 = bf16_replay(arrs, ref, scale)
    allow = H.bf16_backward_allowance(arrs, ref, o16, scale)
    return arrs, scale, ref, sim, allow


def test_replayed_bf16_roundings_fall_inside_the_allowance(case):
    arrs, scale, ref, sim, allow = case
    # without the allowance the replay exceeds the plain bf16 bound (the reason it exists)
    with pytest.raises(AssertionError):
        H.compare(sim, ref, "bf16", "replay, plain bound", names=("dq",))
    H.compare(sim, ref, "bf16", "replay", names=("dq", "dk", "dv"), allow=allow,
              terms=H.term_sizes(arrs, scale))


@pytest.mark.parametrize("mistake", ["dq_row_sign", "dk_one_head", "dv_unnormalised",
                                     "dq_scale_dropped", "dk_row_shift"])
def test_planted_mistakes_exceed_the_allowance(case, mistake):
    arrs, scale, ref, sim, allow = case
    bad = {n: a.copy() for n, a in sim.items()}
    if mistake == "dq_row_sign":        # one rising row's dS with the wrong sign
        bad["dq"][0, 0, 200] *= -1
    elif mistake == "dk_one_head":      # group sum over the first query head only
        bad["dk"] = bf16_replay({**arrs, "q": arrs["q"][:, :1], "dO": arrs["dO"][:, :1]},
                                {n: ref[n][:, :1] for n in ("o", "lse")}, scale)[0]["dk"]
    elif mistake == "dv_unnormalised":  # probabilities 5% too large
        bad["dv"] *= 1.05
    elif mistake == "dq_scale_dropped":
        bad["dq"] /= scale
    elif mistake == "dk_row_shift":     # dk written one key row off
        bad["dk"] = np.roll(bad["dk"], 1, axis=2)
    with pytest.raises(AssertionError):
        H.compare(bad, ref, "bf16", f"planted {mistake}", names=("dq", "dk", "dv"), allow=allow,
                  terms=H.term_sizes(arrs, scale))

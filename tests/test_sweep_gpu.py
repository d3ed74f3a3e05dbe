"""Seeded random shapes against the fp64 oracle (GPU, through the C ABI).

Sixteen shapes drawn from a fixed generator: batch 1-4, sequence length 1-700,
head dimension 16/32/64, GQA groups 1, 2, 3, 4, 5, 6 or 8 over 1-3 kv heads,
fp32 or bf16, and in about half the cases right-padded batches with random
lengths in 0..S (NaN in every padding input).  They reach the
combinations the hand-picked edge shapes do not name: odd lengths with every
group size, the group split of the dk/dv kernel at odd sizes, ragged GQA.
Tolerance as for every attention output: max|err| <= tau * max|ref| with tau =
1e-4 (fp32) or 2e-2 (bf16), padding rows exactly zero (lse -inf).
"""
import numpy as np
import pytest

import gpu_helpers as Hh
from bwd_head_rms_amd import inputs
from oracle import default
from test_ragged_gpu import _check_oracle

pytestmark = pytest.mark.gpu

N_CASES = 16


def _shape(i):
    rng = np.random.default_rng(1005 + i)
    for _ in range(100):
        B = int(rng.integers(1, 5))
        S = int(rng.integers(1, 701))
        hd = int(rng.choice([16, 32, 64]))
        group = int(rng.choice([1, 2, 3, 4, 5, 6, 8]))
        Hkv = int(rng.integers(1, 4))
        H = group * Hkv
        if B * H * S * S <= 3_000_000:  # keeps the oracle to a few seconds
            break
    dtype = "bf16" if rng.random() < 0.5 else "f32"
    lens = None
    if rng.random() < 0.5:
        lens = [int(x) for x in rng.integers(0, S + 1, size=B)]
        if B > 1:
            lens[int(rng.integers(0, B))] = S  # one full sequence
    return B, S, H, Hkv, hd, dtype, lens


@pytest.mark.parametrize("i", range(N_CASES),
                         ids=lambda i: "B{}_S{}_H{}_Hkv{}_hd{}_{}_{}".format(
                             *_shape(i)[:6], "ragged" if _shape(i)[6] else "plain"))
def test_random_shape(i):
    B, S, H, Hkv, hd, dtype, lens = _shape(i)
    Hh.log(f"sweep {i}: B{B} S{S} H{H}/{Hkv} hd{hd} {dtype} lens={lens}")
    if lens is not None:
        _check_oracle(B, S, H, Hkv, hd, dtype, lens, seed=500 + i)
        return
    arrs = inputs.generate(B, S, H, Hkv, hd, seed=500 + i, shaped=True, dtype=dtype)
    scale = 1.0 / np.sqrt(hd)
    gpu = Hh.gpu_run(arrs, dtype, scale)
    r = default().run(arrs["q"], arrs["k"], arrs["v"], arrs["dO"], scale=scale)
    Hh.compare(gpu, r, dtype, f"sweep {i}", terms=Hh.term_sizes(arrs, scale))

"""The single-kernel backward for short bf16 sequences (S <= 256, hd <= 32, one
query head per kv head; xattn_bwd_kernel_count == 1):

* bitwise equal to the dq and dk/dv kernel pair (xattn_bwd_dq, then
  xattn_bwd_dkdv) on the same inputs, across full and partial 32-row blocks,
  S = 1, both head dimensions and the largest S the kernel takes;
* within the bf16 parity tolerance of the fp64 oracle on right-padded batches
  (xattn_bwd_ragged), with NaN in every padding input and exact zeros in the
  padding rows of dq, dk, dv;
* a ragged batch bitwise equal to each sequence run alone.
The full-size dim384 bf16 workload takes this kernel too and is checked against
the oracle by the plain parity tests."""
import numpy as np
import pytest

import gpu_helpers as Hh
from bwd_head_rms_amd import inputs
from test_ragged_gpu import _check_oracle, _draw, _gpu

pytestmark = pytest.mark.gpu

SHAPES = [  # B, S, H, hd
    (2, 256, 3, 32),
    (3, 100, 2, 16),
    (1, 1, 1, 32),
    (2, 33, 2, 32),
    (1, 255, 2, 16),
    (4, 64, 1, 32),
    (2, 200, 2, 16),
    # 256 CUs hold two workgroups each: below 512 heads some heads are split
    # into a key-side and a query-side workgroup (all of them below 256 heads)
    (48, 96, 8, 32),   # 384 heads: 256 whole, 128 split
    (64, 64, 8, 16),   # 512 heads: none split
]


def _pair_and_single(B, S, H, hd, seed):
    import torch
    from bwd_head_rms_amd import _lib, api
    L = _lib.lib()
    assert L.xattn_bwd_kernel_count(B, S, H, H, hd, _lib.BF16) == 1
    a = inputs.generate(B, S, H, H, hd, seed, shaped=True, dtype="bf16")
    t = Hh.to_dev(a, "bf16")
    o, lse = api.fwd(t["q"], t["k"], t["v"])
    scale = 1.0 / np.sqrt(hd)
    single = api.bwd(t["q"], t["k"], t["v"], o, lse, t["dO"], scale)
    f32 = dict(dtype=torch.float32, device="cuda")
    dq = torch.full(t["q"].shape, float("nan"), **f32)
    dk = torch.full(t["k"].shape, float("nan"), **f32)
    dv = torch.full(t["k"].shape, float("nan"), **f32)
    wsb = int(L.xattn_bwd_workspace_bytes(B, S, H, H, hd, _lib.BF16))
    ws = torch.empty(wsb // 4, **f32)
    st = torch.cuda.current_stream().cuda_stream
    dims = (B, S, H, H, hd, scale, _lib.BF16)
    _lib.check(L.xattn_bwd_dq(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), o.data_ptr(),
                              lse.data_ptr(), t["dO"].data_ptr(), dq.data_ptr(), *dims,
                              ws.data_ptr(), wsb, st))
    _lib.check(L.xattn_bwd_dkdv(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(),
                                lse.data_ptr(), t["dO"].data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                *dims, ws.data_ptr(), wsb, st))
    torch.cuda.synchronize()
    return single, (dq, dk, dv)


@pytest.mark.parametrize("shape", SHAPES, ids=[f"B{b}_S{s}_H{h}_hd{d}" for b, s, h, d in SHAPES])
def test_single_kernel_equals_pair_bitwise(shape):
    import torch
    B, S, H, hd = shape
    Hh.log(f"short backward vs kernel pair B{B} S{S} H{H} hd{hd}")
    single, pair = _pair_and_single(B, S, H, hd, seed=60 + S)
    for name, x, y in zip(("dq", "dk", "dv"), single, pair):
        assert torch.isfinite(x).all(), f"{name}: non-finite"
        assert torch.equal(x, y), f"{name}: single kernel differs from the dq + dk/dv pair"


@pytest.mark.parametrize("hd", [16, 32])
def test_ragged_against_oracle(hd):
    _check_oracle(5, 256, 3, 3, hd, "bf16", [256, 1, 0, 129, 200], seed=70 + hd)


def test_ragged_partial_blocks_against_oracle():
    _check_oracle(4, 100, 2, 2, 16, "bf16", [100, 31, 32, 33], seed=72)


def test_ragged_batched_equals_looped_bitwise():
    B, S, H, hd = 4, 256, 2, 32
    lens = [256, 161, 32, 5]
    a = _draw(B, S, H, H, hd, "bf16", 73, lens, pad=np.nan)
    g = _gpu(a, "bf16", lens)
    for b, n in enumerate(lens):
        one = _gpu({k: np.ascontiguousarray(x[b:b + 1, :, :n]) for k, x in a.items()}, "bf16")
        for name in ("o", "lse", "dq", "dk", "dv"):
            assert np.array_equal(g[name][b:b + 1, :, :n], one[name]), \
                f"sequence {b} (length {n}): {name} differs from its own run"
    Hh.log(f"  short ragged batched == looped bitwise (lens {lens})")

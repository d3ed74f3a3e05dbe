"""The allocation-free backward entry point (xattn_bwd_noalloc), called
through the C ABI, against the existing entry point (xattn_bwd) on the same
inputs: two calls in a row, the second on a smaller input (the fixed scratch
keeps the first call's contents); a grouped-query shape that xattn_bwd splits
over workgroups (the no-alloc path keeps groups whole: a different but fixed
summation order, so the tolerance bound applies there); a shape beyond the
scratch limit is refused before anything runs; and no device memory is
allocated across calls."""
import ctypes

import numpy as np
import pytest

import gpu_helpers as H
from bwd_head_rms_amd import inputs

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _run_both(B, S, Hq, Hkv, hd, dtype, seed):
    """(xattn_bwd outputs, xattn_bwd_noalloc outputs) as float64 numpy, plus
    the shape's split factor in xattn_bwd."""
    import torch
    from bwd_head_rms_amd import _lib, api
    L = _lib.lib()
    arrs = inputs.generate(B, S, Hq, Hkv, hd, seed=seed, shaped=True, dtype=dtype)
    t = H.to_dev(arrs, dtype)
    scale = 1.0 / np.sqrt(hd)
    code = _lib.BF16 if dtype == "bf16" else _lib.F32
    o, lse = api.fwd(t["q"], t["k"], t["v"], scale)
    f32 = dict(dtype=torch.float32, device="cuda")
    ref = [torch.full(s, float("nan"), **f32) for s in ((B, Hq, S, hd), (B, Hkv, S, hd), (B, Hkv, S, hd))]
    out = [torch.full(s, float("nan"), **f32) for s in ((B, Hq, S, hd), (B, Hkv, S, hd), (B, Hkv, S, hd))]
    need = L.xattn_bwd_workspace_bytes(B, S, Hq, Hkv, hd, code)
    ws = torch.empty((need // 4,), **f32)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    args = [_ptr(x) for x in (t["q"], t["k"], t["v"], o, lse, t["dO"])]
    _lib.check(L.xattn_bwd(*args, *[_ptr(x) for x in ref], B, S, Hq, Hkv, hd, scale, code,
                           _ptr(ws), need, st))
    _lib.check(L.xattn_bwd_noalloc(*args, *[_ptr(x) for x in out], B, S, Hq, Hkv, hd, scale, code,
                                   st))
    torch.cuda.synchronize()
    split = need > 8 * B * Hq * S
    as_np = lambda xs: {n: x.cpu().double().numpy() for n, x in zip(("dq", "dk", "dv"), xs)}
    return as_np(ref), as_np(out), split


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_bwd_two_calls_in_a_row(order):
    # the long-context workload's shape, then a smaller ragged one: the second
    # call runs on scratch that still holds the first call's values
    # (the second shape has few key tiles, so xattn_bwd splits its GQA groups)
    for shape, seed in (((4, 2048, 16, 16, 64, "bf16"), 5), ((2, 300, 6, 2, 32, "f32"), 9)):
        H.log(f"noalloc vs bwd {shape}")
        ref, out, split = _run_both(*shape, seed)
        for n in ("dq", "dk", "dv"):
            assert np.all(np.isfinite(out[n])), n
        H.compare(out, ref, shape[-1], f"noalloc {shape}", names=("dq", "dk", "dv"))
        # dq comes from the same kernel on the same values either way; dk, dv
        # too unless xattn_bwd split the groups (another fixed summation order)
        for n in (("dq",) if split else ("dq", "dk", "dv")):
            assert np.array_equal(out[n], ref[n]), f"{shape} {n} differs from xattn_bwd"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_gqa_group_kept_whole(dtype):
    shape = (16, 1024, 8, 2, 64, dtype)
    H.log(f"noalloc vs bwd (split there) {shape}")
    ref, out, split = _run_both(*shape, 4)
    assert split, "expected xattn_bwd to split this shape's groups"
    H.compare(out, ref, dtype, f"noalloc GQA {dtype}", names=("dq", "dk", "dv"))
    assert np.array_equal(out["dq"], ref["dq"])  # dq does not depend on the split


def test_noalloc_refuses_shapes_beyond_its_scratch():
    import torch
    from bwd_head_rms_amd import _lib
    L = _lib.lib()
    # 8 * B * H * S = 8 * 1 * 16 * 131073 bytes > 16 MiB; tensors of that shape are
    # not needed: validation fails before any pointer is used, so small buffers do
    x = torch.zeros(64, dtype=torch.float32, device="cuda")
    p = _ptr(x)
    rc = L.xattn_bwd_noalloc(p, p, p, p, p, p, p, p, p, 1, 131073, 16, 16, 64, 0.125, _lib.BF16,
                             ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    assert rc == 11, _lib.strerror(rc)
    assert "noalloc" in _lib.strerror(rc)
    assert torch.count_nonzero(x).item() == 0
    # exactly at the limit: accepted shape sizes are checked, not enqueued here
    assert L.xattn_bwd_workspace_bytes(1, 131072, 16, 16, 64, _lib.BF16) == 16 << 20


def test_noalloc_allocates_nothing():
    import torch
    from bwd_head_rms_amd import api
    B, S, Hq, Hkv, hd = 2, 700, 4, 2, 64
    a = inputs.generate(B, S, Hq, Hkv, hd, seed=12, dtype="bf16")
    t = H.to_dev(a, "bf16")
    o, lse = api.fwd(t["q"], t["k"], t["v"])
    f32 = dict(dtype=torch.float32, device="cuda")
    dq = torch.empty((B, Hq, S, hd), **f32)
    dk, dv = (torch.empty((B, Hkv, S, hd), **f32) for _ in range(2))
    api.bwd_noalloc(t["q"], t["k"], t["v"], o, lse, t["dO"], 0.125, dq, dk, dv)
    torch.cuda.synchronize()
    free0, alloc0 = torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated()
    for _ in range(5):
        api.bwd_noalloc(t["q"], t["k"], t["v"], o, lse, t["dO"], 0.125, dq, dk, dv)
    torch.cuda.synchronize()
    free1, alloc1 = torch.cuda.mem_get_info()[0], torch.cuda.memory_allocated()
    H.log(f"  free {free0} -> {free1}, torch allocated {alloc0} -> {alloc1}")
    assert free1 == free0 and alloc1 == alloc0

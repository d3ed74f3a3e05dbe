"""GPU invariants of the HIP path that hold exactly or to tolerance at any size:
determinism, batch independence, causality, GQA == repeated-K/V MHA, V = 1,
key-shift invariance, gradient identities, and the autograd wrapper."""
import numpy as np
import pytest

import gpu_helpers as H
from bwd_head_rms_amd import inputs

pytestmark = pytest.mark.gpu


def _gen(B, S, Hq, Hkv, hd, dtype, seed=5):
    return inputs.generate(B, S, Hq, Hkv, hd, seed=seed, shaped=True, dtype=dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_run_to_run_bitwise(dtype):
    arrs = _gen(2, 700, 4, 2, 64, dtype)
    a = H.gpu_run(arrs, dtype)
    b = H.gpu_run(arrs, dtype)
    for n in H.NAMES:
        assert np.array_equal(a[n], b[n]), f"{n} differs between identical runs"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_batch_independence_bitwise(dtype):
    arrs = _gen(3, 333, 4, 2, 32, dtype)
    full = H.gpu_run(arrs, dtype)
    for b in range(3):
        one = H.gpu_run({n: a[b:b + 1] for n, a in arrs.items()}, dtype)
        for n in H.NAMES:
            assert np.array_equal(full[n][b:b + 1], one[n]), f"batch entry {b}: {n} differs"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_causality_bitwise(dtype):
    """Changing q, k, v, dO at positions >= t leaves rows < t of o, lse, dq bitwise equal."""
    S, t = 517, 200
    arrs = _gen(2, S, 4, 2, 64, dtype)
    base = H.gpu_run(arrs, dtype)
    rng = np.random.default_rng(9)
    pert = {}
    for n, a in arrs.items():
        a = a.copy()
        a[:, :, t:] = rng.standard_normal(a[:, :, t:].shape).astype(np.float32)
        pert[n] = inputs.bf16_round(a) if dtype == "bf16" else a
    p = H.gpu_run(pert, dtype)
    for n in ("o", "lse", "dq"):
        assert np.array_equal(p[n][:, :, :t], base[n][:, :, :t]), f"{n} rows < t changed"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gqa_equals_repeated_mha(dtype):
    B, S, Hq, Hkv, hd = 2, 300, 8, 2, 64
    group = Hq // Hkv
    arrs = _gen(B, S, Hq, Hkv, hd, dtype)
    gqa = H.gpu_run(arrs, dtype)
    rep = dict(arrs)
    rep["k"] = np.repeat(arrs["k"], group, axis=1)
    rep["v"] = np.repeat(arrs["v"], group, axis=1)
    mha = H.gpu_run(rep, dtype)
    for n in ("o", "lse", "dq"):
        assert np.array_equal(gqa[n], mha[n]), f"GQA {n} differs from repeated-K/V MHA"
    for n in ("dk", "dv"):
        summed = sum(mha[n][:, [g * group + r for g in range(Hkv)]] for r in range(group))
        err = np.max(np.abs(gqa[n] - summed))
        assert err <= 1e-5 * np.max(np.abs(summed)), f"GQA {n} != group sum of MHA ({err})"
        # this shape has few kv tiles, so each query head of a group takes its
        # own workgroup: the partials are the MHA heads' gradients bit for bit
        # and the group sum adds them in fp32 in ascending head order
        heads = [mha[n][:, [g * group + r for g in range(Hkv)]].astype(np.float32)
                 for r in range(group)]
        exact = heads[0]
        for x in heads[1:]:
            exact = exact + x
        assert np.array_equal(gqa[n].astype(np.float32), exact), f"GQA {n}: split sum order"


def test_group_one_is_mha_bitwise():
    """Hkv = H (group 1) goes through the same kernels as MHA; the same inputs
    viewed as MHA give the same bits (the group-sum of one term is the term)."""
    arrs = _gen(1, 260, 3, 3, 32, "f32")
    a = H.gpu_run(arrs, "f32")
    b = H.gpu_run({n: x.copy() for n, x in arrs.items()}, "f32")
    for n in H.NAMES:
        assert np.array_equal(a[n], b[n])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_constant_values_give_constant_output(dtype):
    arrs = _gen(1, 400, 2, 2, 64, dtype)
    arrs["v"] = np.ones_like(arrs["v"])
    out = H.gpu_run(arrs, dtype)
    tau = H.TAU[dtype]  # the parity tolerance, relative to max|o| = 1
    assert np.max(np.abs(out["o"] - 1.0)) <= tau
    # dq = 0 exactly in real arithmetic; bound it by tau times one summand's size
    assert np.max(np.abs(out["dq"])) <= tau * H.term_sizes(arrs, 1.0 / np.sqrt(64))["dq"]


def test_key_shift_invariance_f32():
    """k_j -> k_j + u: o unchanged, lse shifted by scale*q_i.u; the shift makes
    scores exceed the fp32 exp() range, so it also checks max subtraction."""
    B, S, Hq, Hkv, hd = 1, 300, 2, 2, 32
    arrs = _gen(B, S, Hq, Hkv, hd, "f32")
    scale = 1.0 / np.sqrt(hd)
    arrs["q"][..., 0] = 1.0 + 0.1 * np.abs(arrs["q"][..., 0])
    u = np.zeros(hd, dtype=np.float32)
    u[0] = 120.0 / scale
    base = H.gpu_run(arrs, "f32", scale)
    sh = dict(arrs)
    sh["k"] = (arrs["k"] + u).astype(np.float32)
    out = H.gpu_run(sh, "f32", scale)
    assert np.max(np.abs(out["o"] - base["o"])) <= 1e-3 * np.max(np.abs(base["o"]))
    shift = scale * np.einsum("bhsd,d->bhs", arrs["q"].astype(np.float64), u.astype(np.float64))
    assert np.max(np.abs(out["lse"] - shift - base["lse"])) <= 1e-4 * np.max(np.abs(out["lse"]))
    for n in ("dq", "dv"):
        assert np.max(np.abs(out[n] - base[n])) <= 2e-3 * np.max(np.abs(base[n])), n


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gradient_identities(dtype):
    B, S, Hq, Hkv, hd = 2, 256, 6, 2, 32
    group = Hq // Hkv
    arrs = _gen(B, S, Hq, Hkv, hd, dtype)
    out = H.gpu_run(arrs, dtype)
    q, k, dO = (arrs[n].astype(np.float64) for n in ("q", "k", "dO"))
    tau = H.TAU[dtype]
    for b in range(B):
        for g in range(Hkv):
            hs = slice(g * group, (g + 1) * group)
            lhs = out["dv"][b, g].sum(axis=0)
            rhs = dO[b, hs].sum(axis=(0, 1))
            assert np.max(np.abs(lhs - rhs)) <= tau * np.max(np.abs(rhs)) + 1e-4
            qd = float(np.sum(q[b, hs] * out["dq"][b, hs]))
            kd = float(np.sum(k[b, g] * out["dk"][b, g]))
            mag = float(np.sum(np.abs(q[b, hs] * out["dq"][b, hs])))
            assert abs(qd - kd) <= tau * mag


def test_autograd_wrapper_matches_direct_calls():
    import torch
    from bwd_head_rms_amd import api
    arrs = _gen(1, 96, 4, 2, 32, "f32")
    t = H.to_dev(arrs, "f32")
    q, k, v = (t[n].clone().requires_grad_(True) for n in ("q", "k", "v"))
    o = api.causal_attention(q, k, v)
    o.backward(t["dO"])
    o2, lse = api.fwd(t["q"], t["k"], t["v"])
    dq, dk, dv = api.bwd(t["q"], t["k"], t["v"], o2, lse, t["dO"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    assert torch.equal(q.grad, dq) and torch.equal(k.grad, dk) and torch.equal(v.grad, dv)


def test_outputs_fully_overwritten():
    """Outputs are overwritten, not accumulated: garbage in the output buffers
    does not leak into the results."""
    import torch
    from bwd_head_rms_amd import api
    arrs = _gen(1, 130, 2, 1, 64, "bf16")
    t = H.to_dev(arrs, "bf16")
    o1, l1 = api.fwd(t["q"], t["k"], t["v"])
    g1 = api.bwd(t["q"], t["k"], t["v"], o1, l1, t["dO"])
    fill = lambda x: x.fill_(float("nan"))  # noqa: E731
    o2 = fill(torch.empty_like(o1))
    l2 = fill(torch.empty_like(l1))
    api.fwd(t["q"], t["k"], t["v"], o=o2, lse=l2)
    # a group of 2 over few kv tiles: the workspace also holds partial dk, dv
    ws = fill(torch.empty(api.workspace_bytes(1, 130, 2, 1, 64, 1) // 4, dtype=torch.float32,
                          device="cuda"))
    g2 = [fill(torch.empty_like(x)) for x in g1]
    api.bwd(t["q"], t["k"], t["v"], o1, l1, t["dO"], dq=g2[0], dk=g2[1], dv=g2[2], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype,S,hd", [("bf16", 130, 64), ("bf16", 100, 32), ("bf16", 77, 16),
                                        ("f32", 130, 64)])
def test_no_reads_past_input_ends(dtype, S, hd):
    """Every input tensor is followed in memory by NaN: the kernels must never
    read past the end of a (batch, head) plane (the tail tile of a ragged
    sequence included), so the results equal those of ordinary allocations."""
    import torch
    from bwd_head_rms_amd import api
    arrs = _gen(1, S, 4, 2, hd, dtype)
    t = H.to_dev(arrs, dtype)

    def guarded(x):
        buf = torch.full((x.numel() + 8192,), float("nan"), dtype=x.dtype, device=x.device)
        buf[: x.numel()].copy_(x.reshape(-1))
        return buf[: x.numel()].view(x.shape)

    g = {n: guarded(x) for n, x in t.items()}
    o1, l1 = api.fwd(t["q"], t["k"], t["v"])
    r1 = api.bwd(t["q"], t["k"], t["v"], o1, l1, t["dO"])
    o2, l2 = api.fwd(g["q"], g["k"], g["v"])
    r2 = api.bwd(g["q"], g["k"], g["v"], guarded(o1), guarded(l1), g["dO"])
    torch.cuda.synchronize()
    for a, b in zip((o1, l1, *r1), (o2, l2, *r2)):
        assert torch.isfinite(b.float()).all()
        assert torch.equal(a, b)

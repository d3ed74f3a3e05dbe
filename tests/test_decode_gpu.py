"""GPU parity of decode attention (xattn_decode through the C ABI) against its
fp64 oracle on the same seeded inputs.

Tolerance per output X in {o, lse}: max|X_gpu - X_ref| <= tau * max|X_ref| with
tau = 1e-4 for fp32 inputs and 2e-2 for bf16 inputs (the bar of the attention
path); an empty sequence must give o = 0 and lse = -inf exactly.  Cases: the
last query row of the attention workloads against their whole K/V (decode
equals the last row of causal attention there), every head dimension and dtype,
GQA groups that take each heads-per-workgroup variant (1, 2, 4, 8 and two passes
of 8), caches of one chunk and of many (the split and merge path), ragged
lengths on chunk boundaries with NaN beyond each length (never read), empty
sequences, the full-size cache the benchmark times on sampled rows, and the
longest cache accepted (4096 chunks).  The result is also checked bitwise run
to run.
"""
import numpy as np
import pytest

import gpu_helpers as Hh
from bwd_head_rms_amd import inputs
from oracle import default_decode

pytestmark = pytest.mark.gpu


def _gpu(arrs, dtype, lens=None, scale=None):
    import torch
    from bwd_head_rms_amd import api
    t = {n: inputs.to_torch(a, dtype, "cuda") for n, a in arrs.items()}
    tl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = api.decode(t["q"], t["k"], t["v"], lens=tl, scale=scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _check(arrs, dtype, what, lens=None, scale=None, rows=None):
    """Compare with the oracle; ``rows`` = list of batch entries to check (all if None)."""
    o, lse = _gpu(arrs, dtype, lens, scale)
    assert np.all(np.isfinite(o)), f"{what}: o non-finite"
    sel = list(range(o.shape[0])) if rows is None else rows
    sub = {n: a[sel] for n, a in arrs.items()}
    ref = default_decode().decode(sub["q"], sub["k"], sub["v"],
                                  lens=None if lens is None else [lens[b] for b in sel], scale=scale)
    o, lse = o[sel], lse[sel]
    empty = np.isneginf(ref["lse"])
    assert np.array_equal(np.isneginf(lse), empty), f"{what}: lse -inf pattern differs"
    assert np.all(o[empty] == 0.0), f"{what}: empty sequence o != 0"
    tau = Hh.TAU[dtype]
    msg = []
    for n, a, r in (("o", o, ref["o"]), ("lse", lse[~empty], ref["lse"][~empty])):
        if r.size == 0:
            continue
        err, den = float(np.max(np.abs(a - r))), float(np.max(np.abs(r)))
        msg.append(f"{n}={err / den:.2e}")
        assert err <= tau * den, f"{what} {dtype}: {n} max|err| {err:.3e} > {tau:g} * {den:.3e}"
    Hh.log(f"  {what}: " + " ".join(msg))


def _rand(B, T, H, Hkv, hd, dtype, seed):
    rng = np.random.default_rng(seed)
    a = {"q": rng.standard_normal((B, H, hd), dtype=np.float32),
         "k": rng.standard_normal((B, Hkv, T, hd), dtype=np.float32),
         "v": rng.standard_normal((B, Hkv, T, hd), dtype=np.float32)}
    if dtype == "bf16":
        a = {n: inputs.bf16_round(x) for n, x in a.items()}
    return a


@pytest.mark.parametrize("name", [n for n, w in inputs.DECODE_WORKLOADS.items() if w.source])
def test_last_row_of_attention_workloads(name):
    w = inputs.DECODE_WORKLOADS[name]
    Hh.log(f"decode {name}")
    _check(inputs.generate_decode(w), w.dtype, name)


def test_full_size_cache_sampled_rows():
    w = inputs.DECODE_WORKLOADS[inputs.DECODE_BENCH]
    Hh.log(f"decode {w.name} (sampled batch entries)")
    _check(inputs.generate_decode(w), w.dtype, w.name, rows=[0, 3, w.B - 1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hd", [16, 32, 64])
@pytest.mark.parametrize("T", [1, 7, 128, 129, 3000])
def test_head_dims_and_lengths(hd, T, dtype):
    Hh.log(f"decode hd={hd} T={T} {dtype}")
    _check(_rand(3, T, 4, 2, hd, dtype, seed=hd * 7919 + T), dtype, f"hd{hd} T{T}")


@pytest.mark.parametrize("H,Hkv", [(3, 3), (6, 2), (6, 1), (12, 3), (8, 1), (32, 2), (5, 5)])
def test_gqa_groups(H, Hkv):
    Hh.log(f"decode GQA H={H} Hkv={Hkv}")
    for dtype in ("f32", "bf16"):
        _check(_rand(2, 777, H, Hkv, 64, dtype, seed=H * 31 + Hkv), dtype, f"H{H}/{Hkv} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_lengths_and_empty_sequences(dtype):
    B, T, H, Hkv, hd = 8, 2500, 4, 2, 32
    lens = [2500, 1, 0, 1024, 1025, 127, 128, 0]
    a = _rand(B, T, H, Hkv, hd, dtype, seed=99)
    for b, n in enumerate(lens):  # nothing past a sequence's length may be read
        a["k"][b, :, n:] = np.nan
        a["v"][b, :, n:] = np.nan
    Hh.log(f"decode ragged {lens} {dtype}")
    _check(a, dtype, "ragged", lens=lens)


def test_one_chunk_and_many_chunks_agree_with_scale():
    a = _rand(2, 5000, 8, 2, 16, "f32", seed=5)
    _check(a, "f32", "scale 0.05", scale=0.05)
    _check(a, "f32", "scale 2.0", scale=2.0)


def test_bitwise_run_to_run():
    a = _rand(4, 4100, 8, 2, 64, "bf16", seed=11)
    o1, l1 = _gpu(a, "bf16")
    o2, l2 = _gpu(a, "bf16")
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_longest_cache():
    """The longest cache decode accepts (4194304 positions: 4096 chunks of 1024,
    the merge kernel's limit), hd 16 bf16, one sequence; a shorter length on a
    second sequence exercises a partly filled chunk list."""
    T = 1 << 22
    B, H, Hkv, hd = 2, 2, 1, 16
    rng = np.random.default_rng(2024)
    a = {"q": rng.standard_normal((B, H, hd), dtype=np.float32),
         "k": rng.standard_normal((B, Hkv, T, hd), dtype=np.float32),
         "v": rng.standard_normal((B, Hkv, T, hd), dtype=np.float32)}
    a = {n: inputs.bf16_round(x) for n, x in a.items()}
    Hh.log(f"decode longest cache T={T}")
    _check(a, "bf16", "T=2^22", lens=[T, 3 * T // 4 + 5])


def test_lengths_are_clamped():
    """Lengths past the capacity act as T, negative ones as 0 (empty)."""
    T = 600
    a = _rand(3, T, 4, 2, 32, "f32", seed=12)
    o, lse = _gpu(a, "f32", lens=[T + 77, -3, 250])
    o_ref, lse_ref = _gpu(a, "f32", lens=[T, 0, 250])
    assert np.array_equal(o, o_ref) and np.array_equal(lse, lse_ref)
    _check(a, "f32", "clamped lengths", lens=[T, 0, 250])

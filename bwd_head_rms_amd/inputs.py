"""Seeded synthetic inputs for causal attention (shared by tests, smoke and bench).

This module holds no attention arithmetic.  It only draws the tensors that both
the HIP path and the CPU oracle consume, shaped like the activations the pages'
decoder feeds into attention:

* Q, K, V, dO are drawn i.i.d. N(0, 1) in float32, in that order, from
  ``numpy.random.default_rng(seed)``.
* For the model-shaped workloads, Q and K then get the per-head RMS norm the
  pages add before attention ("xtrain evolution overview", infra table row T9:
  Qwen3-style per-head QK-norm; unit weight, eps 1e-6 here) and rotary position
  embedding with the position reset per sequence ("xtrain -- Known Issues & Perf
  Backlog", KI-1 fix: position = row mod S in the flattened [B*S] rows, which in
  BHSD layout is simply the sequence index).  RoPE uses base 10000 and the
  half-split pairing (d, d + hd/2), theta_k = 10000^(-2k/hd); the pages print no
  formula, so this is the common Qwen3/HF convention.  Shaping is done in float64
  and cast to float32.
* bf16 workloads use round-to-nearest-even copies of the float32 draw.

Configurations are named by what they are: the tiny checkable case, the dim384
model's attention (B16, S256, 12 heads of 32), the same at B32 in bf16, the GQA
case (8 query heads over 2 kv heads, hd 64, S1024) and the long-context case
(B4, S2048, 16 heads of 64).
"""
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    S: int
    H: int
    Hkv: int
    hd: int
    dtype: str          # "f32" or "bf16": dtype of q, k, v, o, dO
    shaped: bool        # per-head RMS QK-norm + RoPE on Q and K
    seed: int

    @property
    def scale(self):
        return 1.0 / float(np.sqrt(self.hd))

    @property
    def group(self):
        return self.H // self.Hkv

    def describe(self):
        return (f"{self.name}: B={self.B} S={self.S} H={self.H} Hkv={self.Hkv} "
                f"hd={self.hd} {self.dtype}")


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_b1_s16_h2_hd16_f32", 1, 16, 2, 2, 16, "f32", False, 1),
        Workload("dim384_b16_s256_h12_hd32_f32", 16, 256, 12, 12, 32, "f32", True, 2),
        Workload("dim384_b32_s256_h12_hd32_bf16", 32, 256, 12, 12, 32, "bf16", True, 3),
        Workload("gqa_b16_s1024_h8_kv2_hd64_f32", 16, 1024, 8, 2, 64, "f32", True, 4),
        Workload("gqa_b16_s1024_h8_kv2_hd64_bf16", 16, 1024, 8, 2, 64, "bf16", True, 4),
        Workload("long_b4_s2048_h16_hd64_bf16", 4, 2048, 16, 16, 64, "bf16", True, 5),
    ]
}

# The headline long-context workload the benchmark times.
LONG_CONTEXT = "long_b4_s2048_h16_hd64_bf16"


def rms_qk_norm(x, eps=1e-6):
    """Per-head RMS norm over the last axis, unit weight, float64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x, base=10000.0):
    """Rotary embedding, half-split pairing, position = index along axis -2."""
    x = np.asarray(x, dtype=np.float64)
    S, hd = x.shape[-2], x.shape[-1]
    half = hd // 2
    inv = base ** (-2.0 * np.arange(half, dtype=np.float64) / hd)
    ang = np.arange(S, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size >= 1 << 22:  # large draws: torch's multithreaded conversion, also RNE
        import torch
        out = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        out = out.copy()
    else:
        u = x.view(np.uint32)
        # u + 0x7FFF + lsb stays below 2^32 for every non-NaN pattern (NaNs are set below)
        out = ((u + (((u >> 16) & 1) + np.uint32(0x7FFF))) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_round(x):
    """float32 values rounded to the nearest bfloat16 (returned as float32)."""
    b = bf16_bits(x)
    out = np.empty(b.shape, dtype=np.uint32)
    np.left_shift(b, 16, out=out, dtype=np.uint32)
    return out.view(np.float32)


def generate(B, S, H, Hkv, hd, seed, shaped=True, dtype="f32"):
    """Seeded inputs as float32 numpy arrays (already bf16-rounded if dtype is bf16).

    Returns dict q [B,H,S,hd], k [B,Hkv,S,hd], v [B,Hkv,S,hd], dO [B,H,S,hd].
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, S, hd), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, S, hd), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, S, hd), dtype=np.float32)
    dO = rng.standard_normal((B, H, S, hd), dtype=np.float32)
    if shaped:
        q = rope(rms_qk_norm(q)).astype(np.float32)
        k = rope(rms_qk_norm(k)).astype(np.float32)
    out = {"q": q, "k": k, "v": v, "dO": dO}
    if dtype == "bf16":
        out = {n: bf16_round(a) for n, a in out.items()}
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return out


def generate_workload(w):
    """Inputs for a named workload (see ``WORKLOADS``)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return generate(w.B, w.S, w.H, w.Hkv, w.hd, w.seed, w.shaped, w.dtype)


@dataclass(frozen=True)
class RaggedWorkload:
    """A right-padded batch: B sequences with lengths drawn uniformly from
    [min_len, S] (seeded), padded to S, in the long-context workload's head
    shape.  The pages train on variable-length sequences batched by right
    padding; this length mix stands in for their data."""
    name: str
    B: int
    S: int
    H: int
    Hkv: int
    hd: int
    dtype: str
    seed: int
    min_len: int

    @property
    def scale(self):
        return 1.0 / float(np.sqrt(self.hd))

    def lens(self):
        return [int(x) for x in
                np.random.default_rng(self.seed).integers(self.min_len, self.S + 1, self.B)]


RAGGED_BENCH = RaggedWorkload("ragged_b8_s2048_h16_hd64_bf16_len256to2048", 8, 2048, 16, 16, 64,
                              "bf16", 7, 256)


@dataclass(frozen=True)
class DecodeWorkload:
    """One decode step: a new query per (sequence, head) against a K/V cache of T
    positions.  ``source`` names the attention workload whose last query row
    and full K/V it reuses (decode equals the last row of causal attention
    there); without a source, q, k, v are drawn i.i.d. N(0, 1) (a cache too big
    for the shaping pass to be worth its time; the scores have the same spread,
    |s| ~ N(0, 1) with scale 1/sqrt(hd))."""
    name: str
    B: int
    T: int
    H: int
    Hkv: int
    hd: int
    dtype: str
    seed: int
    source: str = None

    @property
    def scale(self):
        return 1.0 / float(np.sqrt(self.hd))


DECODE_WORKLOADS = {
    w.name: w
    for w in [
        DecodeWorkload("decode_long_b4_t2048_h16_hd64_bf16", 4, 2048, 16, 16, 64, "bf16", 5,
                       "long_b4_s2048_h16_hd64_bf16"),
        DecodeWorkload("decode_gqa_b16_t1024_h8_kv2_hd64_bf16", 16, 1024, 8, 2, 64, "bf16", 4,
                       "gqa_b16_s1024_h8_kv2_hd64_bf16"),
        DecodeWorkload("decode_gqa_b16_t1024_h8_kv2_hd64_f32", 16, 1024, 8, 2, 64, "f32", 4,
                       "gqa_b16_s1024_h8_kv2_hd64_f32"),
        DecodeWorkload("decode_cache_b8_t32768_h16_kv4_hd64_bf16", 8, 32768, 16, 4, 64, "bf16", 6),
    ]
}

# The decode workload the benchmark times against the HBM roofline.
DECODE_BENCH = "decode_cache_b8_t32768_h16_kv4_hd64_bf16"


def _normal_blocks(shape, seed_seq, blocks=16):
    from concurrent.futures import ThreadPoolExecutor
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    edges = np.linspace(0, flat.size, blocks + 1).astype(np.int64)
    gens = [np.random.default_rng(s) for s in seed_seq.spawn(blocks)]

    def fill(i):
        gens[i].standard_normal(dtype=np.float32, out=flat[edges[i]:edges[i + 1]])

    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(fill, range(blocks)))
    return out


def generate_decode(w):
    """q [B,H,hd], k, v [B,Hkv,T,hd] float32 (bf16-rounded for bf16 workloads)."""
    if isinstance(w, str):
        w = DECODE_WORKLOADS[w]
    if w.source:
        a = generate_workload(w.source)
        return {"q": np.ascontiguousarray(a["q"][:, :, w.T - 1]), "k": a["k"], "v": a["v"]}
    # q, k, v from three child streams of the seed; each cache tensor is filled
    # in 16 fixed blocks by 16 further child streams, in threads (the result does
    # not depend on how many threads run)
    sq, sk, sv = np.random.SeedSequence(w.seed).spawn(3)
    out = {"q": np.random.default_rng(sq).standard_normal((w.B, w.H, w.hd), dtype=np.float32),
           "k": _normal_blocks((w.B, w.Hkv, w.T, w.hd), sk),
           "v": _normal_blocks((w.B, w.Hkv, w.T, w.hd), sv)}
    if w.dtype == "bf16":
        out = {n: bf16_round(a) for n, a in out.items()}
    return out


def to_torch(a, dtype, device):
    """numpy float32 array -> torch tensor of ``dtype`` ("f32"/"bf16") on ``device``.

    bf16 tensors are built from the exact RNE bit patterns, so the device sees
    the same values as the oracle.
    """
    import torch
    if dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    elif dtype == "bf16":
        bits = bf16_bits(a).view(np.int16)
        t = torch.from_numpy(bits).view(torch.bfloat16)
    else:
        raise ValueError(dtype)
    return t.to(device).contiguous()

"""PyTorch-facing binding of the causal attention library.

Argument marshalling only: tensors are checked and their device pointers and
the current HIP stream are handed to the C ABI; every arithmetic step runs in
the HIP kernels of libxattn.so.  PyTorch provides device memory and streams.
"""
import math

import torch

from ._lib import BF16, F32, XattnError, check, lib

_DTYPES = {torch.float32: F32, torch.bfloat16: BF16}


def _code(t):
    if t.dtype not in _DTYPES:
        raise XattnError(5, f"unsupported dtype {t.dtype}")
    return _DTYPES[t.dtype]


def _check_tensor(t, name, shape, dtype):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise XattnError(1, f"{name} must be a device tensor")
    if tuple(t.shape) != tuple(shape):
        raise XattnError(2, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise XattnError(5, f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise XattnError(2, f"{name} must be contiguous (BHSD)")


def _dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise XattnError(2, "q and k must be 4-D [B, heads, S, hd]")
    B, H, S, hd = q.shape
    Hkv = k.shape[1]
    return B, S, H, Hkv, hd


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_lens(lens, B):
    if lens is not None:
        _check_tensor(lens, "lens", (B,), torch.int32)


def fwd(q, k, v, scale=None, o=None, lse=None, lens=None):
    """Causal attention forward.  q [B,H,S,hd]; k, v [B,Hkv,S,hd] (fp32 or bf16).
    ``lens`` ([B] int32 on the device): right-padded batch, sequence b holds
    lens[b] rows; padding rows come back as o = 0, lse = -inf.

    Returns (o [B,H,S,hd] in the input dtype, lse [B,H,S] fp32).
    """
    B, S, H, Hkv, hd = _dims(q, k)
    _check_lens(lens, B)
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    _check_tensor(q, "q", (B, H, S, hd), q.dtype)
    _check_tensor(k, "k", (B, Hkv, S, hd), q.dtype)
    _check_tensor(v, "v", (B, Hkv, S, hd), q.dtype)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor(o, "o", (B, H, S, hd), q.dtype)
    _check_tensor(lse, "lse", (B, H, S), torch.float32)
    if lens is None:
        check(lib().xattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), B, S, H, Hkv, hd, scale, _code(q), _stream(q)))
    else:
        check(lib().xattn_fwd_ragged(q.data_ptr(), k.data_ptr(), v.data_ptr(), lens.data_ptr(),
                                     o.data_ptr(), lse.data_ptr(), B, S, H, Hkv, hd, scale,
                                     _code(q), _stream(q)))
    return o, lse


def workspace_bytes(B, S, H, Hkv, hd, dtype_code):
    return int(lib().xattn_bwd_workspace_bytes(B, S, H, Hkv, hd, dtype_code))


def bwd(q, k, v, o, lse, dO, scale=None, dq=None, dk=None, dv=None, workspace=None, lens=None):
    """Causal attention backward.  Returns fp32 (dq [B,H,S,hd], dk, dv [B,Hkv,S,hd]).
    ``lens`` as in ``fwd``: padding rows and keys get zero gradients."""
    B, S, H, Hkv, hd = _dims(q, k)
    _check_lens(lens, B)
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    dt = q.dtype
    for t, n, shp in ((q, "q", (B, H, S, hd)), (k, "k", (B, Hkv, S, hd)), (v, "v", (B, Hkv, S, hd)),
                      (o, "o", (B, H, S, hd)), (dO, "dO", (B, H, S, hd))):
        _check_tensor(t, n, shp, dt)
    _check_tensor(lse, "lse", (B, H, S), torch.float32)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((B, H, S, hd), **f32) if dq is None else dq
    dk = torch.empty((B, Hkv, S, hd), **f32) if dk is None else dk
    dv = torch.empty((B, Hkv, S, hd), **f32) if dv is None else dv
    _check_tensor(dq, "dq", (B, H, S, hd), torch.float32)
    _check_tensor(dk, "dk", (B, Hkv, S, hd), torch.float32)
    _check_tensor(dv, "dv", (B, Hkv, S, hd), torch.float32)
    need = workspace_bytes(B, S, H, Hkv, hd, _code(q))
    if workspace is None:
        workspace = torch.empty((max(1, need // 4),), **f32)
    wbytes = workspace.numel() * workspace.element_size()
    if lens is None:
        check(lib().xattn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), dO.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), B, S, H, Hkv, hd, scale, _code(q),
                              workspace.data_ptr(), wbytes, _stream(q)))
    else:
        check(lib().xattn_bwd_ragged(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), dO.data_ptr(), lens.data_ptr(), dq.data_ptr(),
                                     dk.data_ptr(), dv.data_ptr(), B, S, H, Hkv, hd, scale,
                                     _code(q), workspace.data_ptr(), wbytes, _stream(q)))
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, dO, scale, dq, dk, dv):
    """Causal attention backward through ``xattn_bwd_noalloc``: the caller
    passes every output (fp32 dq [B,H,S,hd], dk, dv [B,Hkv,S,hd]) and nothing
    is allocated, by this wrapper or the library (its scratch is a fixed device
    array: B*H*S at most 2097152 query rows; calls that overlap on one GPU
    race on it).  Arguments as in ``bwd``."""
    B, S, H, Hkv, hd = _dims(q, k)
    dt = q.dtype
    for t, n, shp in ((q, "q", (B, H, S, hd)), (k, "k", (B, Hkv, S, hd)), (v, "v", (B, Hkv, S, hd)),
                      (o, "o", (B, H, S, hd)), (dO, "dO", (B, H, S, hd))):
        _check_tensor(t, n, shp, dt)
    _check_tensor(lse, "lse", (B, H, S), torch.float32)
    _check_tensor(dq, "dq", (B, H, S, hd), torch.float32)
    _check_tensor(dk, "dk", (B, Hkv, S, hd), torch.float32)
    _check_tensor(dv, "dv", (B, Hkv, S, hd), torch.float32)
    check(lib().xattn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), dO.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), B, S, H, Hkv, hd, float(scale), _code(q),
                                  _stream(q)))
    return dq, dk, dv


class CausalAttention(torch.autograd.Function):
    """autograd wrapper: o = causal_attention(q, k, v); grads are fp32 cast to the input dtype.
    With `lens` (int32 device tensor [B]) the batch is right-padded: padding rows of o are zero
    and padding inputs get zero gradients."""

    @staticmethod
    def forward(ctx, q, k, v, scale=None, lens=None):
        o, lse = fwd(q, k, v, scale, lens=lens)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.scale = scale
        ctx.lens = lens
        return o

    @staticmethod
    def backward(ctx, dO):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = bwd(q, k, v, o, lse, dO.contiguous().to(q.dtype), ctx.scale, lens=ctx.lens)
        return dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None


def causal_attention(q, k, v, scale=None, lens=None):
    return CausalAttention.apply(q, k, v, scale, lens)


def qknorm_rope_fwd(x, w, eps=1e-6, rope_base=10000.0, out=None):
    """Per-head RMS QK-norm + rotary embedding.  x [B,S,H,hd] (fp32 or bf16,
    token-major), w [hd] fp32.  Returns out [B,H,S,hd] in x's dtype (head-major)."""
    if x.dim() != 4:
        raise XattnError(2, "x must be 4-D [B, S, heads, hd]")
    B, S, H, hd = x.shape
    _check_tensor(x, "x", (B, S, H, hd), x.dtype)
    _check_tensor(w, "w", (hd,), torch.float32)
    out = torch.empty((B, H, S, hd), dtype=x.dtype, device=x.device) if out is None else out
    _check_tensor(out, "out", (B, H, S, hd), x.dtype)
    check(lib().xattn_qknorm_rope_fwd(x.data_ptr(), w.data_ptr(), out.data_ptr(), B, S, H, hd,
                                      float(eps), float(rope_base), _code(x), _stream(x)))
    return out


def qknorm_rope_workspace_bytes(B, S, H, hd):
    return int(lib().xattn_qknorm_rope_bwd_workspace_bytes(B, S, H, hd))


def qknorm_rope_bwd(x, w, dout, eps=1e-6, rope_base=10000.0, dx=None, dw=None, workspace=None):
    """Backward of qknorm_rope_fwd.  dout [B,H,S,hd] fp32.  Returns fp32
    (dx [B,S,H,hd], dw [hd])."""
    if x.dim() != 4:
        raise XattnError(2, "x must be 4-D [B, S, heads, hd]")
    B, S, H, hd = x.shape
    _check_tensor(x, "x", (B, S, H, hd), x.dtype)
    _check_tensor(w, "w", (hd,), torch.float32)
    _check_tensor(dout, "dout", (B, H, S, hd), torch.float32)
    f32 = dict(dtype=torch.float32, device=x.device)
    dx = torch.empty((B, S, H, hd), **f32) if dx is None else dx
    dw = torch.empty((hd,), **f32) if dw is None else dw
    _check_tensor(dx, "dx", (B, S, H, hd), torch.float32)
    _check_tensor(dw, "dw", (hd,), torch.float32)
    if workspace is None:
        workspace = torch.empty((max(1, qknorm_rope_workspace_bytes(B, S, H, hd) // 4),), **f32)
    check(lib().xattn_qknorm_rope_bwd(x.data_ptr(), w.data_ptr(), dout.data_ptr(), dx.data_ptr(),
                                      dw.data_ptr(), B, S, H, hd, float(eps), float(rope_base),
                                      _code(x), workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(), _stream(x)))
    return dx, dw


class QKNormRope(torch.autograd.Function):
    """autograd wrapper of the per-head RMS QK-norm + RoPE step:
    y [B,H,S,hd] = qknorm_rope(x [B,S,H,hd], w [hd]); dx is cast to x's dtype, dw stays fp32."""

    @staticmethod
    def forward(ctx, x, w, eps=1e-6, rope_base=10000.0):
        ctx.save_for_backward(x, w)
        ctx.eps, ctx.rope_base = eps, rope_base
        return qknorm_rope_fwd(x, w, eps=eps, rope_base=rope_base)

    @staticmethod
    def backward(ctx, dy):
        x, w = ctx.saved_tensors
        dx, dw = qknorm_rope_bwd(x, w, dy.contiguous().float(), eps=ctx.eps,
                                 rope_base=ctx.rope_base)
        return dx.to(x.dtype), dw, None, None


def qknorm_rope(x, w, eps=1e-6, rope_base=10000.0):
    return QKNormRope.apply(x, w, eps, rope_base)


def decode_workspace_bytes(B, T, H, Hkv, hd):
    return int(lib().xattn_decode_workspace_bytes(B, T, H, Hkv, hd))


def decode(q, k, v, lens=None, scale=None, o=None, lse=None, workspace=None):
    """Decode attention: one query per (sequence, head) against the K/V cache.

    q [B,H,hd]; k, v [B,Hkv,T,hd] (fp32 or bf16; T = cache capacity);
    lens [B] int32 on the device (positions held per sequence) or None (all T).
    Returns (o [B,H,hd] in q's dtype, lse [B,H] fp32).
    """
    if q.dim() != 3 or k.dim() != 4:
        raise XattnError(2, "q must be [B, H, hd] and k, v [B, Hkv, T, hd]")
    B, H, hd = q.shape
    Hkv, T = k.shape[1], k.shape[2]
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    _check_tensor(q, "q", (B, H, hd), q.dtype)
    _check_tensor(k, "k", (B, Hkv, T, hd), q.dtype)
    _check_tensor(v, "v", (B, Hkv, T, hd), q.dtype)
    if lens is not None:
        _check_tensor(lens, "lens", (B,), torch.int32)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if lse is None else lse
    _check_tensor(o, "o", (B, H, hd), q.dtype)
    _check_tensor(lse, "lse", (B, H), torch.float32)
    need = decode_workspace_bytes(B, T, H, Hkv, hd)
    if workspace is None and need > 0:
        workspace = torch.empty((need // 4,), dtype=torch.float32, device=q.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check(lib().xattn_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                             None if lens is None else lens.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), B, T, H, Hkv, hd, scale, _code(q), wptr, wbytes,
                             _stream(q)))
    return o, lse


def composed_buffer_bytes(B, S, H):
    return int(lib().xattn_composed_buffer_bytes(B, S, H))


def composed_fwd(q, k, v, scale=None, p=None):
    """The composed path's forward (scores, causal softmax, P.V through an
    S x S fp32 buffer).  Returns (o, lse, p) with p [B,H,S,S] fp32."""
    B, S, H, Hkv, hd = _dims(q, k)
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    _check_tensor(q, "q", (B, H, S, hd), q.dtype)
    _check_tensor(k, "k", (B, Hkv, S, hd), q.dtype)
    _check_tensor(v, "v", (B, Hkv, S, hd), q.dtype)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    p = torch.empty((B, H, S, S), dtype=torch.float32, device=q.device) if p is None else p
    _check_tensor(p, "p", (B, H, S, S), torch.float32)
    check(lib().xattn_composed_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   lse.data_ptr(), p.data_ptr(), p.numel() * 4, B, S, H, Hkv, hd,
                                   scale, _code(q), _stream(q)))
    return o, lse, p


def composed_bwd(q, k, v, p, dO, scale=None, ds=None):
    """The composed path's backward.  Returns fp32 (dq, dk, dv)."""
    B, S, H, Hkv, hd = _dims(q, k)
    scale = 1.0 / math.sqrt(hd) if scale is None else float(scale)
    for t, n, shp in ((q, "q", (B, H, S, hd)), (k, "k", (B, Hkv, S, hd)), (v, "v", (B, Hkv, S, hd)),
                      (dO, "dO", (B, H, S, hd))):
        _check_tensor(t, n, shp, q.dtype)
    _check_tensor(p, "p", (B, H, S, S), torch.float32)
    f32 = dict(dtype=torch.float32, device=q.device)
    ds = torch.empty((B, H, S, S), **f32) if ds is None else ds
    _check_tensor(ds, "ds", (B, H, S, S), torch.float32)
    dq = torch.empty((B, H, S, hd), **f32)
    dk = torch.empty((B, Hkv, S, hd), **f32)
    dv = torch.empty((B, Hkv, S, hd), **f32)
    check(lib().xattn_composed_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), p.data_ptr(),
                                   p.numel() * 4, dO.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), ds.data_ptr(), ds.numel() * 4, B, S, H, Hkv, hd,
                                   scale, _code(q), _stream(q)))
    return dq, dk, dv

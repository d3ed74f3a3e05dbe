"""ctypes wrapper over the fp64 CPU oracle of the per-head RMS QK-norm + RoPE
step (``libxattn_ref_norm.so``, built from ``ref_qknorm_rope.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
benchmark's CPU-baseline leg; never by the product path.  Inputs of any real
dtype are up-cast exactly to float64; outputs are float64.  What is computed is
documented in ``ref_qknorm_rope.c`` ("xtrain evolution overview", section 一,
rows T5, T9, T10; "xtrain -- Known Issues & Perf Backlog", KI-1 fix).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_DP = ctypes.POINTER(ctypes.c_double)


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    return a.ctypes.data_as(_DP)


class NormOracle:
    def __init__(self, path=None):
        path = path or _build.LIB_NORM
        if not os.path.exists(path):
            _build.build(_build.SRC_NORM, _build.LIB_NORM)
        lib = ctypes.CDLL(path)
        i, d = ctypes.c_int, ctypes.c_double
        lib.xattn_ref_qknorm_rope_fwd.argtypes = [_DP, _DP, _DP, i, i, i, i, d, d]
        lib.xattn_ref_qknorm_rope_fwd.restype = i
        lib.xattn_ref_qknorm_rope_bwd.argtypes = [_DP, _DP, _DP, _DP, _DP, i, i, i, i, d, d]
        lib.xattn_ref_qknorm_rope_bwd.restype = i
        self.lib = lib

    def fwd(self, x, w, eps=1e-6, base=10000.0):
        """x [B, S, H, hd], w [hd] -> out [B, H, S, hd] (float64)."""
        x, w = _f64(x), _f64(w)
        B, S, H, hd = x.shape
        out = np.zeros((B, H, S, hd))
        rc = self.lib.xattn_ref_qknorm_rope_fwd(_p(x), _p(w), _p(out), B, S, H, hd, eps, base)
        if rc:
            raise ValueError(f"xattn_ref_qknorm_rope_fwd failed: {rc}")
        return out

    def bwd(self, x, w, dout, eps=1e-6, base=10000.0):
        """x [B, S, H, hd], w [hd], dout [B, H, S, hd] -> (dx [B, S, H, hd], dw [hd])."""
        x, w, dout = _f64(x), _f64(w), _f64(dout)
        B, S, H, hd = x.shape
        dx, dw = np.zeros_like(x), np.zeros(hd)
        rc = self.lib.xattn_ref_qknorm_rope_bwd(_p(x), _p(w), _p(dout), _p(dx), _p(dw),
                                                B, S, H, hd, eps, base)
        if rc:
            raise ValueError(f"xattn_ref_qknorm_rope_bwd failed: {rc}")
        return dx, dw


_default = None


def default_norm():
    global _default
    if _default is None:
        _default = NormOracle()
    return _default

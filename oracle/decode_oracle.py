"""ctypes wrapper over the fp64 CPU oracle of decode attention
(``libxattn_ref_decode.so``, built from ``ref_decode.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
benchmark's CPU-baseline leg; never by the product path.  Inputs of any real
dtype are up-cast exactly to float64; outputs are float64.  What is computed is
documented in ``ref_decode.c`` ("xtrain evolution overview", post-training
stage, milestones M2a-M2c; infra table row T15 for the GQA head mapping).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_DP = ctypes.POINTER(ctypes.c_double)
_IP = ctypes.POINTER(ctypes.c_int)


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


class DecodeOracle:
    def __init__(self, path=None):
        path = path or _build.LIB_DEC
        if not os.path.exists(path):
            _build.build(_build.SRC_DEC, _build.LIB_DEC)
        lib = ctypes.CDLL(path)
        i, d = ctypes.c_int, ctypes.c_double
        lib.xattn_ref_decode.argtypes = [_DP, _DP, _DP, _IP, _DP, _DP, i, i, i, i, i, d]
        lib.xattn_ref_decode.restype = i
        self.lib = lib

    def decode(self, q, k, v, lens=None, scale=None):
        """q [B, H, hd]; k, v [B, Hkv, T, hd]; lens [B] ints or None (all T).
        Returns {"o": [B, H, hd], "lse": [B, H]} in float64."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, hd = q.shape
        Hkv, T = k.shape[1], k.shape[2]
        if k.shape != (B, Hkv, T, hd) or v.shape != k.shape:
            raise ValueError("shape mismatch")
        scale = 1.0 / np.sqrt(hd) if scale is None else float(scale)
        ln = None
        if lens is not None:
            ln = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
            if ln.shape != (B,):
                raise ValueError("lens must have shape [B]")
        o, lse = np.zeros((B, H, hd)), np.zeros((B, H))
        rc = self.lib.xattn_ref_decode(q.ctypes.data_as(_DP), k.ctypes.data_as(_DP),
                                       v.ctypes.data_as(_DP),
                                       None if ln is None else ln.ctypes.data_as(_IP),
                                       o.ctypes.data_as(_DP), lse.ctypes.data_as(_DP),
                                       B, T, H, Hkv, hd, scale)
        if rc:
            raise ValueError(f"xattn_ref_decode failed: {rc}")
        return {"o": o, "lse": lse}


_default = None


def default_decode():
    global _default
    if _default is None:
        _default = DecodeOracle()
    return _default

"""ctypes wrapper over the fp64 CPU oracle (``libxattn_ref.so``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
CPU-baseline leg of ``bench.py``; never by the product path.  Every function
takes numpy arrays of any real dtype, up-casts them exactly to float64 (bf16
inputs are passed as their float32 value, which is exact), and returns float64.

What the oracle computes is documented in ``ref_attn.c`` (plain causal
softmax attention and its analytic backward, GQA by repeating kv heads, after
the "xtrain evolution overview" infra table rows T14 and T15 and the KI-1 fix of
"xtrain -- Known Issues & Perf Backlog").
"""
import ctypes
import os

import numpy as np

from . import build as _build

_DP = ctypes.POINTER(ctypes.c_double)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(_DP)


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


class OracleError(RuntimeError):
    pass


class Oracle:
    """One loaded copy of the oracle library (tests may load mutated builds)."""

    def __init__(self, path=None):
        path = path or _build.LIB
        if not os.path.exists(path):
            _build.build()
        self.path = path
        lib = ctypes.CDLL(path)
        i, d = ctypes.c_int, ctypes.c_double
        lib.xattn_ref_head.argtypes = [_DP, _DP, _DP, _DP, i, i, d] + [_DP] * 9
        lib.xattn_ref_head.restype = i
        lib.xattn_ref_run.argtypes = [_DP] * 9 + [i, i, i, i, i, d, i, i]
        lib.xattn_ref_run.restype = i
        lib.xattn_ref_set_threads.argtypes = [i]
        lib.xattn_ref_set_threads.restype = None
        lib.xattn_ref_max_threads.argtypes = []
        lib.xattn_ref_max_threads.restype = i
        self.lib = lib

    # -- threads -------------------------------------------------------------
    def set_threads(self, n):
        self.lib.xattn_ref_set_threads(int(n))

    def max_threads(self):
        return int(self.lib.xattn_ref_max_threads())

    # -- single head ---------------------------------------------------------
    def head(self, q, k, v, dO=None, scale=None, want=("o", "lse")):
        """Plain attention for one head; q, k, v, dO are [S, hd].

        ``want`` names the outputs to return, from
        {P, dP, dS, rowdot, o, lse, dq, dk, dv}; returns a dict.
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        S, hd = q.shape
        scale = 1.0 / np.sqrt(hd) if scale is None else float(scale)
        dO = None if dO is None else _f64(dO)
        shapes = {"P": (S, S), "dP": (S, S), "dS": (S, S), "rowdot": (S,),
                  "o": (S, hd), "lse": (S,), "dq": (S, hd), "dk": (S, hd), "dv": (S, hd)}
        out = {n: np.zeros(shapes[n]) for n in want}
        order = ["P", "dP", "dS", "rowdot", "o", "lse", "dq", "dk", "dv"]
        rc = self.lib.xattn_ref_head(_ptr(q), _ptr(k), _ptr(v), _ptr(dO), S, hd, scale,
                                     *[_ptr(out.get(n)) for n in order])
        if rc:
            raise OracleError(f"xattn_ref_head failed: {rc}")
        return out

    # -- batched -------------------------------------------------------------
    def run(self, q, k, v, dO=None, scale=None, backward=True, units=None):
        """Batched causal attention, BHSD layout.

        q: [B, H, S, hd]; k, v: [B, Hkv, S, hd]; dO like q.
        Returns dict with o, lse and (if ``backward`` and dO given) dq, dk, dv.
        ``units`` = (lo, hi) restricts the work to flattened (b, kv head) units
        [lo, hi); other entries of the outputs are NaN.
        """
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, S, hd = q.shape
        Hkv = k.shape[1]
        if k.shape != (B, Hkv, S, hd) or v.shape != k.shape:
            raise OracleError("shape mismatch")
        scale = 1.0 / np.sqrt(hd) if scale is None else float(scale)
        bwd = backward and dO is not None
        dO = _f64(dO) if bwd else None
        fill = np.nan if units is not None else 0.0
        out = {"o": np.full(q.shape, fill), "lse": np.full((B, H, S), fill)}
        if bwd:
            out["dq"] = np.full(q.shape, fill)
            out["dk"] = np.full(k.shape, fill)
            out["dv"] = np.full(k.shape, fill)
        lo, hi = (0, B * Hkv) if units is None else units
        rc = self.lib.xattn_ref_run(_ptr(q), _ptr(k), _ptr(v), _ptr(dO),
                                    _ptr(out["o"]), _ptr(out["lse"]),
                                    _ptr(out.get("dq")), _ptr(out.get("dk")), _ptr(out.get("dv")),
                                    B, S, H, Hkv, hd, scale, int(lo), int(hi))
        if rc:
            raise OracleError(f"xattn_ref_run failed: {rc}")
        return out


    # -- right-padded batch ----------------------------------------------------
    def run_ragged(self, q, k, v, lens, dO=None, scale=None, backward=True):
        """Right-padded batch with per-sequence lengths: sequence b holds rows
        0 .. lens[b]-1 of its S-row planes.  Its rows are the plain causal
        attention of that prefix alone (``run`` on the prefix); padding rows
        are o = 0, lse = -inf, dq = dk = dv = 0, and padding inputs are never
        read.  (The pages batch sequences of different lengths by right
        padding: "xtrain evolution overview", post-training stage, M2d.)"""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, H, S, hd = q.shape
        bwd = backward and dO is not None
        out = {"o": np.zeros(q.shape), "lse": np.full((B, H, S), -np.inf)}
        if bwd:
            dO = _f64(dO)
            out.update(dq=np.zeros(q.shape), dk=np.zeros(k.shape), dv=np.zeros(k.shape))
        for b, n in enumerate(lens):
            n = int(n)
            if n < 0 or n > S:
                raise OracleError(f"length {n} outside [0, {S}]")
            if n == 0:
                continue
            r = self.run(q[b:b + 1, :, :n], k[b:b + 1, :, :n], v[b:b + 1, :, :n],
                         dO[b:b + 1, :, :n] if bwd else None, scale=scale, backward=bwd)
            for name, x in r.items():
                out[name][b, :, :n] = x[0]
        return out


_default = None


def default():
    """The oracle built from ``oracle/ref_attn.c`` (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default

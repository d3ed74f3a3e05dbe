"""ctypes loader for the in-tree ``libxattn.so`` (declared in include/xattn.h).

There is no fallback: if the library is not built, every entry point raises.
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libxattn.so")

# Every symbol include/xattn.h declares.
SYMBOLS = ("xattn_fwd", "xattn_bwd", "xattn_bwd_workspace_bytes", "xattn_bwd_dq",
           "xattn_bwd_dkdv", "xattn_qknorm_rope_fwd", "xattn_qknorm_rope_bwd_workspace_bytes",
           "xattn_qknorm_rope_bwd", "xattn_decode_workspace_bytes", "xattn_decode",
           "xattn_fwd_ragged", "xattn_bwd_ragged", "xattn_composed_buffer_bytes",
           "xattn_composed_fwd", "xattn_composed_bwd", "xattn_bwd_noalloc",
           "xattn_bwd_kernel_count", "xattn_strerror")

F32, BF16 = 0, 1
STATUS = {
    0: "XATTN_OK", 1: "XATTN_ERR_NULL", 2: "XATTN_ERR_SHAPE", 3: "XATTN_ERR_GQA",
    4: "XATTN_ERR_HEAD_DIM", 5: "XATTN_ERR_DTYPE", 6: "XATTN_ERR_WORKSPACE",
    7: "XATTN_ERR_SCALE", 8: "XATTN_ERR_HIP", 9: "XATTN_ERR_ALIGN", 10: "XATTN_ERR_PARAM",
    11: "XATTN_ERR_SCRATCH",
}


class XattnError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises XattnError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise XattnError(-1, f"{LIB_PATH} is not built; run `python -m bwd_head_rms_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    L.xattn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.xattn_fwd.restype = i
    L.xattn_bwd_workspace_bytes.argtypes = [i, i, i, i, i, i]
    L.xattn_bwd_workspace_bytes.restype = sz
    L.xattn_bwd.argtypes = [vp] * 9 + [i, i, i, i, i, f, i, vp, sz, vp]
    L.xattn_bwd.restype = i
    L.xattn_bwd_kernel_count.argtypes = [i, i, i, i, i, i]
    L.xattn_bwd_kernel_count.restype = i
    L.xattn_bwd_dq.argtypes = [vp] * 7 + [i, i, i, i, i, f, i, vp, sz, vp]
    L.xattn_bwd_dq.restype = i
    L.xattn_bwd_dkdv.argtypes = [vp] * 7 + [i, i, i, i, i, f, i, vp, sz, vp]
    L.xattn_bwd_dkdv.restype = i
    L.xattn_qknorm_rope_fwd.argtypes = [vp, vp, vp, i, i, i, i, f, f, i, vp]
    L.xattn_qknorm_rope_fwd.restype = i
    L.xattn_qknorm_rope_bwd_workspace_bytes.argtypes = [i, i, i, i]
    L.xattn_qknorm_rope_bwd_workspace_bytes.restype = sz
    L.xattn_qknorm_rope_bwd.argtypes = [vp] * 5 + [i, i, i, i, f, f, i, vp, sz, vp]
    L.xattn_qknorm_rope_bwd.restype = i
    L.xattn_fwd_ragged.argtypes = [vp] * 6 + [i, i, i, i, i, f, i, vp]
    L.xattn_fwd_ragged.restype = i
    L.xattn_bwd_ragged.argtypes = [vp] * 10 + [i, i, i, i, i, f, i, vp, sz, vp]
    L.xattn_bwd_ragged.restype = i
    L.xattn_composed_buffer_bytes.argtypes = [i, i, i]
    L.xattn_composed_buffer_bytes.restype = sz
    L.xattn_composed_fwd.argtypes = [vp] * 6 + [sz, i, i, i, i, i, f, i, vp]
    L.xattn_composed_fwd.restype = i
    L.xattn_composed_bwd.argtypes = [vp] * 4 + [sz] + [vp] * 5 + [sz, i, i, i, i, i, f, i, vp]
    L.xattn_composed_bwd.restype = i
    L.xattn_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    L.xattn_decode_workspace_bytes.restype = sz
    L.xattn_decode.argtypes = [vp] * 6 + [i, i, i, i, i, f, i, vp, sz, vp]
    L.xattn_decode.restype = i
    L.xattn_bwd_noalloc.argtypes = [vp] * 9 + [i, i, i, i, i, f, i, vp]
    L.xattn_bwd_noalloc.restype = i
    L.xattn_strerror.argtypes = [i]
    L.xattn_strerror.restype = ctypes.c_char_p
    _lib = L
    return L


def strerror(status):
    return lib().xattn_strerror(int(status)).decode()


def check(status):
    if status != 0:
        raise XattnError(status, strerror(status))

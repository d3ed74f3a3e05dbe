"""MI355X-native fused causal attention (forward + backward) behind a C ABI.

``fwd``/``bwd`` call ``libxattn.so`` (HIP kernels for gfx950); there is no CPU
or PyTorch fallback.  ``inputs`` draws the seeded synthetic workloads.
"""
from ._lib import XattnError  # noqa: F401


def __getattr__(name):
    # torch is only needed for the tensor-level API; keep `import bwd_head_rms_amd`
    # cheap for the input generator and the C-ABI tests.
    if name in ("fwd", "bwd", "causal_attention", "CausalAttention", "workspace_bytes"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)

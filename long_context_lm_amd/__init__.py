"""long_context_lm_amd: Polar Attention forward (prefill + paged decode) on MI355X.

The computation lives in libpolar.so (HIP kernels for gfx950 behind the C ABI of
include/polar.h).  ``polar`` holds the torch-facing wrappers; ``_lib`` the raw binding.
"""
from .polar import attn_fwd, attn_decode_paged, decode_workspace_bytes  # noqa: F401

__all__ = ["attn_fwd", "attn_decode_paged", "decode_workspace_bytes"]

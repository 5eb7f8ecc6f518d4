"""long_context_lm_amd: Polar Attention (prefill, paged decode, backward, variants, paged
chunks) and the gated-delta memory step on MI355X.

The computation lives in libpolar.so (HIP kernels for gfx950 behind the C ABI of
include/polar.h).  ``polar`` holds the torch-facing wrappers; ``_lib`` the raw binding.
"""
from .polar import (attn_fwd, attn_decode_paged, decode_workspace_bytes,  # noqa: F401
                    attn_fwd_train, attn_bwd, bwd_workspace_bytes, attn_fwd_variant,
                    variant_workspace_bytes, kv_append, attn_prefill_paged, delta_step)

__all__ = ["attn_fwd", "attn_decode_paged", "decode_workspace_bytes", "attn_fwd_train",
           "attn_bwd", "bwd_workspace_bytes", "attn_fwd_variant", "variant_workspace_bytes",
           "kv_append", "attn_prefill_paged", "delta_step"]

"""long_context_lm_amd: Polar Attention (prefill, paged decode, backward, variants, paged
chunks, the three streams summed) and the gated-delta memory (one step, or a whole
sequence) on MI355X.

The computation lives in libpolar.so (HIP kernels for gfx950 behind the C ABI of
include/polar.h).  ``polar`` holds the torch-facing wrappers; ``_lib`` the raw binding.
"""
from .polar import (attn_fwd, attn_fwd_mixed, attn_decode_paged,  # noqa: F401
                    decode_workspace_bytes, attn_fwd_train, attn_bwd, bwd_workspace_bytes,
                    attn_fwd_variant, variant_workspace_bytes, train_variant_workspace_bytes,
                    kv_append, attn_prefill_paged, delta_step, delta_sequence)

__all__ = ["attn_fwd", "attn_fwd_mixed", "attn_decode_paged", "decode_workspace_bytes",
           "attn_fwd_train", "attn_bwd", "bwd_workspace_bytes", "attn_fwd_variant",
           "variant_workspace_bytes", "train_variant_workspace_bytes", "kv_append", "attn_prefill_paged", "delta_step",
           "delta_sequence"]

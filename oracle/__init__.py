"""CPU oracle for Polar Attention (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` legs of ``bench.py``
may import this package.  The product path (``long_context_lm_amd``) never does.
"""
from .polar_oracle import (length_temperature, null_floor, polar_prefill, polar_decode_paged,
                           gather_pages, rope, kv_append, polar_prefill_paged, chunk_start,
                           three_streams, round_bf16, FLAG_LENGTH_TEMP, FLAG_NULL_FLOOR)

from .polar_grad import polar_prefill_grad, arg_max_keys
from .delta_oracle import delta_step, delta_step_pool, delta_sequence_pool, l2_normalize

__all__ = ["polar_prefill_grad", "arg_max_keys", "delta_step", "delta_step_pool",
           "delta_sequence_pool", "l2_normalize",
           "length_temperature", "null_floor", "polar_prefill", "polar_decode_paged",
           "gather_pages", "rope", "kv_append", "polar_prefill_paged", "chunk_start",
           "three_streams", "round_bf16",
           "FLAG_LENGTH_TEMP", "FLAG_NULL_FLOOR"]

"""Seeded synthetic workloads for Polar Attention (prefill and paged decode).

This package only *draws* inputs: random tensors, the L2 normalisation of q and k
that the model applies before attention, planted needle keys, page tables and the
round-to-nearest-even cast to bfloat16, and upstream gradients for the backward pass.  It contains none of the attention
arithmetic; both the CPU oracle and the GPU path consume what it returns.
"""
from .workloads import (CONFIGS, PrefillInputs, DecodeInputs, prefill_inputs,
                        decode_inputs, round_bf16, bf16_bits_to_f32, FLAG_LENGTH_TEMP,
                        FLAG_NULL_FLOOR, Cotangents, cotangents, ChunkInputs,
                        chunk_inputs, DeltaInputs, delta_inputs,
                        DeltaSeqInputs, delta_seq_inputs)

__all__ = ["CONFIGS", "PrefillInputs", "DecodeInputs", "prefill_inputs", "decode_inputs",
           "round_bf16", "bf16_bits_to_f32", "FLAG_LENGTH_TEMP", "FLAG_NULL_FLOOR", "Cotangents",
           "cotangents", "ChunkInputs", "chunk_inputs",
           "DeltaInputs", "delta_inputs", "DeltaSeqInputs", "delta_seq_inputs"]

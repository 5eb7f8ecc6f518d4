"""The allocation-free paged decode (polar_attn_decode_paged_noalloc), through the C ABI:
two calls in a row, the full 256K workload (16 sequences x 262,144 keys) and then a smaller
one, each equal bit for bit to polar_attn_decode_paged with a caller workspace (the same
kernels and grid; only where the split partials live differs), and the second also against
the oracle."""
import pytest
import torch

import synth
from parity import assert_close, gpu_decode, oracle_decode

pytestmark = pytest.mark.gpu

KEYS = ("dir", "count", "n_eff", "gate", "lse")


def test_noalloc_decode_equals_workspace_decode_on_two_calls(gpu_lib):
    from long_context_lm_amd import _lib, decode_workspace_bytes
    print("[case] noalloc decode: C5 full then B=3", flush=True)
    big = synth.decode_inputs("c5")
    small = synth.decode_inputs("c5", B=3, seq_lens=[3000, 1500, 700])
    for d in (big, small):
        assert decode_workspace_bytes(d.Hq, d.Hkv, d.B, d.max_seq_len) <= \
            _lib.POLAR_NOALLOC_SCRATCH_BYTES
    got_big = gpu_decode(big, no_alloc=True)
    got_small = gpu_decode(small, no_alloc=True)      # the scratch still holds big's partials
    ref_big = gpu_decode(big)
    ref_small = gpu_decode(small)
    for label, got, ref in (("C5", got_big, ref_big), ("B=3", got_small, ref_small)):
        for k in KEYS:
            assert torch.equal(got[k], ref[k]), (label, k)
    assert_close(got_small, oracle_decode(small), small.count_vec, small.dtype,
                 label="noalloc decode B=3")


def test_noalloc_decode_refuses_a_workspace_argument(gpu_lib):
    d = synth.decode_inputs("c5", B=1, seq_lens=[100])
    with pytest.raises(ValueError, match="no workspace"):
        gpu_decode(d, no_alloc=True, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))

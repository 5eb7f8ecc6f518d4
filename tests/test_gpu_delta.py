"""GPU parity of the in-place gated-delta memory step against the float64 oracle, through
the C ABI.  fp32 state arithmetic, judged per state and per output vector: the relative
Frobenius error of every (slot, head) state and the relative error of every (sequence, head)
output, at most 1e-5 after one step (64-term fp32 dot products) and 1e-4 after 32 chained
steps; slots the batch does not name must stay bit-identical."""
import numpy as np
import pytest
import torch

import oracle
import synth
from long_context_lm_amd import delta_step

pytestmark = pytest.mark.gpu


def _dev(d):
    conv = (lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
            .view(torch.bfloat16).cuda()) if d.dtype == "bf16" else (lambda a: torch.from_numpy(a).cuda())
    return (torch.from_numpy(d.pool).cuda(), torch.from_numpy(d.slots).cuda(), conv(d.q),
            conv(d.k), conv(d.v), torch.from_numpy(d.alpha).cuda(), torch.from_numpy(d.beta).cuda())


def _err(got, want):
    """Largest relative error of one state (last two axes) or output vector (last axis),
    so that an error in a small-norm state is not hidden by a large one elsewhere."""
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    axes = (-2, -1) if want.ndim >= 4 else (-1,)
    num = np.sqrt(np.sum((got - want) ** 2, axis=axes))
    den = np.sqrt(np.sum(want ** 2, axis=axes))
    return float(np.max(num / np.maximum(den, 1e-30)))


# (bf16, 256, 16, 1024) is the benchmark's step; (f32, 7, 3, 9) leaves a workgroup with a
# partial run of states (21 states, 4 per workgroup).
@pytest.mark.parametrize("dtype,B,H,slots", [("bf16", 64, 16, 256), ("f32", 33, 4, 40),
                                             ("bf16", 1, 1, 1), ("bf16", 256, 16, 1024),
                                             ("f32", 7, 3, 9)])
def test_delta_step_parity(gpu_lib, dtype, B, H, slots):
    print(f"[case] delta {dtype} B={B} H={H} slots={slots}", flush=True)
    d = synth.delta_inputs(B=B, H=H, num_slots=slots, dtype=dtype)
    pool, sl, q, k, v, al, be = _dev(d)
    out = delta_step(pool, sl, q, k, v, al, be)
    torch.cuda.synchronize()
    want_pool, want_out = oracle.delta_step_pool(d.pool, d.slots, d.as_f32("q"), d.as_f32("k"),
                                                 d.as_f32("v"), d.alpha, d.beta)
    got_pool = pool.cpu().numpy()
    used = np.zeros(slots, bool)
    used[d.slots] = True
    np.testing.assert_array_equal(got_pool[~used], d.pool[~used])
    e_pool = _err(got_pool[used].astype(np.float64), want_pool[used])
    e_out = _err(out.cpu().numpy().astype(np.float64), want_out)
    print(f"[delta] {dtype} state {e_pool:.2e} out {e_out:.2e}", flush=True)
    assert e_pool <= 1e-5 and e_out <= 1e-5


def test_delta_step_chain_of_32_steps(gpu_lib):
    d = synth.delta_inputs(B=16, H=8, num_slots=16, dtype="f32")
    pool, sl, *_ = _dev(d)
    ref = d.pool.astype(np.float64)
    r = np.random.default_rng(0)
    for step in range(32):
        q, k, v = (r.standard_normal((16, 8, 64)).astype(np.float32) for _ in range(3))
        al = r.uniform(0.9, 1.0, (16, 8)).astype(np.float32)
        be = r.uniform(0.0, 1.0, (16, 8)).astype(np.float32)
        out = delta_step(pool, sl, *(torch.from_numpy(x).cuda() for x in (q, k, v, al, be)))
        ref, want = oracle.delta_step_pool(ref, d.slots, q, k, v, al, be)
    torch.cuda.synchronize()
    e_pool = _err(pool.cpu().numpy().astype(np.float64), ref)
    e_out = _err(out.cpu().numpy().astype(np.float64), want)
    print(f"[delta] 32 steps: state {e_pool:.2e} out {e_out:.2e}", flush=True)
    assert e_pool <= 1e-4 and e_out <= 1e-4


def test_delta_step_invalid_slot_and_no_normalisation(gpu_lib):
    d = synth.delta_inputs(B=4, H=2, num_slots=6, dtype="f32")
    d.slots[2] = -1
    pool, sl, q, k, v, al, be = _dev(d)
    out = delta_step(pool, sl, q, k, v, al, be, normalize_qk=False)
    torch.cuda.synchronize()
    want_pool, want_out = oracle.delta_step_pool(d.pool, d.slots, d.q, d.k, d.v, d.alpha, d.beta,
                                                 normalize=False)
    assert float(out[2].abs().max()) == 0.0
    used = np.array([s for s in d.slots if s >= 0])
    assert _err(pool.cpu().numpy()[used], want_pool[used]) <= 1e-5
    live = np.arange(4) != 2
    assert _err(out.cpu().numpy()[live], want_out[live]) <= 1e-5

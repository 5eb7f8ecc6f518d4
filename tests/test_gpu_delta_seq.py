"""GPU parity of the memory stream over a sequence (polar_delta_sequence) through the C ABI:
against the float64 oracle (the step applied token by token), and against T chained calls
of the one-step kernel.

Tolerance.  One fp32 step rounds the state by a few ulps per element and its 64-term dots
by at most about 64 ulps (relative 4e-6); the gate alpha >= 0.9 shrinks an earlier error by
at least 0.9 per token, so the error carried in the state stays below 4e-6 / (1 - 0.9) =
4e-5 however long the sequence.  Every state (relative Frobenius error of each (slot,
head)) and every output (each (sequence, head), all tokens together) is held to 1e-4;
outputs are also checked vector by vector at 1e-3, since a single o_t can be small beside
the state it reads.  Slots no sequence names stay bit-identical."""
import numpy as np
import pytest
import torch

import oracle
import synth
from long_context_lm_amd import delta_sequence, delta_step

pytestmark = pytest.mark.gpu


def _dev(d):
    conv = (lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
            .view(torch.bfloat16).cuda()) if d.dtype == "bf16" else (lambda a: torch.from_numpy(a).cuda())
    return (torch.from_numpy(d.pool).cuda(), torch.from_numpy(d.slots).cuda(), conv(d.q),
            conv(d.k), conv(d.v), torch.from_numpy(d.alpha).cuda(), torch.from_numpy(d.beta).cuda())


def _rel(got, want, axes):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    num = np.sqrt(np.sum((got - want) ** 2, axis=axes))
    den = np.sqrt(np.sum(want ** 2, axis=axes))
    return float(np.max(num / np.maximum(den, 1e-30)))


def _check(d, pool, out, want_pool, want_out, live=None, tol=1e-4):
    """States of the named slots and outputs [B,T,H,d] of the live sequences against the
    oracle; untouched slots bit-identical."""
    got_pool = pool.cpu().numpy()
    used = np.zeros(d.pool.shape[0], bool)
    used[[s for s in d.slots if 0 <= s < d.pool.shape[0]]] = True
    np.testing.assert_array_equal(got_pool[~used], d.pool[~used])
    live = np.ones(len(d.slots), bool) if live is None else live
    o = out.cpu().numpy()[live]
    e_state = _rel(got_pool[used], want_pool[used], (-2, -1))
    e_out = _rel(o.transpose(0, 2, 1, 3), want_out[live].transpose(0, 2, 1, 3), (-2, -1))
    e_vec = _rel(o, want_out[live], (-1,))
    print(f"[delta-seq] state {e_state:.2e} out {e_out:.2e} worst vector {e_vec:.2e}", flush=True)
    assert e_state <= tol and e_out <= tol and e_vec <= 10 * tol


def _oracle(d, normalize=True):
    return oracle.delta_sequence_pool(d.pool, d.slots, d.as_f32("q"), d.as_f32("k"),
                                      d.as_f32("v"), d.alpha, d.beta, normalize=normalize)


# T = 2048 at 16 heads; ragged lengths around the 64-token chunk (1, 63, 65, 200 = 3 chunks
# and 8); fp32 inputs; a sharper gate (alpha in [0.5, 1)).
@pytest.mark.parametrize("dtype,B,T,H,slots,arange", [
    ("bf16", 2, 2048, 16, 8, (0.9, 1.0)),
    ("f32", 3, 200, 3, 5, (0.9, 1.0)),
    ("bf16", 2, 1, 2, 2, (0.9, 1.0)),
    ("bf16", 3, 63, 1, 4, (0.9, 1.0)),
    ("f32", 1, 65, 2, 1, (0.9, 1.0)),
    ("bf16", 4, 300, 4, 9, (0.5, 1.0)),
])
def test_delta_sequence_parity(gpu_lib, dtype, B, T, H, slots, arange):
    print(f"[case] delta-seq {dtype} B={B} T={T} H={H} slots={slots} alpha={arange}", flush=True)
    d = synth.delta_seq_inputs(B=B, T=T, H=H, num_slots=slots, dtype=dtype, alpha_range=arange)
    pool, sl, q, k, v, al, be = _dev(d)
    out = delta_sequence(pool, sl, q, k, v, al, be)
    torch.cuda.synchronize()
    _check(d, pool, out, *_oracle(d))


def test_delta_sequence_64k(gpu_lib):
    """A 64K-token sequence: the final state and the outputs at 512 sampled positions (the
    oracle walks every token; the comparison samples)."""
    print("[case] delta-seq bf16 B=1 T=65536 H=4", flush=True)
    d = synth.delta_seq_inputs(B=1, T=65536, H=4, num_slots=2, dtype="bf16")
    pool, sl, q, k, v, al, be = _dev(d)
    out = delta_sequence(pool, sl, q, k, v, al, be)
    torch.cuda.synchronize()
    want_pool, want_out = _oracle(d)
    pick = np.sort(np.random.default_rng(7).choice(65536, 512, replace=False))
    pick[-1] = 65535
    d_s = synth.DeltaSeqInputs(dtype=d.dtype, pool=d.pool, slots=d.slots, q=d.q[:, pick],
                               k=d.k[:, pick], v=d.v[:, pick], alpha=d.alpha[:, pick],
                               beta=d.beta[:, pick])
    _check(d_s, pool, out[:, torch.from_numpy(pick).cuda()], want_pool, want_out[:, pick])


def test_delta_sequence_equals_chained_steps(gpu_lib):
    """T calls of the one-step kernel on token t = 0..T-1 leave the same states and outputs,
    to the fp32 bound (the two kernels reduce in different orders)."""
    B, T, H = 8, 2048, 16
    d = synth.delta_seq_inputs(B=B, T=T, H=H, num_slots=12, dtype="bf16", seed=4102)
    pool, sl, q, k, v, al, be = _dev(d)
    pool2 = pool.clone()
    out = delta_sequence(pool, sl, q, k, v, al, be)
    steps = torch.empty_like(out)
    for t in range(T):
        steps[:, t] = delta_step(pool2, sl, q[:, t].contiguous(), k[:, t].contiguous(),
                                 v[:, t].contiguous(), al[:, t].contiguous(),
                                 be[:, t].contiguous())
    torch.cuda.synchronize()
    used = d.slots
    e_state = _rel(pool.cpu().numpy()[used], pool2.cpu().numpy()[used], (-2, -1))
    e_out = _rel(out.cpu().numpy().transpose(0, 2, 1, 3),
                 steps.cpu().numpy().transpose(0, 2, 1, 3), (-2, -1))
    print(f"[delta-seq] vs {T} chained steps: state {e_state:.2e} out {e_out:.2e}", flush=True)
    assert e_state <= 1e-4 and e_out <= 1e-4
    np.testing.assert_array_equal(np.delete(pool.cpu().numpy(), used, 0),
                                  np.delete(pool2.cpu().numpy(), used, 0))


def test_delta_sequence_bench_shape_sampled(gpu_lib):
    """The timed workload (32 sequences x 2048 tokens x 16 heads, bf16) in the same launch;
    three sequences re-run through the oracle one by one."""
    d = synth.delta_seq_inputs(B=32, T=2048, H=16, num_slots=64, dtype="bf16")
    pool, sl, q, k, v, al, be = _dev(d)
    out = delta_sequence(pool, sl, q, k, v, al, be)
    torch.cuda.synchronize()
    got_pool, got_out = pool.cpu().numpy(), out.cpu().numpy()
    for b in (0, 17, 31):
        s = d.slots[b]
        q1, k1, v1 = (synth.bf16_bits_to_f32(x[b:b + 1]) for x in (d.q, d.k, d.v))
        want_pool, want_out = oracle.delta_sequence_pool(
            d.pool[s:s + 1], [0], q1, k1, v1, d.alpha[b:b + 1], d.beta[b:b + 1])
        e_state = _rel(got_pool[s], want_pool[0], (-2, -1))
        e_out = _rel(got_out[b].transpose(1, 0, 2), want_out[0].transpose(1, 0, 2), (-2, -1))
        print(f"[delta-seq] bench shape b={b}: state {e_state:.2e} out {e_out:.2e}", flush=True)
        assert e_state <= 1e-4 and e_out <= 1e-4


def test_delta_sequence_invalid_slot_and_no_normalisation(gpu_lib):
    d = synth.delta_seq_inputs(B=4, T=130, H=2, num_slots=6, dtype="f32")
    d.q, d.k = d.q / np.float32(8), d.k / np.float32(8)   # |k| near 1 keeps I - beta k k^T stable
    d.slots[2] = -1
    d.slots[3] = 6
    pool, sl, q, k, v, al, be = _dev(d)
    out = delta_sequence(pool, sl, q, k, v, al, be, normalize_qk=False)
    torch.cuda.synchronize()
    want_pool, want_out = _oracle(d, normalize=False)
    assert float(out[2:].abs().max()) == 0.0
    _check(d, pool, out, want_pool, want_out, live=np.array([True, True, False, False]))


@pytest.mark.parametrize("cut", [128, 130])
def test_delta_sequence_in_place_continuation(gpu_lib, cut):
    """Two calls over the two parts of a sequence equal one call over the whole: the state
    left in the pool is the next call's starting state.  The kernel takes tokens in groups
    of 8 from the start of each call, so a cut at a multiple of 8 gives the same bits and
    any other cut the same values to fp32 rounding."""
    d = synth.delta_seq_inputs(B=3, T=320, H=4, num_slots=3, dtype="bf16", seed=4103)
    pool, sl, q, k, v, al, be = _dev(d)
    pool2 = pool.clone()
    out = delta_sequence(pool, sl, q, k, v, al, be)
    o1 = delta_sequence(pool2, sl, q[:, :cut].contiguous(), k[:, :cut].contiguous(),
                        v[:, :cut].contiguous(), al[:, :cut].contiguous(),
                        be[:, :cut].contiguous())
    o2 = delta_sequence(pool2, sl, q[:, cut:].contiguous(), k[:, cut:].contiguous(),
                        v[:, cut:].contiguous(), al[:, cut:].contiguous(),
                        be[:, cut:].contiguous())
    torch.cuda.synchronize()
    both = torch.cat([o1, o2], 1)
    if cut % 8 == 0:
        assert torch.equal(pool, pool2)
        assert torch.equal(out, both)
    else:
        assert _rel(pool.cpu().numpy(), pool2.cpu().numpy(), (-2, -1)) <= 1e-5
        assert _rel(out.cpu().numpy().transpose(0, 2, 1, 3),
                    both.cpu().numpy().transpose(0, 2, 1, 3), (-2, -1)) <= 1e-5


def test_delta_sequence_extreme_gates(gpu_lib):
    """Gates that the deferred form cannot carry (a zero gate, products far below 2^-64,
    a gate above one) take the step as written: the result still follows the oracle."""
    d = synth.delta_seq_inputs(B=2, T=96, H=3, num_slots=2, dtype="f32", seed=4104)
    d.alpha[0, 5, :] = 0.0                  # the state is wiped at token 5
    d.alpha[0, 40:48, 1] = 1e-12            # group product 1e-96
    d.alpha[1, 16:24, 2] = 0.01             # group product 1e-16 (deferred form)
    d.alpha[1, 60, 0] = 1.5                 # a gate above one
    pool, sl, q, k, v, al, be = _dev(d)
    out = delta_sequence(pool, sl, q, k, v, al, be)
    torch.cuda.synchronize()
    _check(d, pool, out, *_oracle(d))

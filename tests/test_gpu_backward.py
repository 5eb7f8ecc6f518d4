"""GPU parity of the training forward (residuals) and the backward pass against the float64
autograd oracle, through the C ABI.  Tolerances are stated in tests/parity.py."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (GRAD_KEYS, assert_grads_close, gpu_backward, gpu_forward_train,
                    gpu_prefill, host, oracle_backward, oracle_prefill)

pytestmark = pytest.mark.gpu


def _inputs(B, T, Hq, Hkv, train_len=64, flags=3, seed=None, rand_params=False):
    p = synth.prefill_inputs("c2", B=B, T=T, Hq=Hq, Hkv=Hkv, train_len=train_len, flags=flags,
                             seed=seed)
    if rand_params:
        rng = np.random.default_rng(5)
        p.beta = rng.uniform(4.0, 12.0, Hq).astype(np.float32)
        p.null_bias = rng.uniform(-1.0, 1.0, Hq).astype(np.float32)
    return p


def _cot(p, seed=2001, drop=()):
    c = synth.cotangents(p.B, p.T, p.Hq, p.d, seed=seed).as_dict()
    return {n: (None if n in drop else x) for n, x in c.items()}


def test_forward_train_matches_forward_and_oracle(gpu_lib):
    print("[case] fwd_train B=2 T=300 Hq=8 Hkv=2", flush=True)
    p = _inputs(2, 300, 8, 2)
    _, tr = gpu_forward_train(p)
    plain = gpu_prefill(p)
    for n in ("dir", "count", "n_eff", "gate", "lse"):
        np.testing.assert_allclose(host(tr[n]), host(plain[n]), rtol=1e-6, atol=1e-6)
    want = oracle_prefill(p)
    un = host(tr["u_norm"])
    assert np.max(np.abs(un - want["u_norm"]) / want["u_norm"]) < 2e-2
    am = tr["arg_max"].cpu().numpy()
    ref = oracle.arg_max_keys(p.as_f32("q"), p.as_f32("k"), p.beta, p.train_len, p.flags)
    assert am.min() >= 0 and np.all(am <= np.arange(p.T)[None, :, None])
    # where the two differ, the GPU's key must tie the maximum to fp32 rounding
    qf, kf = p.as_f32("q").astype(np.float64), p.as_f32("k").astype(np.float64)
    G = p.Hq // p.Hkv
    for b, i, h in zip(*np.nonzero(am != ref)):
        s_gpu = qf[b, i, h] @ kf[b, am[b, i, h], h // G]
        s_ref = qf[b, i, h] @ kf[b, ref[b, i, h], h // G]
        assert abs(s_gpu - s_ref) < 1e-5, (b, i, h)
    print(f"[fwd_train] arg-max mismatches (ties) {int(np.sum(am != ref))} of {am.size}")


@pytest.mark.parametrize("B,T,Hq,Hkv,flags,train_len,rand", [
    (2, 300, 8, 2, 3, 64, False),      # ragged T, GQA 4, temperature and floor active
    (1, 129, 4, 4, 3, 32, True),       # no GQA, per-head beta and bias
    (1, 200, 4, 2, 0, 2048, False),    # flags off, G = 2
    (1, 100, 16, 2, 3, 16, False),     # G = 8
    (1, 1, 4, 1, 3, 2048, False),      # a single row
    (1, 65, 4, 1, 3, 8, True),         # one key past a 64-key tile
    (1, 150, 32, 4, 3, 64, False),     # 32 heads: prep walks 16-head slabs token by token
    (2, 130, 6, 2, 3, 64, True),       # 6 heads (G = 3): prep's one-row fallback, no head split
])
def test_backward_parity(gpu_lib, B, T, Hq, Hkv, flags, train_len, rand):
    print(f"[case] bwd B={B} T={T} Hq={Hq} Hkv={Hkv} flags={flags} L={train_len}", flush=True)
    p = _inputs(B, T, Hq, Hkv, train_len, flags, rand_params=rand)
    cot = _cot(p)
    got = gpu_backward(p, cot)
    want = oracle_backward(p, cot)
    assert_grads_close(got, want, label=f"B{B} T{T} {Hq}/{Hkv} f{flags}")


@pytest.mark.parametrize("drop", [("count", "n_eff", "gate", "lse"), ("dir",),
                                  ("dir", "count", "n_eff"), ("count",)])
def test_backward_partial_cotangents(gpu_lib, drop):
    print(f"[case] bwd partial cotangents without {drop}", flush=True)
    p = _inputs(1, 160, 8, 2)
    cot = _cot(p, drop=drop)
    got = gpu_backward(p, cot)
    want = oracle_backward(p, cot)
    keys = [n for n in GRAD_KEYS if not (n == "d_count_vec" and "count" in drop)]
    assert_grads_close(got, want, keys=keys, label=f"without {drop}")
    if "count" in drop:
        assert float(got["d_count_vec"].abs().max()) == 0.0


def test_backward_without_parameter_grads(gpu_lib):
    p = _inputs(1, 96, 4, 2)
    cot = _cot(p)
    full = gpu_backward(p, cot)
    part = gpu_backward(p, cot, param_grads=False)
    assert set(part) == {"dq", "dk", "dv"}
    for n in ("dq", "dk", "dv"):
        assert torch.equal(full[n], part[n])


def test_backward_is_deterministic(gpu_lib):
    p = _inputs(2, 333, 16, 4)
    cot = _cot(p)
    a = gpu_backward(p, cot)
    b = gpu_backward(p, cot)
    for n in GRAD_KEYS:
        assert torch.equal(a[n], b[n]), n


def test_backward_empty_sequence_zeroes_parameter_grads(gpu_lib):
    from long_context_lm_amd import attn_bwd
    dev = "cuda"
    q = torch.zeros(1, 0, 4, 64, dtype=torch.bfloat16, device=dev)
    k = torch.zeros(1, 0, 2, 64, dtype=torch.bfloat16, device=dev)
    f32 = dict(device=dev, dtype=torch.float32)
    fwd = dict(dir=torch.zeros(1, 0, 4, 64, **f32), n_eff=torch.zeros(1, 0, 4, **f32),
               gate=torch.zeros(1, 0, 4, **f32), lse=torch.zeros(1, 0, 4, **f32),
               u_norm=torch.zeros(1, 0, 4, **f32))
    fwd["arg_max"] = torch.zeros(1, 0, 4, dtype=torch.int32, device=dev)
    g = attn_bwd(q, k, k, fwd, {}, count_vec=np.ones((4, 64), np.float32))
    torch.cuda.synchronize()
    assert g["dq"].numel() == 0
    for n in ("d_beta", "d_null_bias", "d_count_vec"):
        assert float(g[n].abs().max()) == 0.0


def test_backward_full_c2(gpu_lib):
    """The 2K training shape (B=8, T=2048, 16 query / 4 KV heads) at full size: every
    gradient, the per-head parameter gradients (sums over all 8 sequences) included,
    against the oracle differentiating the whole workload."""
    print("[case] bwd full C2 B=8 T=2048 16/4", flush=True)
    p = synth.prefill_inputs("c2")
    cot = _cot(p)
    got = gpu_backward(p, cot, param_grads=True)
    want = oracle_backward(p, cot)
    assert_grads_close(got, want, label="C2 full")


@pytest.mark.parametrize("B,T,Hq,Hkv", [(8, 2048, 16, 4), (128, 600, 4, 4), (64, 600, 8, 4)])
def test_lean_forward_train_equals_pipelined_and_plain(gpu_lib, B, T, Hq, Hkv):
    """At least 512 workgroups choose the lean training instance (held to 128 registers):
    1024 at B=8, T=2048, 16/4 heads; 1536 and 1280 with one and two heads per block (256-
    and 128-row blocks).  Every output and residual bit-identical to one-sequence launches
    (the pipelined instance), and the outputs to the plain forward."""
    print(f"[case] fwd_train lean B={B} T={T} {Hq}/{Hkv}", flush=True)
    import dataclasses
    p = synth.prefill_inputs("c2", B=B, T=T, Hq=Hq, Hkv=Hkv)
    _, tr = gpu_forward_train(p)
    plain = gpu_prefill(p)
    keys = ("dir", "count", "n_eff", "gate", "lse")
    for n in keys:
        assert torch.equal(tr[n], plain[n]), n
    for b in (0, B - 3):
        one = dataclasses.replace(p, B=1, q=p.q[b:b + 1], k=p.k[b:b + 1], v=p.v[b:b + 1],
                                  needles=[x for x in p.needles if x[0] == b])
        _, t1 = gpu_forward_train(one)
        for n in keys + ("u_norm", "arg_max"):
            assert torch.equal(tr[n][b:b + 1], t1[n]), (b, n)

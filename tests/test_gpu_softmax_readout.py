"""GPU parity of the plain softmax read-out u = sum_j p_j v_j in training: the training
forward writes it (polar_attn_fwd_train_variant with var.attn) and the backward takes its
gradient (polar_cotangents.attn), through the C ABI.

The read-out is the softmax arm the pages train beside Polar Attention (technical
summary, section 3.1).  The reference is the float64 autograd oracle
(oracle.polar_prefill_grad with an "attn" cotangent; the rotated q and k rounded to
bfloat16 as the kernels hold them), under the causal backward's tolerances
(tests/parity.py).  The forward read-out is compared with the variant forward's
(polar_attn_fwd_variant: bit for bit in bf16) and with the oracle at the dtype's bound."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import GRAD_KEYS, TOL, assert_grads_close, host, to_dev

pytestmark = pytest.mark.gpu

OUTS = ("dir", "count", "n_eff", "gate", "lse", "u_norm", "arg_max")


def _setup(B, T, Hq, Hkv, train_len=64, dtype="bf16"):
    p = synth.prefill_inputs("c2", B=B, T=T, Hq=Hq, Hkv=Hkv, train_len=train_len, flags=3,
                             dtype=dtype)
    cot = synth.cotangents(p.B, p.T, p.Hq, p.d, seed=2005, attn=True).as_dict()
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    kw = dict(beta=p.beta, null_bias=p.null_bias, count_vec=p.count_vec,
              train_len=p.train_len, flags=p.flags)
    return p, cot, (q, k, v), kw


def _oracle_grads(p, cot, window, theta, batches=None):
    sl = slice(None) if batches is None else list(batches)
    c = {n: np.asarray(x)[sl] for n, x in cot.items() if x is not None}
    return oracle.polar_prefill_grad(p.as_f32("q")[sl], p.as_f32("k")[sl], p.as_f32("v")[sl],
                                     c, p.beta, p.null_bias, p.count_vec, p.train_len, p.flags,
                                     window=window, rope_theta=theta,
                                     rope_bf16=p.dtype == "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("window,theta,B,T,Hq,Hkv", [
    (0, 0.0, 2, 300, 8, 2),           # causal
    (96, 0.0, 1, 400, 16, 4),         # window
    (0, 10000.0, 1, 257, 4, 1),       # RoPE, GQA 4
    (80, 500.0, 2, 200, 8, 2),        # both
])
def test_training_forward_writes_the_readout(gpu_lib, dtype, window, theta, B, T, Hq, Hkv):
    """The read-out of the training forward: the variant forward's, the oracle's within the
    dtype's bound, u = dir |u| to rounding, and the other outputs unchanged by asking for
    it."""
    from long_context_lm_amd import attn_fwd_train, attn_fwd_variant
    print(f"[case] train read-out {dtype} W={window} theta={theta} B={B} T={T} {Hq}/{Hkv}",
          flush=True)
    p, _, (q, k, v), kw = _setup(B, T, Hq, Hkv, dtype=dtype)
    got = attn_fwd_train(q, k, v, window=window, rope_theta=theta, want_attn=True, **kw)
    plain = attn_fwd_train(q, k, v, window=window, rope_theta=theta, **kw)
    torch.cuda.synchronize()
    for n in OUTS:
        assert torch.equal(got[n], plain[n]), n
    ref = attn_fwd_variant(q, k, v, window=window, rope_theta=theta, **kw)
    torch.cuda.synchronize()
    if dtype == "bf16":
        assert torch.equal(got["attn"], ref["attn"])
    else:
        # fp32: the training forward rotates q in a kernel of its own, the variant forward
        # at load, so the two agree to fp32 rounding.
        d = float((got["attn"] - ref["attn"]).abs().max() / ref["attn"].abs().max())
        assert d <= 1e-5, d
    want = oracle.polar_prefill(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.beta,
                                p.null_bias, p.count_vec, p.train_len, p.flags, window=window,
                                rope_theta=theta, rope_bf16=dtype == "bf16")
    a, w = host(got["attn"]), want["attn"]
    err = float(np.max(np.linalg.norm(a - w, axis=-1) / np.linalg.norm(w, axis=-1)))
    assert err <= TOL[dtype], err
    u = host(got["dir"]) * host(got["u_norm"])[..., None]
    np.testing.assert_allclose(a, u, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("window,theta,B,T,Hq,Hkv", [
    (0, 0.0, 2, 300, 8, 2),           # causal, ragged T, GQA 4
    (0, 0.0, 1, 65, 4, 4),            # one key past a tile, no GQA
    (100, 0.0, 1, 257, 4, 1),         # a window that is no multiple of the tiles
    (96, 10000.0, 1, 400, 16, 4),     # window + RoPE
])
def test_readout_backward_parity(gpu_lib, window, theta, B, T, Hq, Hkv):
    """Every cotangent at once, the read-out's included."""
    from long_context_lm_amd import attn_bwd, attn_fwd_train
    print(f"[case] read-out bwd W={window} theta={theta} B={B} T={T} {Hq}/{Hkv}", flush=True)
    p, cot, (q, k, v), kw = _setup(B, T, Hq, Hkv)
    fwd = attn_fwd_train(q, k, v, window=window, rope_theta=theta, **kw)
    got = attn_bwd(q, k, v, fwd, cot, window=window, rope_theta=theta, **kw)
    torch.cuda.synchronize()
    assert_grads_close(got, _oracle_grads(p, cot, window, theta),
                       label=f"read-out W{window} theta{theta}")


@pytest.mark.parametrize("window,theta", [(0, 0.0), (64, 10000.0)])
def test_readout_alone_is_the_softmax_arm(gpu_lib, window, theta):
    """Only the read-out's cotangent: the softmax arm's own gradients.  The gate and count
    parameters get exactly zero, and the others match the oracle."""
    from long_context_lm_amd import attn_bwd, attn_fwd_train
    print(f"[case] read-out alone W={window} theta={theta}", flush=True)
    p, cot, (q, k, v), kw = _setup(2, 300, 8, 2)
    only = {"attn": cot["attn"]}
    fwd = attn_fwd_train(q, k, v, window=window, rope_theta=theta, **kw)
    got = attn_bwd(q, k, v, fwd, only, window=window, rope_theta=theta, **kw)
    torch.cuda.synchronize()
    assert not torch.any(got["d_null_bias"])
    assert not torch.any(got["d_count_vec"])
    assert_grads_close(got, _oracle_grads(p, only, window, theta),
                       keys=("dq", "dk", "dv", "d_beta"), label="read-out alone")


def test_readout_cotangent_adds_linearly(gpu_lib):
    """The backward is linear in the cotangents: gradients with the read-out's cotangent
    equal those without it plus those of the read-out alone (to fp32 rounding of the sum,
    as the kernels hold du in bf16)."""
    from long_context_lm_amd import attn_bwd, attn_fwd_train
    p, cot, (q, k, v), kw = _setup(1, 200, 8, 2)
    fwd = attn_fwd_train(q, k, v, **kw)
    both = attn_bwd(q, k, v, fwd, cot, **kw)
    rest = attn_bwd(q, k, v, fwd, {n: x for n, x in cot.items() if n != "attn"}, **kw)
    alone = attn_bwd(q, k, v, fwd, {"attn": cot["attn"]}, **kw)
    torch.cuda.synchronize()
    for n in GRAD_KEYS:
        s = rest[n] + alone[n]
        scale = float(s.abs().max())
        assert float((both[n] - s).abs().max()) <= 2e-2 * scale, n


def test_readout_backward_training_shape(gpu_lib):
    """The 2K training shape (B=8, T=2048, 16/4 heads) with every cotangent; sequences 0
    and 7 against the oracle, and the run repeated bit for bit."""
    from long_context_lm_amd import attn_bwd, attn_fwd_train
    print("[case] read-out bwd B=8 T=2048", flush=True)
    p, cot, (q, k, v), kw = _setup(8, 2048, 16, 4, train_len=2048)
    fwd = attn_fwd_train(q, k, v, want_attn=True, **kw)
    got = attn_bwd(q, k, v, fwd, cot, **kw)
    again = attn_bwd(q, k, v, fwd, cot, **kw)
    torch.cuda.synchronize()
    for n in GRAD_KEYS:
        assert torch.equal(got[n], again[n]), n
    batches = [0, 7]
    want = _oracle_grads(p, cot, 0, 0.0, batches=batches)
    sel = {n: got[n][batches] for n in ("dq", "dk", "dv")}
    assert_grads_close(sel, want, keys=("dq", "dk", "dv"), label="C2 read-out")

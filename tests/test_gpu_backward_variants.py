"""GPU parity of the variant modes' training forward and backward (sliding window, RoPE,
both) through the C ABI (polar_attn_fwd_train_variant, polar_attn_bwd_variant).

The reference is the float64 autograd oracle with the same window and rotation
(oracle.polar_prefill_grad, the rotated q and k rounded to bfloat16 as the kernels hold
them, that rounding passed through), under the causal backward's tolerances
(tests/parity.py).  The training forward's outputs are compared bit for bit with the
variant forward (polar_attn_fwd_variant), which computes the same rows in another
instance."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import GRAD_KEYS, assert_grads_close, host, to_dev

pytestmark = pytest.mark.gpu

OUTS = ("dir", "count", "n_eff", "gate", "lse")


def _setup(B, T, Hq, Hkv, seed=None, train_len=64):
    p = synth.prefill_inputs("c2", B=B, T=T, Hq=Hq, Hkv=Hkv, train_len=train_len, flags=3,
                             seed=seed)
    cot = synth.cotangents(p.B, p.T, p.Hq, p.d, seed=2003).as_dict()
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    kw = dict(beta=p.beta, null_bias=p.null_bias, count_vec=p.count_vec,
              train_len=p.train_len, flags=p.flags)
    return p, cot, (q, k, v), kw


def _oracle_grads(p, cot, window, theta, batches=None):
    sl = slice(None) if batches is None else list(batches)
    c = {n: np.asarray(x)[sl] for n, x in cot.items()}
    return oracle.polar_prefill_grad(p.as_f32("q")[sl], p.as_f32("k")[sl], p.as_f32("v")[sl],
                                     c, p.beta, p.null_bias, p.count_vec, p.train_len, p.flags,
                                     window=window, rope_theta=theta, rope_bf16=True)


@pytest.mark.parametrize("window,theta,B,T,Hq,Hkv", [
    (64, 0.0, 2, 300, 8, 2),          # window of one tile: every row block cut on the left
    (100, 0.0, 1, 257, 4, 1),         # a window that is no multiple of the tiles, GQA 4
    (1, 0.0, 1, 70, 4, 2),            # W = 1: each row sees only its own key
    (0, 10000.0, 2, 300, 8, 2),       # RoPE
    (0, 500.0, 1, 129, 4, 4),         # RoPE with a small base (fast turns), no GQA
    (96, 10000.0, 1, 400, 16, 4),     # both
])
def test_variant_backward_parity(gpu_lib, window, theta, B, T, Hq, Hkv):
    from long_context_lm_amd import attn_bwd, attn_fwd_train, attn_fwd_variant
    print(f"[case] variant bwd W={window} theta={theta} B={B} T={T} {Hq}/{Hkv}", flush=True)
    p, cot, (q, k, v), kw = _setup(B, T, Hq, Hkv)
    fwd = attn_fwd_train(q, k, v, window=window, rope_theta=theta, **kw)
    ref = attn_fwd_variant(q, k, v, window=window, rope_theta=theta, want_attn=False, **kw)
    torch.cuda.synchronize()
    for n in OUTS:
        assert torch.equal(fwd[n], ref[n]), n
    got = attn_bwd(q, k, v, fwd, cot, window=window, rope_theta=theta, **kw)
    torch.cuda.synchronize()
    assert_grads_close(got, _oracle_grads(p, cot, window, theta),
                       label=f"W{window} theta{theta}")


def test_variant_residuals(gpu_lib):
    """|u| against the oracle, and the arg-max key inside each row's window (where it
    differs from the oracle's, the two scores tie to fp32 rounding)."""
    from long_context_lm_amd import attn_fwd_train
    W, theta = 80, 10000.0
    p, cot, (q, k, v), kw = _setup(1, 333, 8, 2)
    fwd = attn_fwd_train(q, k, v, window=W, rope_theta=theta, **kw)
    torch.cuda.synchronize()
    want = oracle.polar_prefill(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.beta,
                                p.null_bias, p.count_vec, p.train_len, p.flags, window=W,
                                rope_theta=theta, rope_bf16=True)
    un = host(fwd["u_norm"])
    assert np.max(np.abs(un - want["u_norm"]) / want["u_norm"]) < 2e-2
    qr = oracle.round_bf16(oracle.rope(p.as_f32("q"), theta))
    kr = oracle.round_bf16(oracle.rope(p.as_f32("k"), theta))
    ref = oracle.arg_max_keys(qr, kr, p.beta, p.train_len, p.flags, window=W)
    am = fwd["arg_max"].cpu().numpy()
    i = np.arange(p.T)[None, :, None]
    assert np.all(am <= i) and np.all(am > i - W)
    G = p.Hq // p.Hkv
    for b, r, h in zip(*np.nonzero(am != ref)):
        d = qr[b, r, h] @ kr[b, am[b, r, h], h // G] - qr[b, r, h] @ kr[b, ref[b, r, h], h // G]
        assert abs(d) < 1e-5, (b, r, h)


def test_window_past_the_sequence_is_causal(gpu_lib):
    """A window longer than the sequence changes nothing: outputs, residuals and
    gradients bit-identical to the causal calls."""
    from long_context_lm_amd import attn_bwd, attn_fwd_train
    p, cot, (q, k, v), kw = _setup(2, 300, 8, 2)
    a = attn_fwd_train(q, k, v, window=5000, **kw)
    b = attn_fwd_train(q, k, v, **kw)
    torch.cuda.synchronize()
    for n in OUTS + ("u_norm", "arg_max"):
        assert torch.equal(a[n], b[n]), n
    ga = attn_bwd(q, k, v, a, cot, window=5000, **kw)
    gb = attn_bwd(q, k, v, b, cot, **kw)
    torch.cuda.synchronize()
    for n in GRAD_KEYS:
        assert torch.equal(ga[n], gb[n]), n


def test_variant_backward_training_shape(gpu_lib):
    """The 2K training shape (B=8, T=2048, 16/4 heads: the lean training instance and the
    full dk/dv grid) with a 512-key window and RoPE; sequences 0 and 7 against the oracle
    (dq, dk, dv of those sequences), and the run repeated bit for bit."""
    from long_context_lm_amd import attn_bwd, attn_fwd_train
    print("[case] variant bwd B=8 T=2048 W=512 RoPE", flush=True)
    p, cot, (q, k, v), kw = _setup(8, 2048, 16, 4, train_len=2048)
    fwd = attn_fwd_train(q, k, v, window=512, rope_theta=10000.0, **kw)
    got = attn_bwd(q, k, v, fwd, cot, window=512, rope_theta=10000.0, **kw)
    again = attn_bwd(q, k, v, fwd, cot, window=512, rope_theta=10000.0, **kw)
    torch.cuda.synchronize()
    for n in GRAD_KEYS:
        assert torch.equal(got[n], again[n]), n
    batches = [0, 7]
    want = _oracle_grads(p, cot, 512, 10000.0, batches=batches)
    sel = {n: got[n][batches] for n in ("dq", "dk", "dv")}
    assert_grads_close(sel, want, keys=("dq", "dk", "dv"), label="C2 W512 RoPE")


def test_fp32_training_variant_forward(gpu_lib):
    """fp32 inputs: the training forward of the window + RoPE arm (q and k rotated by the
    rotation kernel, no rounding) against the oracle at the fp32 bound, and its outputs
    against the fp32 variant forward (which rotates q at load) within fp32 rounding."""
    from long_context_lm_amd import attn_fwd_train, attn_fwd_variant
    from parity import TOL, assert_close
    W, theta = 70, 10000.0
    p = synth.prefill_inputs("c1", B=1, T=200, Hq=8, Hkv=2, dtype="f32")
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    kw = dict(beta=p.beta, null_bias=p.null_bias, count_vec=p.count_vec,
              train_len=p.train_len, flags=p.flags)
    fwd = attn_fwd_train(q, k, v, window=W, rope_theta=theta, **kw)
    ref = attn_fwd_variant(q, k, v, window=W, rope_theta=theta, want_attn=False, **kw)
    torch.cuda.synchronize()
    want = oracle.polar_prefill(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.beta,
                                p.null_bias, p.count_vec, p.train_len, p.flags, window=W,
                                rope_theta=theta)
    assert_close(fwd, want, p.count_vec, "f32", label="fp32 train variant")
    for n in OUTS:       # relative to each value's magnitude (n_eff runs to the hundreds)
        d = float(((fwd[n] - ref[n]).abs() / ref[n].abs().clamp(min=1.0)).max())
        assert d <= 1e-5, (n, d)
    un = host(fwd["u_norm"])
    assert np.max(np.abs(un - want["u_norm"]) / want["u_norm"]) < TOL["f32"]

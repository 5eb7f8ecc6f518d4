"""Pins of the oracle's variant modes (sliding window, RoPE, plain softmax output).

* the plain softmax output equals torch's scaled_dot_product_attention with the same
  causal (and windowed) mask and scale, GQA expanded by repeat_interleave;
* a windowed row equals the last causal row of the sliced sequence it sees;
* window 1 has closed forms; a window of at least T changes nothing;
* RoPE preserves norms, makes scores depend on position differences only, is the identity
  at position 0, and rotates one pair by pos * theta**(-2t/d);
* the bfloat16 rounding of rotated q and k is nearest-even, and leaves bfloat16 values
  (position 0) unchanged.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

OUTS = ("dir", "count", "n_eff", "gate", "lse", "attn")


def _inputs(seed, B=1, T=40, Hq=4, Hkv=2, d=8):
    rng = np.random.default_rng(seed)
    unit = lambda a: a / np.linalg.norm(a, axis=-1, keepdims=True)
    q = unit(rng.standard_normal((B, T, Hq, d)))
    k = unit(rng.standard_normal((B, T, Hkv, d)))
    v = rng.standard_normal((B, T, Hkv, d))
    beta = rng.uniform(3.0, 9.0, Hq)
    bias = rng.uniform(-0.5, 0.5, Hq)
    w = rng.standard_normal((Hq, d))
    return q, k, v, beta, bias, w


@pytest.mark.parametrize("window", [0, 1, 5, 17])
def test_softmax_output_matches_sdpa(window):
    q, k, v, beta, bias, w = _inputs(1)
    beta[:] = 2.5
    out = oracle.polar_prefill(q, k, v, beta, bias, w, 2048, 0, window=window)
    T = q.shape[1]
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    allowed = (j <= i) & ((j > i - window) if window > 0 else True)
    qt = torch.tensor(q).transpose(1, 2)
    kt = torch.tensor(k).transpose(1, 2).repeat_interleave(2, dim=1)
    vt = torch.tensor(v).transpose(1, 2).repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.tensor(allowed), scale=2.5).transpose(1, 2).numpy()
    np.testing.assert_allclose(out["attn"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window", [3, 11])
def test_window_row_equals_sliced_sequence(window):
    q, k, v, beta, bias, w = _inputs(2, T=30)
    train_len = 4
    out = oracle.polar_prefill(q, k, v, beta, bias, w, train_len, 3, window=window)
    for i in (0, window - 1, window, 29):
        lo = max(0, i - window + 1)
        sub = oracle.polar_prefill(q[:, lo:i + 1], k[:, lo:i + 1], v[:, lo:i + 1], beta, bias,
                                   w, train_len, 3)
        for n in OUTS:
            np.testing.assert_allclose(out[n][:, i], sub[n][:, -1], rtol=1e-12, atol=1e-12)


def test_window_one_closed_form():
    q, k, v, beta, bias, w = _inputs(3, T=12)
    out = oracle.polar_prefill(q, k, v, beta, bias, w, 4, 3, window=1)
    G = 2
    for i in range(12):
        for h in range(4):
            kk, vv = k[0, i, h // G], v[0, i, h // G]
            l = beta[h] * float(q[0, i, h] @ kk)                 # n = 1: tau = 1, floor = b_h
            assert out["n_eff"][0, i, h] == pytest.approx(1.0, abs=1e-12)
            np.testing.assert_allclose(out["dir"][0, i, h], vv / np.linalg.norm(vv), atol=1e-12)
            np.testing.assert_allclose(out["count"][0, i, h], 0.0, atol=1e-12)
            assert out["lse"][0, i, h] == pytest.approx(l, abs=1e-12)
            assert out["gate"][0, i, h] == pytest.approx(1 / (1 + math.exp(bias[h] - l)), abs=1e-12)


def test_window_at_least_T_is_no_window():
    q, k, v, beta, bias, w = _inputs(4, T=25)
    a = oracle.polar_prefill(q, k, v, beta, bias, w, 4, 3)
    b = oracle.polar_prefill(q, k, v, beta, bias, w, 4, 3, window=25)
    for n in OUTS:
        np.testing.assert_array_equal(a[n], b[n])


def test_rope_preserves_norm_and_is_identity_at_zero():
    q, *_ = _inputs(5, T=50, d=16)
    r = oracle.rope(q, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(q, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(r[:, 0], q[:, 0], atol=0)


def test_rope_scores_depend_on_position_difference_only():
    q, k, *_ = _inputs(6, T=20, d=16)
    a_q = oracle.rope(q, 500.0, positions=np.arange(20))
    a_k = oracle.rope(k, 500.0, positions=np.arange(20))
    b_q = oracle.rope(q, 500.0, positions=np.arange(20) + 1234)
    b_k = oracle.rope(k, 500.0, positions=np.arange(20) + 1234)
    sa = np.einsum("bihd,bjhd->bhij", a_q[:, :, :2], a_k)
    sb = np.einsum("bihd,bjhd->bhij", b_q[:, :, :2], b_k)
    np.testing.assert_allclose(sa, sb, atol=1e-11)


def test_rope_pair_rotation_closed_form():
    x = np.zeros((1, 3, 1, 4))
    x[..., 0] = 1.0                                   # pair t=0: (1, 0)
    x[..., 2] = 1.0                                   # pair t=1: (1, 0)
    r = oracle.rope(x, 100.0, positions=np.array([0.0, 1.0, 7.0]))
    for p_i, pos in enumerate([0.0, 1.0, 7.0]):
        np.testing.assert_allclose(r[0, p_i, 0, :2], [math.cos(pos), math.sin(pos)], atol=1e-15)
        a1 = pos * 100.0 ** (-2 * 1 / 4)              # theta^(-2t/d) with t = 1, d = 4
        np.testing.assert_allclose(r[0, p_i, 0, 2:], [math.cos(a1), math.sin(a1)], atol=1e-15)


def test_round_bf16_nearest_even_closed_forms():
    """bfloat16 keeps 8 significant bits: halfway cases go to the even neighbour."""
    r = oracle.polar_oracle.round_bf16
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -7, 1 + 2.0 ** -8 + 2.0 ** -20,
                  -3.0, 2.0 ** -100])
    want = np.array([1.0, 1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, 1 + 2.0 ** -7, -3.0, 2.0 ** -100])
    np.testing.assert_array_equal(r(x), want)


def test_rope_bf16_rounding_keeps_bf16_values_at_position_zero():
    """At position 0 the rotation is the identity, so rounding bf16 inputs changes nothing:
    a one-token prefill with RoPE in bfloat16 equals the plain prefill, while a
    non-bfloat16 input shows the rounding."""
    p = synth.prefill_inputs("c2", B=1, T=1, Hq=4, Hkv=2, train_len=16)
    args = (p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.beta, p.null_bias, p.count_vec,
            p.train_len, p.flags)
    a = oracle.polar_prefill(*args, rope_theta=10000.0, rope_bf16=True)
    b = oracle.polar_prefill(*args)
    for n in ("dir", "count", "n_eff", "gate", "lse"):
        np.testing.assert_array_equal(a[n], b[n])
    q = p.as_f32("q").astype(np.float64) * (1 + 2.0 ** -12)   # off the bf16 grid
    c = oracle.polar_prefill(q, *args[1:], rope_theta=10000.0, rope_bf16=True)
    d = oracle.polar_prefill(q, *args[1:], rope_theta=10000.0)
    assert np.any(c["lse"] != d["lse"])

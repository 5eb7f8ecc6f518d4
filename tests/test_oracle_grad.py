"""Pins of the float64 backward oracle (oracle.polar_grad) against things other than itself.

* central finite differences of the independent numpy forward oracle (every input and
  parameter element, tiny shapes, both flags on and off);
* torch's own scaled-dot-product-attention backward at tau = 1 (direction channel) and
  torch.logsumexp's (lse), with GQA expanded by repeat_interleave;
* closed forms: a single visible key (row 0) and identical keys, where the direction and
  n_eff terms of dq cancel and only the lse and gate terms remain.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

OUTS = ("dir", "count", "n_eff", "gate", "lse", "attn")


def _tiny(seed, B=1, T=6, Hq=2, Hkv=1, d=4):
    rng = np.random.default_rng(seed)
    unit = lambda a: a / np.linalg.norm(a, axis=-1, keepdims=True)
    q = unit(rng.standard_normal((B, T, Hq, d)))
    k = unit(rng.standard_normal((B, T, Hkv, d)))
    v = rng.standard_normal((B, T, Hkv, d))
    beta = rng.uniform(2.0, 6.0, Hq)
    bias = rng.uniform(-0.5, 0.5, Hq)
    w = rng.standard_normal((Hq, d))
    cot = dict(dir=rng.standard_normal((B, T, Hq, d)), count=rng.standard_normal((B, T, Hq, d)),
               n_eff=rng.standard_normal((B, T, Hq)), gate=rng.standard_normal((B, T, Hq)),
               lse=rng.standard_normal((B, T, Hq)), attn=rng.standard_normal((B, T, Hq, d)))
    return q, k, v, beta, bias, w, cot


def _loss_np(q, k, v, beta, bias, w, cot, train_len, flags, window=0, rope_theta=0.0):
    out = oracle.polar_prefill(q, k, v, beta, bias, w, train_len, flags, window=window,
                               rope_theta=rope_theta)
    return sum(float(np.sum(cot[n] * out[n])) for n in OUTS)


@pytest.mark.parametrize("flags,window,rope_theta", [
    (3, 0, 0.0), (0, 0, 0.0),
    (3, 3, 0.0),          # sliding window: rows 3.. lose their first keys, n = min(i+1, 3)
    (3, 0, 7.0),          # RoPE (a small base, so that every pair turns noticeably)
    (0, 2, 7.0),          # both
])
def test_grad_matches_finite_differences(flags, window, rope_theta):
    q, k, v, beta, bias, w, cot = _tiny(7 + flags + window)
    train_len = 2                                  # tau > 1 from the third row on
    g = oracle.polar_prefill_grad(q, k, v, cot, beta, bias, w, train_len, flags,
                                  window=window, rope_theta=rope_theta)
    args = dict(q=q, k=k, v=v, beta=beta, bias=bias, w=w)
    names = dict(q="dq", k="dk", v="dv", beta="d_beta", bias="d_null_bias", w="d_count_vec")
    var = dict(window=window, rope_theta=rope_theta)
    eps = 1e-6
    for name, arr in args.items():
        fd = np.zeros(arr.shape)
        for idx in np.ndindex(arr.shape):
            saved = arr[idx]
            arr[idx] = saved + eps
            lp = _loss_np(**args, cot=cot, train_len=train_len, flags=flags, **var)
            arr[idx] = saved - eps
            lm = _loss_np(**args, cot=cot, train_len=train_len, flags=flags, **var)
            arr[idx] = saved
            fd[idx] = (lp - lm) / (2 * eps)
        got = g[names[name]].reshape(arr.shape)
        scale = max(1.0, float(np.max(np.abs(fd))))
        assert np.max(np.abs(got - fd)) < 1e-6 * scale, (name, np.max(np.abs(got - fd)))


def test_forward_matches_numpy_oracle():
    q, k, v, beta, bias, w, cot = _tiny(3, B=2, T=40, Hq=4, Hkv=2, d=8)
    g = oracle.polar_prefill_grad(q, k, v, cot, beta, bias, w, 4, 3, return_outputs=True)
    ref = oracle.polar_prefill(q, k, v, beta, bias, w, 4, 3)
    for n in OUTS:
        np.testing.assert_allclose(g["outputs"][n], ref[n], rtol=1e-12, atol=1e-12)


def test_direction_and_lse_grads_match_torch_sdpa():
    """tau = 1, no floor: dir = normalize(SDPA(q,k,v; scale=beta)), lse = logsumexp."""
    q, k, v, beta, bias, w, cot = _tiny(11, B=2, T=33, Hq=4, Hkv=2, d=8)
    beta = np.full(4, 3.0)
    c = dict(dir=cot["dir"], lse=cot["lse"])
    g = oracle.polar_prefill_grad(q, k, v, c, beta, bias, w, 2048, 0)
    qt = torch.tensor(q).transpose(1, 2).contiguous().requires_grad_(True)   # [B,H,T,d]
    kt = torch.tensor(k).transpose(1, 2).contiguous().requires_grad_(True)
    vt = torch.tensor(v).transpose(1, 2).contiguous().requires_grad_(True)
    ke = kt.repeat_interleave(2, dim=1)
    ve = vt.repeat_interleave(2, dim=1)
    u = torch.nn.functional.scaled_dot_product_attention(qt, ke, ve, is_causal=True, scale=3.0)
    dir_ = u / u.norm(dim=-1, keepdim=True)
    T = q.shape[1]
    scores = 3.0 * qt @ ke.transpose(-1, -2)
    scores = scores.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)
    loss = (torch.tensor(cot["dir"]).transpose(1, 2) * dir_).sum() + \
        (torch.tensor(cot["lse"]).transpose(1, 2) * lse).sum()
    loss.backward()
    np.testing.assert_allclose(g["dq"], qt.grad.transpose(1, 2).numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(g["dk"], kt.grad.transpose(1, 2).numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(g["dv"], vt.grad.transpose(1, 2).numpy(), rtol=1e-10, atol=1e-10)


def test_softmax_readout_grads_match_torch_sdpa():
    """tau = 1: attn is exactly scaled-dot-product attention, so the gradients of an attn
    cotangent are torch's SDPA backward (GQA expanded by repeat_interleave); with a window,
    SDPA under the matching boolean mask."""
    q, k, v, beta, bias, w, cot = _tiny(23, B=2, T=30, Hq=4, Hkv=2, d=8)
    beta = np.full(4, 2.5)
    for window in (0, 7):
        g = oracle.polar_prefill_grad(q, k, v, dict(attn=cot["attn"]), beta, bias, w, 2048, 0,
                                      window=window)
        qt = torch.tensor(q).transpose(1, 2).contiguous().requires_grad_(True)
        kt = torch.tensor(k).transpose(1, 2).contiguous().requires_grad_(True)
        vt = torch.tensor(v).transpose(1, 2).contiguous().requires_grad_(True)
        T = q.shape[1]
        i = torch.arange(T)
        allowed = i[None, :] <= i[:, None]
        if window:
            allowed &= i[None, :] > i[:, None] - window
        u = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.repeat_interleave(2, dim=1), vt.repeat_interleave(2, dim=1),
            attn_mask=allowed, scale=2.5)
        (torch.tensor(cot["attn"]).transpose(1, 2) * u).sum().backward()
        for name, t in (("dq", qt), ("dk", kt), ("dv", vt)):
            np.testing.assert_allclose(g[name], t.grad.transpose(1, 2).numpy(), rtol=1e-10,
                                       atol=1e-10)
        assert np.all(g["d_count_vec"] == 0) and np.all(g["d_null_bias"] == 0)


def test_single_key_closed_form():
    """Row 0 sees one key: p = 1, n_eff = 1, dir = v0/|v0|, attn = v0,
    gate = sigmoid(beta q.k - b)."""
    q, k, v, beta, bias, w, cot = _tiny(5, T=1, Hq=2, Hkv=1, d=4)
    g = oracle.polar_prefill_grad(q, k, v, cot, beta, bias, w, 2048, 3)
    v0 = v[0, 0, 0]
    dir0 = v0 / np.linalg.norm(v0)
    dv = np.zeros(4)
    dk = np.zeros(4)
    for h in range(2):
        s = float(q[0, 0, h] @ k[0, 0, 0])
        gate = 1.0 / (1.0 + math.exp(-(beta[h] * s - bias[h])))
        coef = cot["lse"][0, 0, h] + cot["gate"][0, 0, h] * gate * (1 - gate)
        np.testing.assert_allclose(g["dq"][0, 0, h], coef * beta[h] * k[0, 0, 0], atol=1e-13)
        dk += coef * beta[h] * q[0, 0, h]
        cd = cot["dir"][0, 0, h]
        dv += (cd - dir0 * (dir0 @ cd)) / np.linalg.norm(v0)
        dv += cot["attn"][0, 0, h]                     # attn = v0, whatever the logit
        np.testing.assert_allclose(g["d_beta"][h], coef * s, atol=1e-13)
        np.testing.assert_allclose(g["d_null_bias"][h], -cot["gate"][0, 0, h] * gate * (1 - gate),
                                   atol=1e-13)
        np.testing.assert_allclose(g["d_count_vec"][h], 0.0, atol=1e-13)   # tanh(log 1) = 0
    np.testing.assert_allclose(g["dk"][0, 0, 0], dk, atol=1e-13)
    np.testing.assert_allclose(g["dv"][0, 0, 0], dv, atol=1e-13)


def test_identical_keys_dq_closed_form():
    """All keys equal: the softmax is uniform, so the direction and n_eff terms of dl sum
    to zero and dq_i = beta*tau_i*(c_lse + (c_gate + th_i*(c_count.w)) gate(1-gate)) kbar."""
    q, k, v, beta, bias, w, cot = _tiny(9, B=1, T=12, Hq=2, Hkv=1, d=4)
    k[:] = k[0, 0, 0]
    train_len = 4
    g = oracle.polar_prefill_grad(q, k, v, cot, beta, bias, w, train_len, 3)
    out = oracle.polar_prefill(q, k, v, beta, bias, w, train_len, 3)
    kbar = k[0, 0, 0]
    for i in range(12):
        n = i + 1
        tau = max(1.0, math.log(n) / math.log(train_len))
        th = (n * n - 1.0) / (n * n + 1.0)
        for h in range(2):
            gate = out["gate"][0, i, h]
            dg = cot["gate"][0, i, h] + th * float(cot["count"][0, i, h] @ w[h])
            coef = beta[h] * tau * (cot["lse"][0, i, h] + dg * gate * (1 - gate))
            np.testing.assert_allclose(g["dq"][0, i, h], coef * kbar, atol=1e-11)


def test_arg_max_keys_first_occurrence():
    q, k, v, beta, bias, w, cot = _tiny(13, B=1, T=20, Hq=2, Hkv=1, d=4)
    k[0, 5] = k[0, 2]                              # exact tie between keys 2 and 5
    j = oracle.arg_max_keys(q, k, beta, 2048, 3)
    for i in range(20):
        for h in range(2):
            L = [beta[h] * float(q[0, i, h] @ k[0, jj, 0]) for jj in range(i + 1)]
            assert j[0, i, h] == L.index(max(L))


def test_arg_max_keys_window():
    """With a window W the maximum is taken over keys max(0, i-W+1)..i only."""
    q, k, v, beta, bias, w, cot = _tiny(17, B=1, T=12, Hq=2, Hkv=1, d=4)
    j = oracle.arg_max_keys(q, k, beta, 2048, 0, window=4)
    for i in range(12):
        for h in range(2):
            lo = max(0, i - 3)
            L = [float(q[0, i, h] @ k[0, jj, 0]) for jj in range(lo, i + 1)]
            assert j[0, i, h] == lo + L.index(max(L))


def test_rope_bf16_rounding_passes_gradients_through():
    """With rope_bf16 the forward sees bfloat16-rounded rotations (equal to the numpy
    oracle's rope_bf16 outputs) and the gradients are those of the rounded point taken as
    exact: here, the direction cotangent against torch's SDPA backward on the rounded
    rotations, carried back through the transposed rotation."""
    q, k, v, beta, bias, w, cot = _tiny(19, B=1, T=9, Hq=2, Hkv=1, d=8)
    g = oracle.polar_prefill_grad(q, k, v, dict(dir=cot["dir"]), np.full(2, 3.0), bias, w,
                                  2048, 0, return_outputs=True, rope_theta=50.0,
                                  rope_bf16=True)
    ref = oracle.polar_prefill(q, k, v, np.full(2, 3.0), bias, w, 2048, 0, rope_theta=50.0,
                               rope_bf16=True)
    np.testing.assert_allclose(g["outputs"]["dir"], ref["dir"], rtol=1e-12, atol=1e-12)
    qr = torch.tensor(oracle.round_bf16(oracle.rope(q, 50.0))).transpose(1, 2).requires_grad_(True)
    kr = torch.tensor(oracle.round_bf16(oracle.rope(k, 50.0))).transpose(1, 2).requires_grad_(True)
    vt = torch.tensor(v).transpose(1, 2)
    u = torch.nn.functional.scaled_dot_product_attention(
        qr, kr.repeat_interleave(2, dim=1), vt.repeat_interleave(2, dim=1), is_causal=True,
        scale=3.0)
    (torch.tensor(cot["dir"]).transpose(1, 2) * (u / u.norm(dim=-1, keepdim=True))).sum().backward()
    # The transposed rotation is the rotation by the opposite angle.
    dq = oracle.rope(qr.grad.transpose(1, 2).numpy(), 50.0, -np.arange(9.0))
    dk = oracle.rope(kr.grad.transpose(1, 2).numpy(), 50.0, -np.arange(9.0))
    np.testing.assert_allclose(g["dq"], dq, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(g["dk"], dk, rtol=1e-10, atol=1e-10)


def test_cotangents_seeded():
    a = synth.cotangents(1, 8, 2, 4, seed=5)
    b = synth.cotangents(1, 8, 2, 4, seed=5)
    assert all(np.array_equal(getattr(a, f), getattr(b, f)) for f in
               ("d_dir", "d_count", "d_n_eff", "d_gate", "d_lse"))
    assert a.d_dir.dtype == np.float32 and a.d_dir.shape == (1, 8, 2, 4)


def test_readout_cotangent_leaves_the_others_unchanged():
    """Asking for the read-out's cotangent draws it from a sixth child stream: the five
    others are the same arrays, and "attn" appears in the dict only when asked for."""
    a = synth.cotangents(2, 8, 3, 4, seed=11)
    b = synth.cotangents(2, 8, 3, 4, seed=11, attn=True)
    assert "attn" not in a.as_dict() and b.as_dict()["attn"].shape == (2, 8, 3, 4)
    for n, x in a.as_dict().items():
        assert np.array_equal(x, b.as_dict()[n]), n
    assert not np.array_equal(b.d_attn, b.d_dir)

"""Float64 reverse-mode oracle of the causal Polar Attention prefill (the backward pass).

TEST INFRASTRUCTURE: imported only by tests/, ``__graft_entry__.smoke()`` and bench.py's
``cpu_baseline`` legs.  It shares no code with the HIP path.

The forward is written out again with torch CPU tensors in float64 (the definitions of
the "ATMA: Length-Invariant Language Modeling via Polar Attention and Gated-Delta
Compression Memory" technical summary, section 2.1, under the readings of the numpy
oracle in ``polar_oracle``: length temperature, extreme-value floor, sigmoid gate,
tanh(log n_eff) count).  Gradients come from ``torch.autograd`` on the scalar

    L = sum(c_dir * dir) + sum(c_count * count) + sum(c_n_eff * n_eff)
        + sum(c_gate * gate) + sum(c_lse * lse) [+ sum(c_attn * attn)]

for caller-given cotangents c_*, with respect to q, k, v and the per-head parameters
beta, null_bias and count_vec.

The row maximum m = max_j l_j that drives the gate is non-differentiable at ties; the
reading taken is the usual subgradient that routes d m entirely to the first key (lowest
position) attaining the maximum.

The variant modes of the forward (the same section's comparison arms) are taken as the
numpy oracle takes them: a sliding window W restricts row i to keys max(0, i-W+1)..i and
its key count n = min(i+1, W) drives tau and the floor; RoPE (RoFormer's rotary position
embedding, pair (2t, 2t+1) of position p turned by p * theta^(-2t/d)) rotates q and k
before the scores, and the gradients reach the unrotated q and k through the rotation.
With ``rope_bf16`` the rotated vectors are rounded to bfloat16 in the forward, as a
bfloat16 model holds them; the rounding passes gradients through unchanged.

Pins (tests/test_oracle_grad.py): central finite differences of the independent numpy
oracle on tiny inputs (also with a window and with RoPE), torch's own
scaled-dot-product-attention backward at tau = 1, and closed forms (a single visible key;
identical keys, where the direction and n_eff terms cancel from dq).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

FLAG_LENGTH_TEMP = 1
FLAG_NULL_FLOOR = 2

# The five Polar outputs, and the plain softmax read-out ("attn" = sum_j p_j v_j, the
# "Softmax + Memory" arm of the pages' ablation), which may also carry a cotangent.
_OUT = ("dir", "count", "n_eff", "gate", "lse", "attn")


def _rows_forward(Qr, K, V, hi, lo, beta_h, bias_h, w_h, train_len: int, flags: int):
    """Polar outputs of rows Qr [R,d] over keys K[lo[r]:hi[r]], as torch float64 graphs."""
    R, d = Qr.shape
    nmax = int(hi.max())
    n = torch.as_tensor(hi - lo, dtype=torch.float64)        # keys each row sees
    if flags & FLAG_LENGTH_TEMP:
        tau = torch.clamp(torch.log(n) / math.log(train_len), min=1.0)
    else:
        tau = torch.ones_like(n)
    S = Qr @ K[:nmax].T
    logits = (beta_h * tau)[:, None] * S
    j = torch.arange(nmax)[None, :]
    visible = (j < torch.as_tensor(hi)[:, None]) & (j >= torch.as_tensor(lo)[:, None])
    logits = logits.masked_fill(~visible, float("-inf"))
    jstar = torch.as_tensor(np.argmax(logits.detach().numpy(), axis=1))   # first maximum
    m = logits.gather(1, jstar[:, None])[:, 0]
    e = torch.exp(logits - m[:, None])
    Z = e.sum(dim=1)
    p = e / Z[:, None]
    lse = m + torch.log(Z)
    n_eff = 1.0 / (p * p).sum(dim=1)
    u = p @ V[:nmax]
    norm = torch.sqrt((u * u).sum(dim=1))
    dir_ = u / norm[:, None]
    floor = bias_h + torch.zeros_like(n)
    if flags & FLAG_NULL_FLOOR:
        floor = floor + (beta_h * tau / math.sqrt(d)) * torch.sqrt(2.0 * torch.log(n))
    gate = torch.sigmoid(m - floor)
    count = (gate * torch.tanh(torch.log(n_eff)))[:, None] * w_h[None, :]
    return dict(dir=dir_, count=count, n_eff=n_eff, gate=gate, lse=lse, attn=u)


def _rotate(x, theta: float, bf16: bool):
    """RoPE of x [B,T,H,d] (float64 torch graph) at positions 0..T-1; with ``bf16`` the
    result is rounded to bfloat16 in value, its gradient passed through unchanged."""
    T, d = x.shape[1], x.shape[3]
    freq = theta ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * freq[None, :]      # [T, d/2]
    c, s = torch.cos(ang)[None, :, None, :], torch.sin(ang)[None, :, None, :]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = torch.stack((x0 * c - x1 * s, x0 * s + x1 * c), dim=-1).reshape(x.shape)
    if bf16:
        yr = y.detach().to(torch.float32).to(torch.bfloat16).to(torch.float64)
        y = y + (yr - y).detach()
    return y


def polar_prefill_grad(q, k, v, cot: dict, beta=None, null_bias=None, count_vec=None,
                       train_len: int = 2048, flags: int = FLAG_LENGTH_TEMP | FLAG_NULL_FLOOR,
                       max_elems: int = 1 << 21, return_outputs: bool = False,
                       window: int = 0, rope_theta: float = 0.0,
                       rope_bf16: bool = False) -> dict:
    """Gradients of the causal prefill with respect to q, k, v, beta, null_bias, count_vec.

    q [B,T,Hq,d], k and v [B,T,Hkv,d]; ``cot`` maps output names ("dir", "count",
    "n_eff", "gate", "lse", and "attn" for the plain softmax read-out) to cotangents of
    the output shapes (a missing name means zero).  ``window``, ``rope_theta`` and
    ``rope_bf16`` select the variant modes as in ``polar_prefill`` (0 = off).  Rows are processed in blocks of about ``max_elems``
    scores, each block's graph differentiated on its own; gradients accumulate in the
    leaves.  Returns float64 numpy arrays dq, dk, dv, d_beta [Hq], d_null_bias [Hq],
    d_count_vec [Hq,d] (and the forward outputs when ``return_outputs``).
    """
    q = np.asarray(q)
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    f64 = lambda a: torch.tensor(np.asarray(a, np.float64))
    qt = f64(q).requires_grad_(True)
    kt = f64(k).requires_grad_(True)
    vt = f64(v).requires_grad_(True)
    bt = f64(np.full(Hq, math.sqrt(d)) if beta is None else beta).requires_grad_(True)
    nb = f64(np.zeros(Hq) if null_bias is None else null_bias).requires_grad_(True)
    wt = f64(np.zeros((Hq, d)) if count_vec is None
             else np.asarray(count_vec).reshape(Hq, d)).requires_grad_(True)
    cts = {name: f64(cot[name]) for name in _OUT if cot.get(name) is not None}
    outs = {name: np.zeros((B, T, Hq, d) if name in ("dir", "count", "attn") else (B, T, Hq))
            for name in _OUT} if return_outputs else None
    for b in range(B):
        for h in range(Hq):
            g = h // G
            r0 = 0
            while r0 < T:
                r1 = min(T, r0 + max(1, max_elems // max(1, T)))
                rows = np.arange(r0, r1)
                lo = np.maximum(0, rows - window + 1) if window > 0 else np.zeros_like(rows)
                # The rotation is recomputed per block, inside the block's own graph.
                qb, kb = qt[b:b + 1, r0:r1, h:h + 1], kt[b:b + 1, :, g:g + 1]
                if rope_theta > 0:
                    qb = _rotate(qt[b:b + 1, :r1, h:h + 1], rope_theta, rope_bf16)[:, r0:r1]
                    kb = _rotate(kb, rope_theta, rope_bf16)
                res = _rows_forward(qb[0, :, 0], kb[0, :, 0], vt[b, :, g], rows + 1, lo,
                                    bt[h], nb[h], wt[h], train_len, flags)
                loss = torch.zeros((), dtype=torch.float64)
                for name, c in cts.items():
                    loss = loss + (c[b, r0:r1, h] * res[name]).sum()
                if loss.requires_grad:
                    loss.backward()
                if outs is not None:
                    for name in _OUT:
                        outs[name][b, r0:r1, h] = res[name].detach().numpy()
                r0 = r1

    def grad(t):
        return np.zeros(tuple(t.shape)) if t.grad is None else t.grad.numpy().copy()

    r = dict(dq=grad(qt), dk=grad(kt), dv=grad(vt), d_beta=grad(bt), d_null_bias=grad(nb),
             d_count_vec=grad(wt))
    if outs is not None:
        r["outputs"] = outs
    return r


def arg_max_keys(q, k, beta=None, train_len: int = 2048,
                 flags: int = FLAG_LENGTH_TEMP | FLAG_NULL_FLOOR, window: int = 0) -> np.ndarray:
    """First key position attaining each row's maximum logit, [B,T,Hq] int64 (float64).
    q and k are taken as given (rotate them first for RoPE); ``window`` as in
    ``polar_prefill_grad``."""
    q = np.asarray(q, np.float64)
    B, T, Hq, d = q.shape
    G = Hq // k.shape[2]
    beta = np.full(Hq, math.sqrt(d)) if beta is None else np.asarray(beta, np.float64)
    out = np.zeros((B, T, Hq), np.int64)
    i = np.arange(T)
    n = (np.minimum(i + 1, window) if window > 0 else i + 1).astype(np.float64)
    tau = np.maximum(1.0, np.log(n) / math.log(train_len)) if flags & FLAG_LENGTH_TEMP else np.ones(T)
    hidden = i[None, :] > i[:, None]
    if window > 0:
        hidden |= i[None, :] <= i[:, None] - window
    for b in range(B):
        for h in range(Hq):
            S = q[b, :, h] @ np.asarray(k[b, :, h // G], np.float64).T
            L = (beta[h] * tau)[:, None] * S
            L[hidden] = -np.inf
            out[b, :, h] = np.argmax(L, axis=1)
    return out

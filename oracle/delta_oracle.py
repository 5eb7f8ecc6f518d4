"""Float64 CPU oracle of the gated-delta memory step (the recurrent memory stream).

TEST INFRASTRUCTURE: imported only by tests/, ``__graft_entry__.smoke()`` and bench.py's
``cpu_baseline`` legs.  It shares no code with the HIP path.

The "ATMA: Length-Invariant Language Modeling via Polar Attention and Gated-Delta
Compression Memory" technical summary (gist.science) adds to Polar Attention a third,
recurrent stream driven by a gated-delta memory derived from gated DeltaNet (section 2.1,
recurrent memory channel; the arXiv abstract), stabilised by L2-normalising its keys and
queries, and updated in place by a step kernel (section 2.2).  The pages print no update
rule; the reading taken is the published gated delta rule, one token per step:

    k <- k / |k|,  q <- q / |q|
    S' = alpha * S (I - beta k k^T) + beta v k^T          S: [d_v, d_k]
    o  = S' q

with per-(sequence, head) gate alpha and write strength beta.  Written out literally
(identity matrix, outer products), in float64.

The memory stream over a sequence (``delta_sequence_pool``) applies that step token after
token, in order, reading every output o_t and leaving the last state in the pool.
"""
from __future__ import annotations

import numpy as np


def l2_normalize(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-12)


def delta_step(S: np.ndarray, q, k, v, alpha, beta, normalize: bool = True):
    """One gated-delta step.  S [..., d_v, d_k]; q, k [..., d_k]; v [..., d_v]; alpha, beta
    [...].  Returns (S', o) in float64."""
    S = np.asarray(S, np.float64)
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    if normalize:
        q, k = l2_normalize(q), l2_normalize(k)
    a = np.asarray(alpha, np.float64)[..., None, None]
    b = np.asarray(beta, np.float64)[..., None, None]
    dk = S.shape[-1]
    eye = np.eye(dk)
    kkT = k[..., :, None] * k[..., None, :]
    vkT = v[..., :, None] * k[..., None, :]
    S_new = a * (S @ (eye - b * kkT)) + b * vkT
    o = (S_new @ q[..., :, None])[..., 0]
    return S_new, o


def delta_step_pool(pool: np.ndarray, slots, q, k, v, alpha, beta, normalize: bool = True):
    """The step on states held in a pool [num_slots, H, d_v, d_k]: sequence b updates
    pool[slots[b]] in place (a copy is returned).  Sequences with a slot outside the pool
    are skipped (their outputs are zero).  q, k [B,H,d_k]; v [B,H,d_v]; alpha, beta [B,H]."""
    pool = np.array(pool, np.float64)
    B, H = np.asarray(q).shape[:2]
    out = np.zeros((B, H, np.asarray(v).shape[-1]))
    for b in range(B):
        s = int(slots[b])
        if not 0 <= s < pool.shape[0]:
            continue
        pool[s], out[b] = delta_step(pool[s], q[b], k[b], v[b], alpha[b], beta[b], normalize)
    return pool, out


def delta_sequence_pool(pool: np.ndarray, slots, q, k, v, alpha, beta, normalize: bool = True):
    """The memory stream over T tokens for B sequences whose states sit in a pool
    [num_slots, H, d_v, d_k]: for t = 0..T-1 in order, S <- step(S, q_t, k_t, v_t, alpha_t,
    beta_t) and o_t = S q_t.  q, k [B,T,H,d_k]; v [B,T,H,d_v]; alpha, beta [B,T,H].
    Returns (pool with the final states, o [B,T,H,d_v]) in float64; sequences whose slot
    lies outside the pool are skipped (zero outputs)."""
    pool = np.array(pool, np.float64)
    q, k, v = (np.asarray(a) for a in (q, k, v))
    B, T, H = q.shape[:3]
    out = np.zeros((B, T, H, v.shape[-1]))
    for b in range(B):
        s = int(slots[b])
        if not 0 <= s < pool.shape[0]:
            continue
        S = pool[s]
        for t in range(T):
            S, out[b, t] = delta_step(S, q[b, t], k[b, t], v[b, t], alpha[b, t], beta[b, t],
                                      normalize)
        pool[s] = S
    return pool, out

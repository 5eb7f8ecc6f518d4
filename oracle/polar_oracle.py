"""Plain float64 CPU oracle of the Polar Attention forward (prefill and paged decode).

TEST INFRASTRUCTURE: imported only by tests/, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` legs of bench.py.  It shares no code with the HIP path.

What it computes follows the "ATMA: Length-Invariant Language Modeling via Polar Attention
and Gated-Delta Compression Memory" technical summary (gist.science), section 2.1
"Polar Attention: A Three-Channel Decomposition":

* Direction channel: the softmax-weighted ("matched") value sum projected onto the unit
  sphere, under a length-temperature logit scale.
* Magnitude channel: the participation ratio (inverse Simpson index) n_eff = 1 / sum p^2,
  gated by a signal-detection confidence against an extreme-value-corrected null floor and
  mapped through tanh(log n_eff) onto a per-head vector.
* out = content + count + memory; the memory stream is not part of this operation, so
  ``dir`` (content) and ``count`` are returned separately, and ``three_streams`` forms the
  sum from them and a memory-stream output.

The pages fix no formula for the temperature, the floor or the gate.  Readings taken here
(each one is listed with its reason in the design notes):
  tau(n)   = max(1, ln n / ln T_train)                   (length temperature)
  l_j      = beta_h * tau(n) * <q, k_j>                  (logit; q, k are unit vectors)
  floor(n) = b_h + (beta_h * tau(n) / sqrt(d)) * sqrt(2 ln n)
             (leading-order expected maximum of n standard noise logits of std
              beta_h*tau/sqrt(d), plus a per-head null scalar)
  gate     = sigmoid(max_j l_j - floor(n))
  count    = gate * tanh(ln n_eff) * w_h
with n the number of keys the row sees (i+1 in causal prefill, the sequence length in
decode) and query head h reading KV head floor(h / (Hq/Hkv)).

Parity pins: closed forms (uniform and one-hot rows, two-level rows, tau and floor values),
the first causal row, unit-norm direction, a library softmax-attention cross-check at
tau = 1, count-blindness under key duplication, count bounds and monotonicity, and a
pure-Python brute force on tiny inputs.  The *forms* of tau, floor and gate above are
pinned only by the definitions written here ("parity unpinned" by the pages).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch
from scipy.special import expit

FLAG_LENGTH_TEMP = 1
FLAG_NULL_FLOOR = 2


def length_temperature(n, train_len: int, on: bool) -> np.ndarray:
    """Length temperature tau(n) = max(1, ln n / ln T_train); 1 when switched off.

    The pages say only that the temperature sharpens distributions as context grows
    (section 2.1, direction channel); log-length scaling equal to 1 up to the
    training length is the reading taken.
    """
    n = np.asarray(n, dtype=np.float64)
    if not on:
        return np.ones_like(n)
    return np.maximum(1.0, np.log(n) / math.log(train_len))


def null_floor(n, beta_h: float, tau, d: int, null_bias_h: float, on: bool) -> np.ndarray:
    """Extreme-value-corrected null floor: b_h + sigma * sqrt(2 ln n), sigma = beta*tau/sqrt(d).

    For unit q and random unit k, <q,k> has variance 1/d, so a noise logit has standard
    deviation beta*tau/sqrt(d); sigma*sqrt(2 ln n) is the leading-order expected maximum
    of n such logits (section 2.1: the floor calibrates logits against random noise).
    """
    n = np.asarray(n, dtype=np.float64)
    base = np.full_like(n, float(null_bias_h))
    if not on:
        return base
    sigma = beta_h * np.asarray(tau, dtype=np.float64) / math.sqrt(d)
    return base + sigma * np.sqrt(2.0 * np.log(n))


def _polar_rows(Qr: np.ndarray, K: np.ndarray, V: np.ndarray, n_vis: np.ndarray,
                beta_h: float, null_bias_h: float, w_h: np.ndarray, train_len: int,
                flags: int, lo: Optional[np.ndarray] = None) -> dict:
    """Polar outputs for query rows Qr [R,d] attending keys K[lo[r]:n_vis[r]] (float64).

    ``lo`` (default 0) is the first visible key of each row; the row sees n = n_vis - lo
    keys, and that n drives the temperature and the floor.  Full score rows are formed (no
    streaming): scores, mask, max, exponentials, then the normalised probabilities in a
    second pass.
    """
    R, d = Qr.shape
    lo = np.zeros_like(n_vis) if lo is None else np.asarray(lo)
    n_keys = n_vis - lo
    nmax = int(n_vis.max())
    S = Qr @ K[:nmax].T                                        # raw cosines [R, nmax]
    tau = length_temperature(n_keys, train_len, bool(flags & FLAG_LENGTH_TEMP))
    logits = (beta_h * tau)[:, None] * S
    cols = np.arange(nmax)[None, :]
    visible = (cols < n_vis[:, None]) & (cols >= lo[:, None])
    logits = np.where(visible, logits, -np.inf)
    m = logits.max(axis=1)                                     # row maximum logit
    e = np.exp(logits - m[:, None])                            # masked entries -> 0
    Z = e.sum(axis=1)
    p = e / Z[:, None]                                         # attention distribution
    lse = m + np.log(Z)
    n_eff = 1.0 / np.sum(p * p, axis=1)                        # inverse Simpson index
    u = p @ V[:nmax]                                           # matched value sum
    norm = np.sqrt(np.sum(u * u, axis=1))
    dir_ = np.divide(u, norm[:, None], out=np.zeros_like(u), where=norm[:, None] > 0)
    floor = null_floor(n_keys, beta_h, tau, d, null_bias_h, bool(flags & FLAG_NULL_FLOOR))
    gate = expit(m - floor)
    count = (gate * np.tanh(np.log(n_eff)))[:, None] * np.asarray(w_h, np.float64)[None, :]
    return dict(dir=dir_, count=count, n_eff=n_eff, gate=gate, lse=lse, u_norm=norm, attn=u)


def rope(x: np.ndarray, theta: float, positions: Optional[np.ndarray] = None) -> np.ndarray:
    """Rotary position embedding of RoFormer (Su et al.): for each pair of dimensions
    (2t, 2t+1) a rotation by the angle pos * theta**(-2t/d).  x [B,T,H,d]; position of
    row t is t unless ``positions`` [T] says otherwise.  float64."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    pos = np.arange(x.shape[1], dtype=np.float64) if positions is None else \
        np.asarray(positions, np.float64)
    freq = theta ** (-np.arange(0, d, 2, dtype=np.float64) / d)          # [d/2]
    ang = pos[:, None] * freq[None, :]                                    # [T, d/2]
    c, s = np.cos(ang)[None, :, None, :], np.sin(ang)[None, :, None, :]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 values rounded to bfloat16 (torch's conversion: nearest, ties to even) and
    widened back to float64.  Values are first narrowed to float32, which is exact for
    the rounding to bfloat16 except in a double-rounding tie far below these tensors'
    scale."""
    t = torch.from_numpy(np.ascontiguousarray(x, np.float64)).to(torch.float32)
    return t.to(torch.bfloat16).to(torch.float64).numpy()


def _params(Hq, d, beta, null_bias, count_vec):
    beta = np.full(Hq, math.sqrt(d)) if beta is None else np.asarray(beta, np.float64)
    null_bias = np.zeros(Hq) if null_bias is None else np.asarray(null_bias, np.float64)
    count_vec = (np.zeros((Hq, d)) if count_vec is None
                 else np.asarray(count_vec, np.float64).reshape(Hq, d))
    return beta, null_bias, count_vec


def polar_prefill(q, k, v, beta=None, null_bias=None, count_vec=None, train_len: int = 2048,
                  flags: int = FLAG_LENGTH_TEMP | FLAG_NULL_FLOOR,
                  rows: Optional[np.ndarray] = None, heads: Optional[np.ndarray] = None,
                  batches: Optional[np.ndarray] = None, max_elems: int = 1 << 24,
                  window: int = 0, rope_theta: float = 0.0, rope_bf16: bool = False) -> dict:
    """Causal Polar Attention prefill.

    Variants: ``window`` W >= 1 restricts row i to keys max(0, i-W+1)..i (so it sees
    n = min(i+1, W) keys); ``rope_theta`` > 0 rotates q and k by RoPE at their positions
    before the scores.  ``attn`` is the plain softmax attention output sum_j p_j v_j.
    ``rope_bf16``: the model works in bfloat16, so the rotated q and k it attends with are
    bfloat16 values: the exact rotation is rounded to bfloat16 (nearest, ties to even)
    before the scores.

    q [B,T,Hq,d], k and v [B,T,Hkv,d] (any float dtype; computed in float64).
    Row i of head h sees keys 0..i of KV head h // (Hq // Hkv).
    ``rows``/``heads``/``batches`` restrict the computation to a sample; the outputs are
    then indexed [len(batches), len(rows), len(heads), ...].
    Returns float64 dir, count, attn [B,R,H,d] and n_eff, gate, lse [B,R,H], plus u_norm
    [B,R,H], the norm |u| of the matched value sum (a residual of the backward pass).
    """
    if rope_theta > 0:
        q, k = rope(q, rope_theta), rope(k, rope_theta)
        if rope_bf16:
            q, k = round_bf16(q), round_bf16(k)
    q = np.asarray(q)
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    assert Hq % Hkv == 0
    G = Hq // Hkv
    beta, null_bias, count_vec = _params(Hq, d, beta, null_bias, count_vec)
    rows = np.arange(T) if rows is None else np.asarray(rows, np.int64)
    heads = np.arange(Hq) if heads is None else np.asarray(heads, np.int64)
    batches = np.arange(B) if batches is None else np.asarray(batches, np.int64)
    R, H, Bs = len(rows), len(heads), len(batches)
    out = dict(dir=np.zeros((Bs, R, H, d)), count=np.zeros((Bs, R, H, d)),
               n_eff=np.zeros((Bs, R, H)), gate=np.zeros((Bs, R, H)), lse=np.zeros((Bs, R, H)),
               u_norm=np.zeros((Bs, R, H)), attn=np.zeros((Bs, R, H, d)))
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            g = h // G
            K = np.asarray(k[b, :, g], np.float64)
            V = np.asarray(v[b, :, g], np.float64)
            r0 = 0
            while r0 < R:
                # row block sized so the score block stays about max_elems doubles
                n_hi = int(rows[r0]) + 1
                r1 = r0 + 1
                while r1 < R and (r1 - r0 + 1) * max(n_hi, int(rows[r1]) + 1) <= max_elems:
                    n_hi = max(n_hi, int(rows[r1]) + 1)
                    r1 += 1
                sel = rows[r0:r1]
                lo = np.maximum(0, sel - window + 1) if window > 0 else None
                res = _polar_rows(np.asarray(q[b, sel, h], np.float64), K, V, sel + 1,
                                  beta[h], null_bias[h], count_vec[h], train_len, flags, lo)
                for key in out:
                    out[key][bi, r0:r1, hi] = res[key]
                r0 = r1
    return out


def three_streams(fwd: dict, memory=None) -> np.ndarray:
    """The layer output of section 2.1, out = content + count + memory, in float64: the
    prefill's ``dir`` (content) plus its ``count`` (zero when the prefill had no count
    vector) plus the memory stream's output for the same token and head (zero when None).
    All three are [B,T,Hq,d]."""
    out = np.asarray(fwd["dir"], np.float64).copy()
    if fwd.get("count") is not None:
        out = out + np.asarray(fwd["count"], np.float64)
    if memory is not None:
        out = out + np.asarray(memory, np.float64)
    return out


def gather_pages(pool: np.ndarray, page_table_row: np.ndarray, kv_head: int, length: int,
                 page_size: int) -> np.ndarray:
    """Logical [length, d] keys (or values) of one sequence from a paged pool.

    Pool layout [num_pages, Hkv, page_size, d]; logical token t lives in physical page
    page_table_row[t // page_size], slot t % page_size.
    """
    n_pages = -(-length // page_size)
    ids = np.asarray(page_table_row[:n_pages], np.int64)
    blk = pool[ids, kv_head]                                   # [n_pages, page_size, d]
    return blk.reshape(n_pages * page_size, -1)[:length]


def polar_decode_paged(q, k_pool, v_pool, page_table, seq_lens, page_size: int, beta=None,
                       null_bias=None, count_vec=None, train_len: int = 2048,
                       flags: int = FLAG_LENGTH_TEMP | FLAG_NULL_FLOOR,
                       to_f64=lambda a: np.asarray(a, np.float64),
                       batches: Optional[np.ndarray] = None) -> dict:
    """One-token decode over a paged KV cache.

    q [B,Hq,d]: the query of the newest token of each sequence, whose own key and value are
    already in the cache, so it sees all seq_lens[b] keys (the same as causal prefill row
    seq_lens[b]-1).  ``to_f64`` widens the pool storage (e.g. bf16 bit patterns).
    Returns float64 dir, count [B,Hq,d] and n_eff, gate, lse [B,Hq].
    """
    B, Hq, d = np.asarray(q).shape
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    beta, null_bias, count_vec = _params(Hq, d, beta, null_bias, count_vec)
    batches = np.arange(B) if batches is None else np.asarray(batches, np.int64)
    Bs = len(batches)
    out = dict(dir=np.zeros((Bs, Hq, d)), count=np.zeros((Bs, Hq, d)), n_eff=np.zeros((Bs, Hq)),
               gate=np.zeros((Bs, Hq)), lse=np.zeros((Bs, Hq)))
    qf = np.asarray(q, np.float64)
    for bi, b in enumerate(batches):
        L = int(seq_lens[b])
        for g in range(Hkv):
            K = to_f64(gather_pages(k_pool, page_table[b], g, L, page_size))
            V = to_f64(gather_pages(v_pool, page_table[b], g, L, page_size))
            for h in range(g * G, (g + 1) * G):
                res = _polar_rows(qf[b, h][None, :], K, V, np.array([L]), beta[h],
                                  null_bias[h], count_vec[h], train_len, flags)
                for key in out:
                    out[key][bi, h] = res[key][0]
    return out


def chunk_start(start_pos, C: int, max_seq_len: Optional[int]) -> np.ndarray:
    """Position of each chunk's first token.  The library's own rule (the pages say nothing
    of out-of-range starts): a start is clamped to [0, max_seq_len - C], so that the chunk
    fits the sequence bound and append and chunked prefill agree on where it lies."""
    s = np.asarray(start_pos, np.int64)
    if max_seq_len is None:
        return s
    assert max_seq_len >= C, "the sequence bound must hold the chunk"
    return np.minimum(np.maximum(s, 0), max_seq_len - C)


def kv_append(k_pool: np.ndarray, v_pool: np.ndarray, page_table: np.ndarray,
              start_pos: np.ndarray, k_new: np.ndarray, v_new: np.ndarray, page_size: int,
              max_seq_len: int):
    """Write a chunk of new keys and values into the paged pools (returns new pools).

    Token t of sequence b goes to logical position s + t (s = start_pos[b] clamped by
    ``chunk_start``), i.e. physical page page_table[b, pos // page_size], slot
    pos % page_size, for every KV head.  Tokens whose page id is outside the pool are
    dropped.
    """
    k_pool, v_pool = k_pool.copy(), v_pool.copy()
    B, C = k_new.shape[:2]
    num_pages = k_pool.shape[0]
    starts = chunk_start(start_pos, C, max_seq_len)
    for b in range(B):
        for t in range(C):
            pos = int(starts[b]) + t
            page = int(page_table[b, pos // page_size])
            if not 0 <= page < num_pages:
                continue
            k_pool[page, :, pos % page_size] = k_new[b, t]
            v_pool[page, :, pos % page_size] = v_new[b, t]
    return k_pool, v_pool


def polar_prefill_paged(q, k_pool, v_pool, page_table, start_pos, page_size: int, beta=None,
                        null_bias=None, count_vec=None, train_len: int = 2048,
                        flags: int = FLAG_LENGTH_TEMP | FLAG_NULL_FLOOR,
                        to_f64=lambda a: np.asarray(a, np.float64),
                        max_seq_len: Optional[int] = None) -> dict:
    """Chunked prefill over a paged cache: row t of sequence b is the token at position
    s + t (s = start_pos[b], clamped by ``chunk_start`` when ``max_seq_len`` is given) and
    attends the logical keys 0..s + t (the cached prefix and the chunk up to itself),
    gathered through the page table.
    q [B,C,Hq,d]; returns float64 dir, count [B,C,Hq,d] and n_eff, gate, lse [B,C,Hq].
    """
    q = np.asarray(q, np.float64)
    B, C, Hq, d = q.shape
    start_pos = chunk_start(start_pos, C, max_seq_len)
    Hkv = k_pool.shape[1]
    G = Hq // Hkv
    beta, null_bias, count_vec = _params(Hq, d, beta, null_bias, count_vec)
    out = dict(dir=np.zeros((B, C, Hq, d)), count=np.zeros((B, C, Hq, d)),
               n_eff=np.zeros((B, C, Hq)), gate=np.zeros((B, C, Hq)), lse=np.zeros((B, C, Hq)))
    for b in range(B):
        L = int(start_pos[b]) + C
        pos = int(start_pos[b]) + np.arange(C)
        for g in range(Hkv):
            K = to_f64(gather_pages(k_pool, page_table[b], g, L, page_size))
            V = to_f64(gather_pages(v_pool, page_table[b], g, L, page_size))
            for h in range(g * G, (g + 1) * G):
                res = _polar_rows(q[b, :, h], K, V, pos + 1, beta[h], null_bias[h],
                                  count_vec[h], train_len, flags)
                for key in out:
                    out[key][b, :, h] = res[key]
    return out

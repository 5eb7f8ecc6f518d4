"""Pins of the CPU oracle against closed forms, invariants and a library routine.

The Polar Attention pages ("ATMA" technical summary, section 2.1) print no worked example,
so the oracle is pinned by what the definitions fix mathematically:
  * n_eff is the inverse Simpson index: uniform rows give the key count, one-hot rows 1,
    k tied dominant keys give k, two-level rows a closed form;
  * the first causal row sees one key;
  * the direction is unit-norm and, at tau = 1, is the normalised output of a library
    softmax attention (torch CPU scaled_dot_product_attention);
  * the direction is count-blind: duplicating every key/value leaves it unchanged and
    multiplies n_eff by the duplication factor (section 2.1, direction channel);
  * count is bounded by gate * tanh(ln n_eff) * |w_h| and grows with n_eff;
  * decode of a length-L sequence equals prefill row L-1 and ignores page placement.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

OFF = 0
ON = oracle.FLAG_LENGTH_TEMP | oracle.FLAG_NULL_FLOOR


def unit(x):
    x = np.asarray(x, np.float64)
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def single_row(qv, K, V, beta=8.0, flags=OFF, w=None, b_h=0.0, train_len=2048):
    """Polar outputs of one query attending all rows of K, through the decode entry."""
    L, d = K.shape
    pool_k = K.reshape(L, 1, 1, d).transpose(0, 1, 2, 3)      # pages of one token
    pool_v = V.reshape(L, 1, 1, d)
    table = np.arange(L, dtype=np.int32)[None, :]
    w = np.zeros(d) if w is None else w
    o = oracle.polar_decode_paged(qv[None, None, :], pool_k, pool_v, table, np.array([L]), 1,
                                  beta=[beta], null_bias=[b_h], count_vec=w[None, :],
                                  train_len=train_len, flags=flags)
    return {key: val[0, 0] for key, val in o.items()}


# ---------------------------------------------------------------- n_eff closed forms
@pytest.mark.parametrize("n", [1, 2, 7, 64, 1000])
def test_uniform_row_neff_equals_key_count(n):
    g = np.random.default_rng(n)
    d = 16
    qv = unit(g.standard_normal(d))
    kv = unit(g.standard_normal(d))
    K = np.tile(kv, (n, 1))                                   # all keys identical
    V = g.standard_normal((n, d))
    r = single_row(qv, K, V, beta=5.0)
    assert abs(r["n_eff"] - n) <= 1e-12 * n
    # q orthogonal to every key: all logits 0
    K2 = np.zeros((n, d)); K2[:, 1] = 1.0
    q2 = np.zeros(d); q2[0] = 1.0
    r2 = single_row(q2, K2, V, beta=5.0)
    assert abs(r2["n_eff"] - n) <= 1e-12 * n
    assert abs(r2["lse"] - math.log(n)) < 1e-12


def test_one_hot_row_neff_is_one():
    g = np.random.default_rng(3)
    d, n = 32, 500
    qv = unit(g.standard_normal(d))
    K = unit(g.standard_normal((n, d)))
    K[123] = qv                                               # one aligned key
    V = g.standard_normal((n, d))
    r = single_row(qv, K, V, beta=1e3)
    assert abs(r["n_eff"] - 1.0) < 1e-9
    assert np.allclose(r["dir"], V[123] / np.linalg.norm(V[123]), atol=1e-9)


@pytest.mark.parametrize("ties", [1, 2, 5, 17])
def test_k_tied_dominant_keys_give_k(ties):
    g = np.random.default_rng(ties)
    d, n = 32, 300
    qv = unit(g.standard_normal(d))
    K = unit(g.standard_normal((n, d)))
    K -= (K @ qv)[:, None] * qv[None, :] * 1.2                # push others away from q
    K = unit(K)
    pos = g.choice(n, ties, replace=False)
    K[pos] = qv
    V = g.standard_normal((n, d))
    r = single_row(qv, K, V, beta=400.0)
    assert abs(r["n_eff"] - ties) < 1e-6 * ties


@pytest.mark.parametrize("a,c,x,y", [(3, 10, 1.0, 0.0), (1, 50, 2.5, -0.5), (7, 2, 0.3, 0.9)])
def test_two_level_row_closed_form(a, c, x, y):
    # logits beta*<q,k>: build keys with cosines x/beta and y/beta to q
    d, beta = 8, 4.0
    qv = np.zeros(d); qv[0] = 1.0
    def key(cos):
        k = np.zeros(d); k[0] = cos; k[1] = math.sqrt(1 - cos * cos); return k
    K = np.array([key(x / beta)] * a + [key(y / beta)] * c)
    V = np.random.default_rng(0).standard_normal((a + c, d))
    r = single_row(qv, K, V, beta=beta)
    want = (a * math.exp(x) + c * math.exp(y)) ** 2 / (a * math.exp(2 * x) + c * math.exp(2 * y))
    assert abs(r["n_eff"] - want) < 1e-12 * want
    assert abs(r["lse"] - math.log(a * math.exp(x) + c * math.exp(y))) < 1e-12


# ---------------------------------------------------------------- tau and floor
def test_length_temperature_values():
    tl = 2048
    n = np.array([1, 2, 2047, 2048, 4096, 16384, 65536, 262144])
    tau = oracle.length_temperature(n, tl, True)
    want = [1, 1, 1, 1, 12 / 11, 14 / 11, 16 / 11, 18 / 11]
    assert np.allclose(tau, want, rtol=0, atol=1e-15)
    assert np.all(oracle.length_temperature(n, tl, False) == 1)


def test_null_floor_values():
    # sigma = beta*tau/sqrt(d); floor = b_h + sigma*sqrt(2 ln n)
    n = np.array([1, 2048, 16384, 65536, 262144])
    tau = oracle.length_temperature(n, 2048, True)
    f = oracle.null_floor(n, 8.0, tau, 64, 0.0, True)
    want = [0.0, 3.9050, 5.6073, 6.8500, 8.1742]
    assert np.allclose(f, want, atol=5e-4)
    assert f[0] == 0.0                                         # ln 1 = 0: floor = b_h
    assert np.all(oracle.null_floor(n, 8.0, tau, 64, 0.25, False) == 0.25)


# ---------------------------------------------------------------- first row, SDPA
def _inputs(name, **kw):
    p = synth.prefill_inputs(name, **kw)
    return p, p.as_f32("q"), p.as_f32("k"), p.as_f32("v")


def test_first_causal_row_special_case():
    p, q, k, v = _inputs("c2", B=2, T=64)
    o = oracle.polar_prefill(q, k, v, p.beta, p.null_bias, p.count_vec, p.train_len, ON)
    G = p.Hq // p.Hkv
    for b in range(p.B):
        for h in range(p.Hq):
            v0 = v[b, 0, h // G].astype(np.float64)
            l0 = 8.0 * float(q[b, 0, h].astype(np.float64) @ k[b, 0, h // G].astype(np.float64))
            assert o["n_eff"][b, 0, h] == 1.0
            assert np.all(o["count"][b, 0, h] == 0.0)
            assert np.allclose(o["dir"][b, 0, h], v0 / np.linalg.norm(v0), atol=1e-15)
            assert abs(o["lse"][b, 0, h] - l0) < 1e-12
            assert abs(o["gate"][b, 0, h] - 1 / (1 + math.exp(-l0))) < 1e-12


@pytest.mark.parametrize("cfg,kw", [("c1", {}), ("c2", dict(B=2, T=300))])
def test_direction_matches_library_sdpa_at_unit_temperature(cfg, kw):
    p, q, k, v = _inputs(cfg, **kw)
    o = oracle.polar_prefill(q, k, v, p.beta, p.null_bias, p.count_vec, p.train_len, OFF)
    G = p.Hq // p.Hkv
    qt = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(G, 1)
    vt = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(G, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           scale=8.0)
    ref = ref.permute(0, 2, 1, 3).numpy()
    ref_dir = ref / np.linalg.norm(ref, axis=-1, keepdims=True)
    assert np.abs(o["dir"] - ref_dir).max() < 1e-12
    assert np.allclose(np.linalg.norm(o["dir"], axis=-1), 1.0, atol=1e-14)
    scores = 8.0 * (qt @ kt.transpose(-1, -2))
    T = p.T
    scores = scores.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), -math.inf)
    lse = torch.logsumexp(scores, -1).permute(0, 2, 1).numpy()
    assert np.abs(o["lse"] - lse).max() < 1e-11


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("c", [2, 3])
def test_count_blind_direction_under_key_duplication(c):
    g = np.random.default_rng(c)
    d, n = 64, 200
    qv = unit(g.standard_normal(d))
    K = unit(g.standard_normal((n, d)))
    K[17] = unit(qv + 0.1 * unit(g.standard_normal(d)))
    V = g.standard_normal((n, d))
    base = single_row(qv, K, V)
    dup = single_row(qv, np.repeat(K, c, axis=0), np.repeat(V, c, axis=0))
    assert np.abs(dup["dir"] - base["dir"]).max() < 1e-12
    assert abs(dup["n_eff"] - c * base["n_eff"]) < 1e-10 * c * base["n_eff"]
    assert abs(dup["lse"] - (base["lse"] + math.log(c))) < 1e-12


def test_count_bounded_and_monotone_in_neff():
    g = np.random.default_rng(11)
    d, n = 32, 256
    w = 0.02 * g.standard_normal(d)
    qv = unit(g.standard_normal(d))
    Kb = unit(g.standard_normal((n, d)))
    Kb -= (Kb @ qv)[:, None] * qv[None, :] * 0.9
    Kb = unit(Kb)
    V = g.standard_normal((n, d))
    prev = None
    for ties in range(1, 12):
        K = Kb.copy()
        K[:ties] = qv                                          # same max logit, same n
        r = single_row(qv, K, V, beta=8.0, flags=ON, w=w, train_len=16)
        bound = r["gate"] * math.tanh(math.log(r["n_eff"])) * np.linalg.norm(w)
        assert np.linalg.norm(r["count"]) <= bound * (1 + 1e-12)
        assert np.linalg.norm(r["count"]) < np.linalg.norm(w)
        if prev is not None:
            assert abs(r["gate"] - prev["gate"]) < 1e-15     # gate fixed: m, n unchanged
            assert r["n_eff"] > prev["n_eff"]
            assert np.linalg.norm(r["count"]) > np.linalg.norm(prev["count"])
        prev = r


def test_decode_equals_prefill_last_row_and_ignores_page_placement():
    p, q, k, v = _inputs("c3", B=2, T=333)
    P = 64
    rows = np.array([0, 63, 64, 200, 332])
    pre = oracle.polar_prefill(q, k, v, p.beta, p.null_bias, p.count_vec, p.train_len, ON,
                               rows=rows)
    g = np.random.default_rng(5)
    for ri, r in enumerate(rows):
        L = int(r) + 1
        n_pages = -(-L // P)
        num = p.B * n_pages + 3
        perm = g.permutation(num)
        kp = np.zeros((num, p.Hkv, P, p.d)); vp = np.zeros_like(kp)
        table = np.zeros((p.B, n_pages), np.int32)
        for b in range(p.B):
            for j in range(n_pages):
                phys = perm[b * n_pages + j]
                table[b, j] = phys
                seg = slice(j * P, min(L, (j + 1) * P))
                cnt = seg.stop - seg.start
                kp[phys, :, :cnt] = k[b, seg].transpose(1, 0, 2)
                vp[phys, :, :cnt] = v[b, seg].transpose(1, 0, 2)
        dec = oracle.polar_decode_paged(q[:, r], kp, vp, table, np.full(p.B, L), P, p.beta,
                                        p.null_bias, p.count_vec, p.train_len, ON)
        for key in dec:
            assert np.abs(dec[key] - pre[key][:, ri]).max() < 1e-12, key
        # same logical cache under a different physical placement: bit-identical
        perm2 = g.permutation(num)
        kp2 = np.zeros_like(kp); vp2 = np.zeros_like(vp)
        kp2[perm2] = kp; vp2[perm2] = vp
        dec2 = oracle.polar_decode_paged(q[:, r], kp2, vp2, perm2[table].astype(np.int32),
                                         np.full(p.B, L), P, p.beta, p.null_bias,
                                         p.count_vec, p.train_len, ON)
        for key in dec:
            assert np.array_equal(dec[key], dec2[key]), key

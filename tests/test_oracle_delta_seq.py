"""Pins of the memory stream over a sequence (oracle.delta_sequence_pool), against forms of
the gated delta rule other than the token-by-token loop it is written as:

* the state after token t in closed form, S_t = S_0 A_1..A_t + sum_i beta_i v_i k_i^T
  A_{i+1}..A_t with A_s = alpha_s (I - beta_s k_s k_s^T), and o_t = S_t q_t, in pure Python
  (math.fsum over nested lists);
* the chunkwise (WY) form: with gamma_t the running product of alpha inside a chunk, the
  write vectors u_t = beta_t (v_t - alpha_t S_{t-1} k_t) solve one unit lower triangular
  system per chunk, S_t = gamma_t S_0 + sum_{i<=t} (gamma_t / gamma_i) u_i k_i^T;
* closed forms: beta = 0 decays the state by alpha each token; orthonormal keys with
  alpha = beta = 1 from a zero state store sum_i v_i k_i^T exactly;
* one token equals the one-step pool oracle; invalid slots are skipped.
"""
import math

import numpy as np
import pytest

import oracle


def _seq(seed, B=2, T=9, H=2, dv=3, dk=4, slots=None, num_slots=4):
    r = np.random.default_rng(seed)
    pool = r.standard_normal((num_slots, H, dv, dk))
    q = r.standard_normal((B, T, H, dk))
    k = r.standard_normal((B, T, H, dk))
    v = r.standard_normal((B, T, H, dv))
    al = r.uniform(0.5, 1.0, (B, T, H))
    be = r.uniform(0.0, 1.0, (B, T, H))
    slots = np.arange(B) if slots is None else np.asarray(slots)
    return pool, slots, q, k, v, al, be


def _unit(x):
    n = math.sqrt(math.fsum(c * c for c in x) + 1e-12)
    return [c / n for c in x]


def test_sequence_equals_closed_form_state_pure_python():
    pool, slots, q, k, v, al, be = _seq(1, B=1, T=6, H=1)
    new, out = oracle.delta_sequence_pool(pool, slots, q, k, v, al, be)
    dv, dk = pool.shape[2:]
    ks = [_unit(list(k[0, t, 0])) for t in range(6)]
    qs = [_unit(list(q[0, t, 0])) for t in range(6)]

    def matmul(A, Bm):
        return [[math.fsum(A[i][x] * Bm[x][j] for x in range(len(Bm)))
                 for j in range(len(Bm[0]))] for i in range(len(A))]

    def Amat(s):
        return [[al[0, s, 0] * ((1.0 if i == j else 0.0) - be[0, s, 0] * ks[s][i] * ks[s][j])
                 for j in range(dk)] for i in range(dk)]

    S0 = [list(r) for r in pool[0, 0]]
    for t in range(6):
        St = S0
        for s in range(t + 1):
            St = matmul(St, Amat(s))
        for i in range(t + 1):
            M = [[be[0, i, 0] * v[0, i, 0][a] * ks[i][c] for c in range(dk)] for a in range(dv)]
            for s in range(i + 1, t + 1):
                M = matmul(M, Amat(s))
            St = [[St[a][c] + M[a][c] for c in range(dk)] for a in range(dv)]
        o = [math.fsum(St[a][c] * qs[t][c] for c in range(dk)) for a in range(dv)]
        np.testing.assert_allclose(out[0, t, 0], o, atol=1e-12)
        if t == 5:
            np.testing.assert_allclose(new[0, 0], St, atol=1e-12)


def _wy_chunk(S0, Q, K, V, al, be):
    """One chunk of the memory stream in the chunkwise form (float64)."""
    C = K.shape[0]
    g = np.cumprod(al)                                  # gamma_t, inclusive
    A = np.tril((be * g)[:, None] / g[None, :] * (K @ K.T), -1)
    rhs = be[:, None] * V - (be * g)[:, None] * (K @ S0.T)
    U = np.linalg.solve(np.eye(C) + A, rhs)             # rows u_t
    ratio = np.tril(g[:, None] / g[None, :])
    O = g[:, None] * (Q @ S0.T) + (ratio * (Q @ K.T)) @ U
    S = g[-1] * S0 + (U * (g[-1] / g)[:, None]).T @ K
    return O, S


@pytest.mark.parametrize("C", [1, 3, 8])
def test_sequence_equals_chunkwise_form(C):
    pool, slots, q, k, v, al, be = _seq(2, B=2, T=8, H=3, dv=5, dk=6)
    new, out = oracle.delta_sequence_pool(pool, slots, q, k, v, al, be)
    for b in range(2):
        for h in range(3):
            S = pool[b, h]
            Qn = oracle.l2_normalize(q[b, :, h])
            Kn = oracle.l2_normalize(k[b, :, h])
            for c0 in range(0, 8, C):
                sl = slice(c0, c0 + C)
                O, S = _wy_chunk(S, Qn[sl], Kn[sl], v[b, sl, h], al[b, sl, h], be[b, sl, h])
                np.testing.assert_allclose(out[b, sl, h], O, atol=1e-11)
            np.testing.assert_allclose(new[b, h], S, atol=1e-11)


def test_beta_zero_decays_the_state():
    pool, slots, q, k, v, al, be = _seq(3, B=1, T=5, H=2)
    al[:] = 0.8
    be[:] = 0.0
    new, out = oracle.delta_sequence_pool(pool, slots, q, k, v, al, be)
    for t in range(5):
        for h in range(2):
            qn = q[0, t, h] / np.linalg.norm(q[0, t, h])
            np.testing.assert_allclose(out[0, t, h], 0.8 ** (t + 1) * pool[0, h] @ qn, atol=1e-13)
    np.testing.assert_allclose(new[0], 0.8 ** 5 * pool[0], atol=1e-13)


def test_orthonormal_keys_store_every_value():
    r = np.random.default_rng(4)
    dk, dv, T = 6, 4, 5
    basis, _ = np.linalg.qr(r.standard_normal((dk, dk)))
    k = basis[:, :T].T[None, :, None, :]                  # [1,T,1,dk], orthonormal rows
    q = r.standard_normal((1, T, 1, dk))
    v = r.standard_normal((1, T, 1, dv))
    ones = np.ones((1, T, 1))
    new, out = oracle.delta_sequence_pool(np.zeros((1, 1, dv, dk)), [0], q, k, v, ones, ones)
    for t in range(T):
        qn = q[0, t, 0] / np.linalg.norm(q[0, t, 0])
        want = sum(v[0, i, 0] * (k[0, i, 0] @ qn) for i in range(t + 1))
        np.testing.assert_allclose(out[0, t, 0], want, atol=1e-12)
    np.testing.assert_allclose(new[0, 0], sum(np.outer(v[0, i, 0], k[0, i, 0]) for i in range(T)),
                               atol=1e-12)


def test_one_token_equals_the_step_and_invalid_slots_are_skipped():
    pool, _, q, k, v, al, be = _seq(5, B=3, T=1, H=2, num_slots=5)
    slots = np.array([4, -1, 1])
    new, out = oracle.delta_sequence_pool(pool, slots, q, k, v, al, be)
    p1, o1 = oracle.delta_step_pool(pool, slots, q[:, 0], k[:, 0], v[:, 0], al[:, 0], be[:, 0])
    np.testing.assert_allclose(new, p1, atol=1e-15)
    np.testing.assert_allclose(out[:, 0], o1, atol=1e-15)
    np.testing.assert_array_equal(out[1], 0.0)
    np.testing.assert_array_equal(new[[0, 2, 3]], pool[[0, 2, 3]])

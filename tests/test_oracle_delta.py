"""Pins of the gated-delta step oracle (oracle.delta_oracle) against properties of the
rule itself, not against its own formula.

* beta = 0 is a pure decay: S' = alpha S, o = alpha S q;
* alpha = beta = 1 writes v at key k exactly: S' k = v (the delta rule's defining
  property for a unit key);
* a query orthogonal to k reads only the decayed old memory;
* |S'|_F <= alpha |S|_F + beta |v| (I - beta k k^T has spectral norm <= 1 for unit k and
  beta in [0, 1]: the stability the L2 normalisation buys);
* a whole sequence of steps equals the unrolled sum over t of
  beta_t v_t k_t^T prod_{s>t} alpha_s (I - beta_s k_s k_s^T), computed with pure-Python
  loops over tiny matrices;
* normalisation: scaling q or k by a positive constant changes nothing.
"""
import math

import numpy as np
import pytest

import oracle


def _rand(seed, dv=6, dk=5):
    r = np.random.default_rng(seed)
    S = r.standard_normal((dv, dk))
    q, k = r.standard_normal(dk), r.standard_normal(dk)
    v = r.standard_normal(dv)
    return r, S, q, k, v


def test_beta_zero_is_pure_decay():
    _, S, q, k, v = _rand(1)
    S2, o = oracle.delta_step(S, q, k, v, 0.7, 0.0)
    np.testing.assert_allclose(S2, 0.7 * S, atol=1e-15)
    np.testing.assert_allclose(o, 0.7 * S @ (q / np.linalg.norm(q)), atol=1e-14)


def test_full_write_stores_v_at_k():
    _, S, q, k, v = _rand(2)
    S2, _ = oracle.delta_step(S, q, k, v, 1.0, 1.0)
    np.testing.assert_allclose(S2 @ (k / np.linalg.norm(k)), v, atol=1e-13)


def test_orthogonal_query_reads_decayed_memory():
    _, S, q, k, v = _rand(3)
    kn = k / np.linalg.norm(k)
    q = q - (q @ kn) * kn                          # q orthogonal to k
    _, o = oracle.delta_step(S, q, k, v, 0.6, 0.8)
    np.testing.assert_allclose(o, 0.6 * S @ (q / np.linalg.norm(q)), atol=1e-13)


@pytest.mark.parametrize("seed", range(5))
def test_norm_bound(seed):
    r, S, q, k, v = _rand(10 + seed)
    alpha, beta = r.uniform(0, 1), r.uniform(0, 1)
    S2, _ = oracle.delta_step(S, q, k, v, alpha, beta)
    assert np.linalg.norm(S2) <= alpha * np.linalg.norm(S) + beta * np.linalg.norm(v) + 1e-12


def test_sequence_equals_unrolled_sum_pure_python():
    r = np.random.default_rng(7)
    dv, dk, T = 3, 4, 6
    ks = [list(oracle.l2_normalize(r.standard_normal(dk))) for _ in range(T)]
    vs = [list(r.standard_normal(dv)) for _ in range(T)]
    al = list(r.uniform(0.5, 1.0, T))
    be = list(r.uniform(0.0, 1.0, T))
    S = np.zeros((dv, dk))
    for t in range(T):
        S, _ = oracle.delta_step(S, np.ones(dk), ks[t], vs[t], al[t], be[t], normalize=False)

    def matmul(A, Bm):
        return [[math.fsum(A[i][x] * Bm[x][j] for x in range(len(Bm)))
                 for j in range(len(Bm[0]))] for i in range(len(A))]
    want = [[0.0] * dk for _ in range(dv)]
    for t in range(T):
        M = [[be[t] * vs[t][i] * ks[t][j] for j in range(dk)] for i in range(dv)]
        for s in range(t + 1, T):
            P = [[al[s] * ((1.0 if i == j else 0.0) - be[s] * ks[s][i] * ks[s][j])
                  for j in range(dk)] for i in range(dk)]
            M = matmul(M, P)
        want = [[want[i][j] + M[i][j] for j in range(dk)] for i in range(dv)]
    np.testing.assert_allclose(S, np.array(want), atol=1e-13)


def test_scaling_q_and_k_changes_nothing():
    _, S, q, k, v = _rand(4)
    a = oracle.delta_step(S, q, k, v, 0.9, 0.4)
    b = oracle.delta_step(S, 3.5 * q, 0.25 * k, v, 0.9, 0.4)
    np.testing.assert_allclose(a[0], b[0], atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], atol=1e-14)


def test_pool_step_skips_invalid_slots_and_leaves_other_slots():
    r = np.random.default_rng(8)
    pool = r.standard_normal((5, 2, 3, 4))
    q, k = r.standard_normal((3, 2, 4)), r.standard_normal((3, 2, 4))
    v = r.standard_normal((3, 2, 3))
    al, be = r.uniform(0, 1, (3, 2)), r.uniform(0, 1, (3, 2))
    new, out = oracle.delta_step_pool(pool, [4, -1, 1], q, k, v, al, be)
    np.testing.assert_array_equal(new[[0, 2, 3]], pool[[0, 2, 3]])
    np.testing.assert_array_equal(out[1], 0.0)
    s4, o0 = oracle.delta_step(pool[4], q[0], k[0], v[0], al[0], be[0])
    np.testing.assert_allclose(new[4], s4)
    np.testing.assert_allclose(out[0], o0)

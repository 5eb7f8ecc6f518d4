"""Pure-Python brute force (math.fsum, no NumPy in the arithmetic) on tiny inputs.

Written separately from the oracle from the same definitions ("ATMA" technical summary,
section 2.1): per query row i and head h, keys 0..i of KV head (h*Hkv)//Hq, logits
beta*tau*<q,k>, softmax probabilities, inverse Simpson index, normalised value sum,
floor-gated tanh(log n_eff) count.  Catches index, mask, GQA-map, sign and missing-term
slips in the vectorised oracle.
"""
import math
import random

import numpy as np
import pytest

import oracle


def brute_prefill(q, k, v, Hq, Hkv, beta, b_h, w, train_len, flags):
    T, d = len(q), len(q[0][0])
    res = {}
    for i in range(T):
        for h in range(Hq):
            g = (h * Hkv) // Hq
            n = i + 1
            tau = 1.0
            if flags & 1:
                tau = max(1.0, math.log(n) / math.log(train_len))
            logits = [beta[h] * tau * math.fsum(q[i][h][t] * k[j][g][t] for t in range(d))
                      for j in range(n)]
            m = max(logits)
            lse = m + math.log(math.fsum(math.exp(x - m) for x in logits))
            p = [math.exp(x - lse) for x in logits]
            neff = 1.0 / math.fsum(x * x for x in p)
            u = [math.fsum(p[j] * v[j][g][t] for j in range(n)) for t in range(d)]
            nu = math.sqrt(math.fsum(x * x for x in u))
            direction = [x / nu for x in u]
            floor = b_h[h]
            if flags & 2:
                floor += beta[h] * tau / math.sqrt(d) * math.sqrt(2.0 * math.log(n))
            gate = 1.0 / (1.0 + math.exp(floor - m))
            count = [gate * math.tanh(math.log(neff)) * w[h][t] for t in range(d)]
            res[(i, h)] = dict(dir=direction, count=count, n_eff=neff, gate=gate, lse=lse)
    return res


@pytest.mark.parametrize("seed,Hq,Hkv,flags", [(0, 4, 2, 3), (1, 4, 4, 3), (2, 6, 2, 0),
                                               (3, 4, 1, 1), (4, 2, 2, 2)])
def test_oracle_matches_brute_force(seed, Hq, Hkv, flags):
    rnd = random.Random(seed)
    T, d, train_len = 8, 4, 3
    q = [[[rnd.gauss(0, 1) for _ in range(d)] for _ in range(Hq)] for _ in range(T)]
    k = [[[rnd.gauss(0, 1) for _ in range(d)] for _ in range(Hkv)] for _ in range(T)]
    v = [[[rnd.gauss(0, 1) for _ in range(d)] for _ in range(Hkv)] for _ in range(T)]
    beta = [rnd.uniform(0.5, 3.0) for _ in range(Hq)]
    b_h = [rnd.uniform(-1.0, 1.0) for _ in range(Hq)]
    w = [[rnd.gauss(0, 0.02) for _ in range(d)] for _ in range(Hq)]
    want = brute_prefill(q, k, v, Hq, Hkv, beta, b_h, w, train_len, flags)
    got = oracle.polar_prefill(np.array([q]), np.array([k]), np.array([v]), beta, b_h,
                               np.array(w), train_len, flags)
    for (i, h), ref in want.items():
        for key in ("n_eff", "gate", "lse"):
            assert abs(got[key][0, i, h] - ref[key]) <= 1e-12 * max(1.0, abs(ref[key])), key
        for key in ("dir", "count"):
            assert np.abs(got[key][0, i, h] - np.array(ref[key])).max() <= 1e-13, key

"""Input generator checks: bf16 rounding, determinism, unit norms, needle structure."""
import numpy as np
import torch

import synth


def test_round_bf16_matches_torch_rne():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -2.5, 3.0e-39, 65504.0, 1.00390625, 1.01171875,
                                  -1.00390625, 0.0, -0.0], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.round_bf16(x), ref)
    back = synth.bf16_bits_to_f32(ref)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16)
                          .to(torch.float32).numpy())


def test_deterministic_and_unit_norm():
    a = synth.prefill_inputs("c3", T=700)
    b = synth.prefill_inputs("c3", T=700)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.k, b.k) and np.array_equal(a.v, b.v)
    for name in ("q", "k"):
        n = np.linalg.norm(a.as_f32(name).astype(np.float64), axis=-1)
        assert np.abs(n - 1).max() < 1e-2          # bf16 rounding of unit vectors
    c = synth.prefill_inputs("c1")
    assert c.q.dtype == np.float32
    assert np.abs(np.linalg.norm(c.q, axis=-1) - 1).max() < 1e-6


def test_needles_are_near_copies():
    p = synth.prefill_inputs("c4", T=4096)
    assert len(p.needles) == 8 and sorted({h for _, h, _, _ in p.needles}) == list(range(0, 16, 2))
    q, k = p.as_f32("q").astype(np.float64), p.as_f32("k").astype(np.float64)
    for b, h, j, i in p.needles:
        assert i == p.T - 1
        cos = q[b, i, h] @ k[b, j, h // 4]
        assert 0.98 < cos <= 1.01
    p2 = synth.prefill_inputs("c2", B=2, T=400)
    assert len(p2.needles) == 2 * 4 * 20
    for b, h, j, i in p2.needles:
        assert j <= i


def test_decode_layout_and_needles():
    d = synth.decode_inputs("c5", B=3, seq_lens=[1000, 64, 129], extra_pages=4)
    P = d.page_size
    used = np.concatenate([d.page_table[b, :-(-d.seq_lens[b] // P)] for b in range(3)])
    assert len(np.unique(used)) == len(used) and used.max() < d.num_pages
    assert d.k_pool.shape == (d.num_pages, 4, 64, 64) and d.k_pool.dtype == np.uint16
    q = d.as_f32("q").astype(np.float64)
    kp = d.as_f32("k_pool").astype(np.float64)
    for b, h, j in d.needles:
        key = kp[d.page_table[b, j // P], h // 4, j % P]
        assert q[b, h] @ key > 0.98

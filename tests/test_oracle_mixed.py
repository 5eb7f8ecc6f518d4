"""Pins of the three-stream sum (oracle.three_streams), the layer output that section 2.1
of the technical summary writes as out = content + count + memory:

* with no count vector and no memory the sum is the content stream alone, a unit vector
  per row;
* the memory stream enters additively: the sum moves by exactly the memory added;
* the count stream is gate tanh(ln n_eff) w_h, rebuilt here from the oracle's own scalar
  outputs rather than taken from its count output.
"""
import numpy as np

import oracle
import synth


def _fwd(count_vec=True, T=40):
    p = synth.prefill_inputs("c2", B=2, T=T, Hq=4, Hkv=2)
    f = oracle.polar_prefill(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.beta, p.null_bias,
                             p.count_vec if count_vec else None, p.train_len, p.flags)
    return p, f


def test_content_alone_is_unit_rows():
    p, f = _fwd(count_vec=False)
    out = oracle.three_streams(f)
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1), 1.0, rtol=1e-12)
    np.testing.assert_array_equal(out, f["dir"])


def test_memory_adds_exactly():
    p, f = _fwd()
    m = np.random.default_rng(5).standard_normal(f["dir"].shape)
    diff = oracle.three_streams(f, m) - oracle.three_streams(f)
    np.testing.assert_allclose(diff, m, atol=1e-14)


def test_count_stream_from_the_scalars():
    p, f = _fwd()
    n = f["n_eff"]
    th = np.tanh(np.log(n))
    want = f["dir"] + (f["gate"] * th)[..., None] * p.count_vec[None, None, :, :]
    np.testing.assert_allclose(oracle.three_streams(f), want, rtol=1e-12, atol=1e-15)

"""GPU parity of the variant modes (sliding window, RoPE on load, plain softmax output)
against the float64 oracle, through the C ABI.  Tolerances as in tests/parity.py; the
plain softmax output uses the direction metric scaled by |attn|."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from parity import TOL, assert_close, gpu_prefill, host, oracle_prefill, select, to_dev
from long_context_lm_amd import attn_fwd_variant

pytestmark = pytest.mark.gpu


def run(p, **var):
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    out = attn_fwd_variant(q, k, v, beta=p.beta, null_bias=p.null_bias, count_vec=p.count_vec,
                           train_len=p.train_len, flags=p.flags, **var)
    torch.cuda.synchronize()
    return out


def check(p, got, want, label, heads=None):
    assert_close(got, want, p.count_vec, p.dtype, heads=heads, label=label)
    a, w = host(got["attn"]), want["attn"]
    err = float(np.max(np.linalg.norm(a - w, axis=-1) / np.linalg.norm(w, axis=-1)))
    print(f"[variant] {label} attn {err:.2e}", flush=True)
    assert err <= TOL[p.dtype], (label, err)


@pytest.mark.parametrize("cfg,B,T,Hq,Hkv,window,theta", [
    ("c2", 2, 300, 8, 2, 100, 0.0),          # window only, ragged
    ("c2", 1, 257, 4, 4, 1, 0.0),            # window 1: closed forms
    ("c2", 1, 200, 8, 2, 0, 10000.0),        # RoPE only
    ("c2", 1, 333, 16, 4, 64, 500.0),        # window + RoPE, GQA 4
    ("c2", 1, 130, 4, 2, 200, 0.0),          # window >= T
    ("c1", 1, 256, 4, 4, 37, 10000.0),       # float32 inputs
    ("c1", 1, 100, 4, 2, 0, 0.0),            # float32, softmax output only
])
def test_variant_parity(gpu_lib, cfg, B, T, Hq, Hkv, window, theta):
    print(f"[case] variant {cfg} B={B} T={T} {Hq}/{Hkv} W={window} theta={theta}", flush=True)
    p = synth.prefill_inputs(cfg, B=B, T=T, Hq=Hq, Hkv=Hkv, train_len=64)
    got = run(p, window=window, rope_theta=theta)
    want = oracle_prefill(p, window=window, rope_theta=theta)
    check(p, got, want, f"{cfg} W={window} theta={theta}")


@pytest.mark.parametrize("beta,T,window", [(16.0, 2048, 0), (24.0, 700, 0), (16.0, 3000, 1000)])
def test_rope_at_sharper_beta(gpu_lib, beta, T, window):
    """RoPE with sharper logits than the default beta = 8 (near one-hot rows dominate).  The
    kernel rounds the rotated q and k to bfloat16, as a bfloat16 model holds them, and so
    does the oracle; what is left is the rounding of P and the hardware sine and cosine,
    so the errors do not grow with beta."""
    print(f"[case] rope beta={beta} T={T} W={window}", flush=True)
    p = synth.prefill_inputs("c2", B=1, T=T, Hq=8, Hkv=2, train_len=2048)
    p = dataclasses.replace(p, beta=np.full(p.Hq, beta, np.float32))
    got = run(p, window=window, rope_theta=10000.0)
    want = oracle_prefill(p, window=window, rope_theta=10000.0)
    check(p, got, want, f"rope beta={beta} T={T} W={window}")


@pytest.mark.parametrize("cfg,T,window,attn", [("c2", 333, 0, True), ("c2", 200, 64, False),
                                              ("c1", 150, 37, True)])
def test_keys_rotated_once_equal_keys_rotated_in_staging(gpu_lib, cfg, T, window, attn):
    """The workspace path (keys rotated by their own kernel before the prefill) and the
    in-staging rotation use the same arithmetic, so every output is bit-identical."""
    print(f"[case] rotate once vs in staging {cfg} T={T} W={window}", flush=True)
    p = synth.prefill_inputs(cfg, B=2, T=T, Hq=8, Hkv=2, train_len=64)
    a = run(p, window=window, rope_theta=10000.0, want_attn=attn, rotate_keys_once=True)
    b = run(p, window=window, rope_theta=10000.0, want_attn=attn, rotate_keys_once=False)
    for n in ("dir", "count", "n_eff", "gate", "lse", "attn"):
        if a.get(n) is not None:
            assert torch.equal(a[n], b[n]), n


def test_variant_without_modes_equals_plain_forward(gpu_lib):
    p = synth.prefill_inputs("c2", B=1, T=200, Hq=8, Hkv=2, train_len=64)
    a = run(p, want_attn=False)
    b = gpu_prefill(p)
    for n in ("dir", "count", "n_eff", "gate", "lse"):
        assert torch.equal(a[n], b[n]), n


def test_variant_full_size_sampled(gpu_lib):
    """T = 64K extrapolation workload with RoPE and a 4096-key window, sampled rows."""
    print("[case] variant C4 W=4096 theta=10000 sampled", flush=True)
    p = synth.prefill_inputs("c4")
    got = run(p, window=4096, rope_theta=10000.0)
    rows = np.array([0, 1, 63, 64, 4095, 4096, 4097, 30000, 65534, 65535])
    heads = np.array([0, 5, 10, 15])
    want = oracle_prefill(p, rows=rows, heads=heads, window=4096, rope_theta=10000.0)
    check(p, select(got, rows=rows, heads=heads), want, "C4 W=4096 rope", heads=heads)


def test_variant_full_size_rope_softmax_sampled(gpu_lib):
    """T = 64K with RoPE on load and the plain softmax output, no window (the variant
    workload of the benchmark), sampled rows."""
    print("[case] variant C4 W=0 theta=10000 sampled", flush=True)
    p = synth.prefill_inputs("c4")
    got = run(p, window=0, rope_theta=10000.0)
    rows = np.array([0, 1, 2, 63, 64, 2047, 2048, 40000, 65535])
    heads = np.array([0, 3, 8, 15])
    want = oracle_prefill(p, rows=rows, heads=heads, window=0, rope_theta=10000.0)
    check(p, select(got, rows=rows, heads=heads), want, "C4 W=0 rope", heads=heads)


def test_lean_variant_ragged_rows_and_equal_to_pipelined(gpu_lib):
    """Window 1000 with RoPE at B=4, T=8000: the lean variant instance (keys rotated once
    into the workspace), sampled rows against the oracle, and bit-identical to the
    pipelined instance of a one-sequence launch."""
    print("[case] variant lean B=4 T=8000 W=1000 theta=10000", flush=True)
    p = synth.prefill_inputs("c2", B=4, T=8000)
    var = dict(window=1000, rope_theta=10000.0)
    got = run(p, **var)
    rows = np.array([0, 1, 127, 128, 999, 1000, 1001, 5000, 7936, 7999])
    batches = np.array([0, 3])
    want = oracle_prefill(p, rows=rows, batches=batches, **var)
    check(p, select(got, batches=batches, rows=rows), want, "lean W=1000 rope")
    one = run(dataclasses.replace(p, B=1, q=p.q[:1], k=p.k[:1], v=p.v[:1],
                                  needles=[n for n in p.needles if n[0] == 0]), **var)
    for key in ("dir", "count", "n_eff", "gate", "lse", "attn"):
        assert torch.equal(got[key][:1], one[key]), key

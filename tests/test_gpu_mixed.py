"""GPU parity of the three streams summed (polar_attn_fwd_mixed) through the C ABI.

The sum dir + count + memory is judged per row against the oracle's sum: |x^ - x|_2 over
(1 + |w_h|_2), the scales of the content error (dir is a unit vector) and the count error
(tests/parity.py's metrics), with the same bounds (1e-4 fp32, 2e-2 bf16); the memory is an
exact input and adds no error of its own.  Against the separate outputs of polar_attn_fwd
on the same GPU, the sum agrees to fp32 rounding (the kernel may fuse the content and
count terms into one multiply-add)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from long_context_lm_amd import _lib, attn_fwd, attn_fwd_mixed
from parity import TOL, gpu_prefill, oracle_prefill, to_dev

pytestmark = pytest.mark.gpu


def _memory(p, seed=9):
    m = np.random.default_rng(seed).standard_normal((p.B, p.T, p.Hq, p.d)).astype(np.float32)
    return m, torch.from_numpy(m).cuda()


def _mixed(p, mem=None):
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    out = attn_fwd_mixed(q, k, v, memory=mem, beta=p.beta, null_bias=p.null_bias,
                         count_vec=p.count_vec, train_len=p.train_len, flags=p.flags)
    torch.cuda.synchronize()
    return out


def _err(got, want, count_vec, heads=None):
    w = np.linalg.norm(np.asarray(count_vec, np.float64), axis=-1)      # [Hq]
    if heads is not None:
        w = w[heads]
    d = np.linalg.norm(np.asarray(got, np.float64) - want, axis=-1)    # [B,R,H]
    return float(np.max(d / (1.0 + w)))


@pytest.mark.parametrize("name,B,T,Hq,Hkv,dtype", [
    ("c2", 2, 300, 16, 4, "bf16"),      # pipelined instance, ragged tail
    ("c1", 1, 256, 4, 4, "f32"),        # fp32 instance
    ("c2", 3, 77, 8, 2, "bf16"),
])
def test_mixed_matches_oracle(gpu_lib, name, B, T, Hq, Hkv, dtype):
    print(f"[case] mixed {name} B={B} T={T} Hq={Hq} Hkv={Hkv} {dtype}", flush=True)
    p = synth.prefill_inputs(name, B=B, T=T, Hq=Hq, Hkv=Hkv, dtype=dtype)
    m, mem = _memory(p)
    got = _mixed(p, mem)
    want = oracle_prefill(p)
    e = _err(got["mixed"].cpu().numpy(), oracle.three_streams(want, m), p.count_vec)
    e_n = float(np.max(np.abs(got["n_eff"].cpu().numpy() - want["n_eff"]) / want["n_eff"]))
    print(f"[mixed] {dtype} sum {e:.2e} n_eff {e_n:.2e}", flush=True)
    assert e <= TOL[dtype] and e_n <= TOL[dtype]


def test_mixed_lean_instance_sampled_rows(gpu_lib):
    """B = 8, T = 2048 (1024 workgroups: the lean instance), sampled rows of two sequences
    against the oracle, and every row against the separate outputs of the same launch
    shape."""
    print("[case] mixed lean B=8 T=2048", flush=True)
    p = synth.prefill_inputs("c2")
    m, mem = _memory(p)
    got = _mixed(p, mem)
    rows = np.array([0, 1, 63, 64, 127, 1000, 2047])
    batches = np.array([0, 7])
    want = oracle_prefill(p, rows=rows, batches=batches)
    g = got["mixed"].cpu().numpy()[batches][:, rows]
    e = _err(g, oracle.three_streams(want, m[batches][:, rows]), p.count_vec)
    sep = gpu_prefill(p)
    ref = (sep["dir"] + sep["count"]) + mem
    d = float((got["mixed"] - ref).abs().max())
    print(f"[mixed] lean sum {e:.2e}, against dir + count + memory {d:.2e}", flush=True)
    assert e <= TOL["bf16"] and d <= 1e-5
    for key in ("n_eff", "gate", "lse"):
        assert torch.equal(got[key], sep[key]), key


def test_mixed_without_memory_or_count(gpu_lib):
    """memory = NULL gives dir + count; no count vector gives dir + memory."""
    p = synth.prefill_inputs("c2", B=2, T=200)
    sep = gpu_prefill(p)
    got = _mixed(p)
    assert float((got["mixed"] - (sep["dir"] + sep["count"])).abs().max()) <= 1e-6
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    m, mem = _memory(p, seed=11)
    nc = attn_fwd_mixed(q, k, v, memory=mem, beta=p.beta, null_bias=p.null_bias,
                        train_len=p.train_len, flags=p.flags)
    d0 = attn_fwd(q, k, v, beta=p.beta, null_bias=p.null_bias, train_len=p.train_len,
                  flags=p.flags)
    torch.cuda.synchronize()
    assert float((nc["mixed"] - (d0["dir"] + mem)).abs().max()) <= 1e-6


def test_mixed_in_place_over_memory(gpu_lib):
    """The C ABI lets the output overwrite the memory input (each element is read before
    it is written): the result equals the out-of-place call."""
    p = synth.prefill_inputs("c2", B=2, T=150)
    m, mem = _memory(p, seed=12)
    want = _mixed(p, mem)["mixed"]
    buf = mem.clone()
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    n_eff = torch.empty(p.B, p.T, p.Hq, device="cuda")
    beta_t = torch.from_numpy(p.beta).cuda()
    bias_t = torch.from_numpy(p.null_bias).cuda()
    cv_t = torch.from_numpy(np.ascontiguousarray(p.count_vec)).cuda()
    prm = _lib.polar_params(p.Hq, p.Hkv, p.d, p.train_len, p.flags, beta_t.data_ptr(),
                            bias_t.data_ptr(), cv_t.data_ptr())
    outs = _lib.polar_outputs(None, None, n_eff.data_ptr(), None, None)
    s = torch.cuda.current_stream().cuda_stream
    _lib.check(_lib.polar_attn_fwd_mixed(prm, 1, p.B, p.T, q.data_ptr(), k.data_ptr(),
                                         v.data_ptr(), buf.data_ptr(), buf.data_ptr(), outs, s))
    torch.cuda.synchronize()
    assert torch.equal(buf, want)

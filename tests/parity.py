"""Shared helpers of the GPU parity tests: move seeded inputs to the GPU, run libpolar,
run the oracle on the same values, and measure the errors the tolerances are stated in.

Error metrics, per output, maximum over rows (b, i, h):
  n_eff  |x^ - x| / x                       (x >= 1)
  dir    |x^ - x|_2 / |x|_2                 (|x| = 1)
  count  |x^ - x|_2 / |w_h|_2               (count -> 0 as n_eff -> 1, so the bound of
                                             the tanh map is the natural scale)
  count_rel |x^ - x|_2 / |x|_2              over rows with tanh(ln n_eff) >= 1/2 (n_eff >=
                                             sqrt 3): the relative error of the count
                                             output itself.  Below that floor the tanh map
                                             multiplies the relative n_eff error by
                                             (1 - th^2) / th > 3/2, and count -> 0, so
                                             those rows are judged by the |w_h| metric
  gate   |x^ - x|                           (in [0, 1])
  lse    |x^ - x| / max(1, |x|)
Thresholds: 1e-4 for float32 inputs, 2e-2 for bfloat16 inputs with fp32 accumulation.
"""
import numpy as np
import torch

import oracle
import synth
from long_context_lm_amd import attn_decode_paged, attn_fwd

TOL = {"f32": 1e-4, "bf16": 2e-2}
COUNT_REL_FLOOR = 0.5       # tanh(ln n_eff) at or above which count is judged relatively


def to_dev(a: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_prefill(p: synth.PrefillInputs, **kw) -> dict:
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    out = attn_fwd(q, k, v, beta=p.beta, null_bias=p.null_bias, count_vec=p.count_vec,
                   train_len=p.train_len, flags=p.flags, **kw)
    torch.cuda.synchronize()
    return out


def oracle_prefill(p: synth.PrefillInputs, rows=None, heads=None, batches=None, window=0,
                   rope_theta=0.0) -> dict:
    return oracle.polar_prefill(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.beta,
                                p.null_bias, p.count_vec, p.train_len, p.flags, rows=rows,
                                heads=heads, batches=batches, window=window,
                                rope_theta=rope_theta, rope_bf16=p.dtype == "bf16")


def gpu_decode(d: synth.DecodeInputs, **kw) -> dict:
    q = to_dev(d.q, d.dtype)
    kc, vc = to_dev(d.k_pool, d.dtype), to_dev(d.v_pool, d.dtype)
    table = torch.from_numpy(d.page_table).cuda()
    lens = torch.from_numpy(d.seq_lens).cuda()
    out = attn_decode_paged(q, kc, vc, table, lens, d.max_seq_len, beta=d.beta,
                            null_bias=d.null_bias, count_vec=d.count_vec,
                            train_len=d.train_len, flags=d.flags, **kw)
    torch.cuda.synchronize()
    return out


def oracle_decode(d: synth.DecodeInputs, batches=None) -> dict:
    conv = synth.bf16_bits_to_f32 if d.dtype == "bf16" else (lambda a: a)
    return oracle.polar_decode_paged(conv(d.q), d.k_pool, d.v_pool, d.page_table, d.seq_lens,
                                     d.page_size, d.beta, d.null_bias, d.count_vec,
                                     d.train_len, d.flags,
                                     to_f64=lambda a: conv(a).astype(np.float64),
                                     batches=batches)


def host(t):
    return None if t is None else t.double().cpu().numpy()


def errors(got: dict, want: dict, count_vec: np.ndarray, heads=None) -> dict:
    """Errors of GPU outputs ``got`` (already indexed like ``want``) against the oracle."""
    w = np.asarray(count_vec, np.float64)
    w = w if heads is None else w[heads]
    wn = np.linalg.norm(w, axis=-1)                       # [H]
    e = {}
    g = {k: host(v) if isinstance(v, torch.Tensor) else v for k, v in got.items()}
    e["n_eff"] = float(np.max(np.abs(g["n_eff"] - want["n_eff"]) / want["n_eff"]))
    dn = np.linalg.norm(want["dir"], axis=-1)
    e["dir"] = float(np.max(np.linalg.norm(g["dir"] - want["dir"], axis=-1) /
                            np.where(dn > 0, dn, 1.0)))
    if g.get("count") is not None:
        dc = np.linalg.norm(g["count"] - want["count"], axis=-1)
        e["count"] = float(np.max(dc / wn))
        cn = np.linalg.norm(want["count"], axis=-1)
        rel_rows = (np.tanh(np.log(want["n_eff"])) >= COUNT_REL_FLOOR) & (cn > 0)
        e["count_rel"] = float(np.max(dc[rel_rows] / cn[rel_rows])) if rel_rows.any() else 0.0
    if g.get("gate") is not None:
        e["gate"] = float(np.max(np.abs(g["gate"] - want["gate"])))
    if g.get("lse") is not None:
        e["lse"] = float(np.max(np.abs(g["lse"] - want["lse"]) /
                                np.maximum(1.0, np.abs(want["lse"]))))
    return e


def assert_close(got: dict, want: dict, count_vec, dtype: str, heads=None, label=""):
    e = errors(got, want, count_vec, heads)
    tol = TOL[dtype]
    bad = {k: v for k, v in e.items() if not (v <= tol)}
    print(f"[parity] {label} dtype={dtype} errors={ {k: f'{v:.2e}' for k, v in e.items()} }",
          flush=True)
    assert not bad, f"{label}: errors above {tol}: {bad}"
    return e


def select(out: dict, batches=None, rows=None, heads=None) -> dict:
    """Index GPU prefill outputs [B,T,H,...] like the oracle's sampled outputs."""
    res = {}
    for k, v in out.items():
        if v is None:
            res[k] = None
            continue
        t = v
        if batches is not None:
            t = t[torch.as_tensor(batches, device=t.device)]
        if rows is not None:
            t = t[:, torch.as_tensor(rows, device=t.device)]
        if heads is not None:
            t = t[:, :, torch.as_tensor(heads, device=t.device)]
        res[k] = t
    return res


# ------------------------------------------------------------------ backward pass
# Gradient error metric, per tensor: max |g^ - g| / max |g| (the largest gradient entry
# sets the scale, so near-zero entries are not judged by their own size), and the
# relative Frobenius error |g^ - g|_F / |g|_F.  Bound for bfloat16 inputs: 2e-2 on the
# first, 1e-2 on the second (the P, dS and du operands of the MFMA products are rounded to
# bfloat16, a relative 2^-9 per element, summed over up to T terms in fp32).
GRAD_TOL = {"max": 2e-2, "fro": 1e-2}
GRAD_KEYS = ("dq", "dk", "dv", "d_beta", "d_null_bias", "d_count_vec")


def gpu_forward_train(p: synth.PrefillInputs):
    from long_context_lm_amd import attn_fwd_train
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    out = attn_fwd_train(q, k, v, beta=p.beta, null_bias=p.null_bias, count_vec=p.count_vec,
                         train_len=p.train_len, flags=p.flags)
    torch.cuda.synchronize()
    return (q, k, v), out


def gpu_backward(p: synth.PrefillInputs, cot: dict, param_grads: bool = True):
    from long_context_lm_amd import attn_bwd
    (q, k, v), fwd = gpu_forward_train(p)
    g = attn_bwd(q, k, v, fwd, cot, beta=p.beta, null_bias=p.null_bias, count_vec=p.count_vec,
                 train_len=p.train_len, flags=p.flags, param_grads=param_grads)
    torch.cuda.synchronize()
    return g


def oracle_backward(p: synth.PrefillInputs, cot: dict, batches=None) -> dict:
    sl = slice(None) if batches is None else list(batches)
    c = {n: (None if x is None else np.asarray(x)[sl]) for n, x in cot.items()}
    return oracle.polar_prefill_grad(p.as_f32("q")[sl], p.as_f32("k")[sl], p.as_f32("v")[sl],
                                     c, p.beta, p.null_bias, p.count_vec, p.train_len, p.flags)


def grad_errors(got: dict, want: dict, keys=GRAD_KEYS) -> dict:
    e = {}
    for n in keys:
        g = host(got[n]) if isinstance(got[n], torch.Tensor) else np.asarray(got[n])
        w = np.asarray(want[n], np.float64)
        scale = float(np.max(np.abs(w)))
        if scale == 0.0:
            e[n] = (float(np.max(np.abs(g))), 0.0)
            continue
        e[n] = (float(np.max(np.abs(g - w))) / scale,
                float(np.linalg.norm(g - w) / max(np.linalg.norm(w), 1e-300)))
    return e


def assert_grads_close(got: dict, want: dict, keys=GRAD_KEYS, label=""):
    e = grad_errors(got, want, keys)
    print(f"[grad] {label} " + " ".join(f"{n}={m:.1e}/{f:.1e}" for n, (m, f) in e.items()),
          flush=True)
    bad = {n: v for n, v in e.items() if not (v[0] <= GRAD_TOL["max"] and v[1] <= GRAD_TOL["fro"])}
    assert not bad, f"{label}: gradient errors above {GRAD_TOL}: {bad}"
    return e

"""Benchmark of the Polar Attention hot path on one MI355X.

One step = one causal prefill of the T=64K extrapolation workload (B=1, T=65536, 16 query /
4 KV heads, d=64, bf16, length temperature and extreme-value floor on, 8 planted needles)
followed by one GQA paged decode of the 256K workload (16 sequences x 262144 keys, 64-token
pages behind a shuffled page table, one needle per (sequence, head)).  Inputs are the seeded
synthetic workloads of ``synth`` and are resident in HBM before timing starts.

Prints one JSON line.  ``value`` is prefill TFLOP/s over the timed steps, with the
algorithmic flop count 4*d*Hq*T(T+1)/2 (QK^T and PV over visible pairs only); the decode
figure (GB/s of K+V read once, plus table, queries and outputs) sits in ``decode``.  After
the timed steps, the backward pass is timed on its own at the 2K training shape and
reported in ``backward`` (TFLOP/s over the five products of the gradient, 2.5x the
forward count).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --copy-probe BYTES   (plain device copy, for counter calibration)
       python bench.py --memory-step-probe fused|ref --steps K
                                            (one form of the memory step, for counters)
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Polar attn fwd TFLOP/s (bf16, T=64K) + paged decode GB/s at 256K KV"
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E


# Sources each timed kernel is built from; a counter record stays valid while these are unchanged.
_PREFILL_SRC = ["polar_prefill.hip", "polar_mfma.h", "polar_kernels.h"]
_DECODE_SRC = ["polar_decode.hip", "polar_mfma.h", "polar_kernels.h"]
KERNEL_SOURCES = {
    "prefill": _PREFILL_SRC,
    "decode": _DECODE_SRC,
    "decode_b1": _DECODE_SRC,
    "backward": ["polar_backward.hip", "polar_mfma.h", "polar_kernels.h"],
    "variant": _PREFILL_SRC,            # key rotation + variant prefill, full causal range
    "variant_window": _PREFILL_SRC,     # key rotation + variant prefill, 4096-key window
    "paged": _PREFILL_SRC,
    "append": ["polar_paged.hip", "polar_kernels.h"],
    "memory_step": ["polar_delta.hip", "polar_kernels.h"],
}


def src_hash(kind: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "long_context_lm_amd", "csrc", name), "rb") as fh:
            h.update(name.encode())
            h.update(fh.read())
    return h.hexdigest()


def prefill_flops(B, T, Hq, d):
    return 4.0 * d * B * Hq * T * (T + 1) / 2.0


def backward_flops(B, T, Hq, d):
    """Five products over visible pairs (S = QK^T, dP = du V^T, dV, dK, dQ): 2.5x forward."""
    return 2.5 * prefill_flops(B, T, Hq, d)


def decode_bytes(B, L, Hq, Hkv, d, page, stride):
    kv = 2.0 * B * L * Hkv * d * 2            # K and V, bf16, each byte once
    table = 4.0 * B * stride + 4.0 * B        # page table + seq_lens
    qb = 2.0 * B * Hq * d
    outs = 4.0 * B * Hq * (2 * d + 3)         # dir, count, n_eff, gate, lse
    return kv + table + qb + outs


def traffic_record(kind: str):
    """HBM bytes per launch from the committed counter summary, if the kernels are unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    r = rec.get(kind)
    if r is None or r.get("src_sha256") != src_hash(kind):
        return None
    return r["fetch_bytes"] * rec["fetch_factor"] + r["write_bytes"] * rec["write_factor"]


# Oracle timings run after every GPU leg (each leg queues its own), so that seconds of CPU
# work never sit between a leg's warmup and its timed calls.
CPU_JOBS = []


def blas_threads() -> int:
    """Threads the oracle's NumPy BLAS runs with."""
    try:
        from threadpoolctl import threadpool_info
        return int(max(i["num_threads"] for i in threadpool_info()))
    except Exception:  # pragma: no cover
        return int(os.cpu_count() or 1)


def cpu_baseline(pre, dec):
    """The CPU oracle, as it stands, on a bounded sample of the same two workloads."""
    import oracle
    import synth
    cores = blas_threads()
    rows = np.linspace(0, pre.T - 1, 3072).astype(np.int64)
    t0 = time.perf_counter()
    oracle.polar_prefill(pre.as_f32("q"), pre.as_f32("k"), pre.as_f32("v"), pre.beta,
                         pre.null_bias, pre.count_vec, pre.train_len, pre.flags, rows=rows)
    t_pre = time.perf_counter() - t0
    flops = 4.0 * pre.d * pre.Hq * float((rows + 1).sum())
    batches = list(range(dec.B))
    t0 = time.perf_counter()
    oracle.polar_decode_paged(synth.bf16_bits_to_f32(dec.q), dec.k_pool, dec.v_pool,
                              dec.page_table, dec.seq_lens, dec.page_size, dec.beta,
                              dec.null_bias, dec.count_vec, dec.train_len, dec.flags,
                              to_f64=lambda a: synth.bf16_bits_to_f32(a).astype(np.float64),
                              batches=batches)
    t_dec = time.perf_counter() - t0
    dbytes = decode_bytes(len(batches), dec.max_seq_len, dec.Hq, dec.Hkv, dec.d, dec.page_size,
                          dec.page_table.shape[1])
    return {"value": flops / t_pre / 1e12, "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"prefill rows {len(rows)} evenly spaced of T=65536, all 16 heads "
                      f"({t_pre:.1f} s)",
            "decode": {"value": dbytes / t_dec / 1e9, "unit": "GB/s",
                       "sample": f"decode, all {len(batches)} sequences ({t_dec:.1f} s)"}}


def measure_backward(dev, steps: int, warmup: int, with_cpu: bool):
    """Training forward + backward at the 2K training shape (B=8, T=2048, 16/4 heads)."""
    import torch
    import synth
    from long_context_lm_amd import attn_bwd, attn_fwd_train, bwd_workspace_bytes
    p = synth.prefill_inputs("c2")

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
    kw = dict(beta=torch.from_numpy(p.beta).to(dev), null_bias=torch.from_numpy(p.null_bias).to(dev),
              count_vec=torch.from_numpy(p.count_vec).to(dev), train_len=p.train_len, flags=p.flags)
    cot_np = synth.cotangents(p.B, p.T, p.Hq, p.d).as_dict()
    cot = {n: torch.from_numpy(x).to(dev) for n, x in cot_np.items()}
    ws = torch.empty(bwd_workspace_bytes(p.Hq, p.Hkv, p.B, p.T), dtype=torch.uint8, device=dev)
    fwd = attn_fwd_train(q, k, v, **kw)
    for _ in range(warmup):
        attn_fwd_train(q, k, v, **kw)
        attn_bwd(q, k, v, fwd, cot, workspace=ws, **kw)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        fwd = attn_fwd_train(q, k, v, **kw)
        e[1].record()
        attn_bwd(q, k, v, fwd, cot, workspace=ws, **kw)
        e[2].record()
    torch.cuda.synchronize()
    f_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    b_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    Fb = backward_flops(p.B, p.T, p.Hq, p.d)
    tf = Fb / (b_ms * 1e-3) / 1e12
    rec = {"workload": "backward of the causal prefill, B=8 T=2048 Hq=16 Hkv=4 d=64 bf16 "
                       "(2K training shape), all five cotangents, parameter gradients on",
           "value": round(tf, 2), "unit": "TFLOP/s", "bwd_ms": round(b_ms, 4),
           "fwd_train_ms": round(f_ms, 4),
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                        "traffic": traffic_record("backward")}}
    print(f"[bench] backward mean {b_ms:.3f} ms ({tf:.1f} TFLOP/s), training forward "
          f"{f_ms:.3f} ms", file=sys.stderr, flush=True)
    if with_cpu:
        def job():
            import oracle
            t0 = time.perf_counter()
            oracle.polar_prefill_grad(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), cot_np,
                                      p.beta, p.null_bias, p.count_vec, p.train_len, p.flags)
            t = time.perf_counter() - t0
            rec["cpu_baseline"] = {
                "value": round(backward_flops(p.B, p.T, p.Hq, p.d) / t / 1e12, 5),
                "unit": "TFLOP/s", "cores": int(torch.get_num_threads()), "kind": "oracle",
                "sample": f"float64 autograd backward of the whole workload, all 8 sequences "
                          f"({t:.1f} s)"}
        CPU_JOBS.append(job)
    return rec


def visible_pairs(T: int, window: int) -> float:
    """Sum over rows i of the keys row i sees: i+1, or min(i+1, W) with a window."""
    if window <= 0 or window >= T:
        return T * (T + 1) / 2.0
    return window * (window + 1) / 2.0 + float(T - window) * window


def measure_variants(dev, q, k, v, pkw, pre, steps: int, warmup: int, with_cpu: bool = False):
    """The variant modes on the T=64K workload: RoPE + softmax output over the full causal
    range, and RoPE with a 4096-key sliding window.  With ``with_cpu``, the oracle's variant
    prefill is timed beside each on a bounded sample of rows (RoPE of the whole q and k
    included, as the oracle does it)."""
    import torch
    from long_context_lm_amd import attn_fwd_variant, variant_workspace_bytes
    res = {}
    ws = torch.empty(variant_workspace_bytes(pre.Hq, pre.Hkv, pre.B, pre.T), dtype=torch.uint8,
                     device=dev)
    for name, var in (("rope_softmax_out", dict(window=0, rope_theta=10000.0, workspace=ws)),
                      ("rope_window4096", dict(window=4096, rope_theta=10000.0, workspace=ws))):
        for _ in range(warmup):
            attn_fwd_variant(q, k, v, **var, **pkw)
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in ev:
            e[0].record()
            attn_fwd_variant(q, k, v, **var, **pkw)
            e[1].record()
        torch.cuda.synchronize()
        ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
        F = 4.0 * pre.d * pre.B * pre.Hq * visible_pairs(pre.T, var["window"])
        tf = F / (ms * 1e-3) / 1e12
        res[name] = {"window": var["window"], "rope_theta": var["rope_theta"], "attn_out": True,
                     "ms": round(ms, 4), "value": round(tf, 2), "unit": "TFLOP/s",
                     "roofline": {"bound": "mfma", "achieved": round(tf, 2),
                                  "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                  "traffic": traffic_record("variant_window" if var["window"]
                                                            else "variant")}}
        print(f"[bench] variant {name}: {ms:.3f} ms ({tf:.1f} TFLOP/s)", file=sys.stderr,
              flush=True)
        if with_cpu:
            def job(r=res[name], window=var["window"], theta=var["rope_theta"]):
                import oracle
                n_rows = 1024
                rows = np.linspace(0, pre.T - 1, n_rows).astype(np.int64)
                t0 = time.perf_counter()
                oracle.polar_prefill(pre.as_f32("q"), pre.as_f32("k"), pre.as_f32("v"),
                                     pre.beta, pre.null_bias, pre.count_vec, pre.train_len,
                                     pre.flags, rows=rows, window=window, rope_theta=theta)
                dt = time.perf_counter() - t0
                vis = np.minimum(rows + 1, window) if window else rows + 1
                fl = 4.0 * pre.d * pre.Hq * float(vis.sum())
                r["cpu_baseline"] = {
                    "value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
                    "kind": "oracle",
                    "sample": f"{n_rows} rows evenly spaced of T=65536, all 16 heads, RoPE of "
                              f"the whole q and k included ({dt:.1f} s)"}
            CPU_JOBS.append(job)
    res["workload"] = ("prefill variants at B=1 T=65536 Hq=16 Hkv=4 d=64 bf16: flops over the "
                       "visible pairs of each mode; the time includes rotating the keys once "
                       "into the caller's workspace")
    return res


def measure_decode_b1(dev, steps: int, warmup: int, with_cpu: bool = False):
    """The other reading of the 16 single-token queries: one sequence whose 16 query heads
    decode against a 262,144-token cache (4 KV heads, 268 MB of K and V)."""
    import torch
    import synth
    from long_context_lm_amd import attn_decode_paged, decode_workspace_bytes
    d = synth.decode_inputs("c5", B=1)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    qd, kc, vc = to_dev(d.q), to_dev(d.k_pool), to_dev(d.v_pool)
    table = torch.from_numpy(d.page_table).to(dev)
    lens = torch.from_numpy(d.seq_lens).to(dev)
    kw = dict(beta=torch.from_numpy(d.beta).to(dev), null_bias=torch.from_numpy(d.null_bias).to(dev),
              count_vec=torch.from_numpy(d.count_vec).to(dev), train_len=d.train_len,
              flags=d.flags)
    ws = torch.empty(decode_workspace_bytes(d.Hq, d.Hkv, d.B, d.max_seq_len), dtype=torch.uint8,
                     device=dev)
    f = lambda: attn_decode_paged(qd, kc, vc, table, lens, d.max_seq_len, workspace=ws, **kw)
    for _ in range(warmup):
        f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        f()
        e[1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    byt = decode_bytes(d.B, d.max_seq_len, d.Hq, d.Hkv, d.d, d.page_size, d.page_table.shape[1])
    gbs = byt / (ms * 1e-3) / 1e9
    print(f"[bench] decode B=1: {ms:.3f} ms ({gbs:.1f} GB/s)", file=sys.stderr, flush=True)
    rec = {"workload": "paged decode B=1 L=262144 Hq=16 Hkv=4 d=64 page=64 shuffled table "
                       "(one token's 16 heads)",
           "value": round(gbs, 1), "unit": "GB/s", "ms": round(ms, 4), "bytes": byt,
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": traffic_record("decode_b1")},
           "cpu_baseline": None}
    if with_cpu:
        def job():
            import oracle
            t0 = time.perf_counter()
            oracle.polar_decode_paged(synth.bf16_bits_to_f32(d.q), d.k_pool, d.v_pool,
                                      d.page_table, d.seq_lens, d.page_size, d.beta,
                                      d.null_bias, d.count_vec, d.train_len, d.flags,
                                      to_f64=lambda a: synth.bf16_bits_to_f32(a).astype(np.float64))
            t = time.perf_counter() - t0
            rec["cpu_baseline"] = {"value": byt / t / 1e9, "unit": "GB/s", "cores": blas_threads(),
                                   "kind": "oracle",
                                   "sample": f"the whole workload ({t:.1f} s)"}
        CPU_JOBS.append(job)
    return rec


def measure_paged(dev, pre, steps: int, warmup: int, with_cpu: bool = False):
    """The last 4096-token chunk of the T=64K sequence over a shuffled page pool: KV append
    of the chunk, then its chunked prefill over the 61440 cached tokens and itself.  With
    ``with_cpu``, the oracle's chunked prefill is timed on the chunk's first 512 rows."""
    import torch
    import synth
    from long_context_lm_amd import attn_prefill_paged, kv_append
    C, start = 4096, pre.T - 4096
    ci = synth.chunk_inputs(B=1, C=C, starts=(start,), full=pre)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    kc, vc = to_dev(ci.k_pool), to_dev(ci.v_pool)
    table = torch.from_numpy(ci.page_table).to(dev)
    sp = torch.from_numpy(ci.start_pos).to(dev)
    qn, kn, vn = to_dev(ci.chunk("q")), to_dev(ci.chunk("k")), to_dev(ci.chunk("v"))
    kw = dict(beta=torch.from_numpy(pre.beta).to(dev), count_vec=torch.from_numpy(pre.count_vec).to(dev),
              null_bias=torch.from_numpy(pre.null_bias).to(dev), train_len=pre.train_len,
              flags=pre.flags)
    for _ in range(warmup):
        kv_append(kn, vn, kc, vc, table, sp, ci.max_seq_len)
        attn_prefill_paged(qn, kc, vc, table, sp, ci.max_seq_len, **kw)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        kv_append(kn, vn, kc, vc, table, sp, ci.max_seq_len)
        e[1].record()
        attn_prefill_paged(qn, kc, vc, table, sp, ci.max_seq_len, **kw)
        e[2].record()
    torch.cuda.synchronize()
    a_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    p_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    F = 4.0 * pre.d * pre.Hq * float(np.sum(start + np.arange(C) + 1.0))
    tf = F / (p_ms * 1e-3) / 1e12
    a_bytes = 2.0 * 2 * C * pre.Hkv * pre.d * 2            # K and V, read and written once
    gbs = a_bytes / (a_ms * 1e-3) / 1e9
    print(f"[bench] paged: append {a_ms * 1e3:.1f} us ({gbs:.0f} GB/s), chunked prefill "
          f"{p_ms:.3f} ms ({tf:.1f} TFLOP/s)", file=sys.stderr, flush=True)
    rec = {"workload": "last 4096-token chunk of the B=1 T=65536 Hq=16 Hkv=4 d=64 bf16 sequence "
                       "(61440 tokens cached in shuffled 64-token pages)",
           "cpu_baseline": None,
           "value": round(tf, 2), "unit": "TFLOP/s", "prefill_ms": round(p_ms, 4),
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                        "traffic": traffic_record("paged")},
           "append": {"us": round(a_ms * 1e3, 2), "value": round(gbs, 1), "unit": "GB/s",
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                   "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                   "frac": round(gbs / PEAK_HBM_GBS, 4),
                                   "traffic": traffic_record("append")}}}
    if with_cpu:
        def job():
            import oracle
            n_rows = 512
            # the chunk's own keys are appended first (untimed), as on the GPU
            kp, vp = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, ci.start_pos,
                                      ci.chunk("k"), ci.chunk("v"), ci.page_size, ci.max_seq_len)
            t0 = time.perf_counter()
            oracle.polar_prefill_paged(synth.bf16_bits_to_f32(ci.chunk("q"))[:, :n_rows], kp, vp,
                                       ci.page_table, ci.start_pos, ci.page_size, pre.beta,
                                       pre.null_bias, pre.count_vec, pre.train_len, pre.flags,
                                       to_f64=lambda a: synth.bf16_bits_to_f32(a).astype(np.float64))
            dt = time.perf_counter() - t0
            fl = 4.0 * pre.d * pre.Hq * float(np.sum(start + np.arange(n_rows) + 1.0))
            rec["cpu_baseline"] = {"value": fl / dt / 1e12, "unit": "TFLOP/s",
                                   "cores": blas_threads(), "kind": "oracle",
                                   "sample": f"first {n_rows} rows of the chunk, all 16 heads "
                                             f"({dt:.1f} s)"}
        CPU_JOBS.append(job)
    return rec


def _delta_setup(dev):
    import torch
    import synth
    d = synth.delta_inputs()                     # B=256 sequences, H=16, 1024-slot pool

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    return d, (torch.from_numpy(d.pool).to(dev), torch.from_numpy(d.slots).to(dev), bf(d.q),
               bf(d.k), bf(d.v), torch.from_numpy(d.alpha).to(dev), torch.from_numpy(d.beta).to(dev))


def delta_step_reference(pool, slots, q, k, v, alpha, beta):
    """The same step written as separate torch operations on a gathered batch and scattered
    back (the gather-scatter form the pages' in-place kernel replaces).  Measurement aid."""
    import torch
    idx = slots.long()
    S = pool[idx]                                            # gather  [B,H,dv,dk]
    qn = torch.nn.functional.normalize(q.float(), dim=-1, eps=1e-6)
    kn = torch.nn.functional.normalize(k.float(), dim=-1, eps=1e-6)
    Sk = torch.matmul(S, kn.unsqueeze(-1)).squeeze(-1)
    Sq = torch.matmul(S, qn.unsqueeze(-1)).squeeze(-1)
    u = beta.unsqueeze(-1) * (v.float() - alpha.unsqueeze(-1) * Sk)
    S = alpha[..., None, None] * S + u.unsqueeze(-1) * kn.unsqueeze(-2)
    o = alpha.unsqueeze(-1) * Sq + u * (kn * qn).sum(-1, keepdim=True)
    pool[idx] = S                                            # scatter
    return o


def measure_memory_step(dev, steps: int, warmup: int, with_cpu: bool = False):
    """In-place gated-delta step for 256 sequences x 16 heads (64x64 fp32 states in a
    1024-slot pool), and the gather-scatter torch form of the same step beside it."""
    import torch
    from long_context_lm_amd import delta_step
    d, (pool, sl, q, k, v, al, be) = _delta_setup(dev)
    B, H = d.q.shape[:2]
    times = {}
    for name, fn in (("fused", lambda: delta_step(pool, sl, q, k, v, al, be)),
                     ("reference", lambda: delta_step_reference(pool, sl, q, k, v, al, be))):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in ev:
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        times[name] = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    state = B * H * 64 * 64 * 4
    algo = 2.0 * state + B * H * 64 * (3 * 2 + 4) + B * H * 8 + B * 4
    gbs = algo / (times["fused"] * 1e-3) / 1e9
    print(f"[bench] memory step: fused {times['fused'] * 1e3:.1f} us ({gbs:.0f} GB/s), "
          f"gather-scatter torch form {times['reference'] * 1e3:.1f} us", file=sys.stderr,
          flush=True)
    rec = {"workload": "in-place gated-delta memory step, 256 sequences x 16 heads, 64x64 fp32 "
                       "states in a 1024-slot pool, bf16 q/k/v",
           "value": round(gbs, 1), "unit": "GB/s", "us": round(times["fused"] * 1e3, 2),
           "reference_us": round(times["reference"] * 1e3, 2),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                        "traffic": traffic_record("memory_step")}}
    if with_cpu:
        def job():
            import oracle
            t0 = time.perf_counter()
            oracle.delta_step_pool(d.pool, d.slots, d.as_f32("q"), d.as_f32("k"),
                                   d.as_f32("v"), d.alpha, d.beta)
            t = time.perf_counter() - t0
            rec["cpu_baseline"] = {"value": round(algo / t / 1e9, 3), "unit": "GB/s",
                                   "cores": 1, "kind": "oracle",
                                   "sample": f"float64 step of all 256 x 16 states ({t:.1f} s)"}
        CPU_JOBS.append(job)
    return rec


def memory_step_probe(which: str, steps: int):
    """Run only one form of the memory step (for per-step HBM counters)."""
    import torch
    from long_context_lm_amd import _lib, delta_step
    _lib.load()
    d, (pool, sl, q, k, v, al, be) = _delta_setup("cuda")
    fn = (lambda: delta_step(pool, sl, q, k, v, al, be)) if which == "fused" else \
        (lambda: delta_step_reference(pool, sl, q, k, v, al, be))
    torch.cuda.synchronize()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    print(json.dumps({"memory_step_probe": which, "steps": steps}))


def copy_probe(nbytes: int):
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0)
    ap.add_argument("--memory-step-probe", choices=("fused", "ref"), default=None)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the Polar Attention path here is a single-GPU "
              "kernel library (see the sharding notes in DESIGN.md); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.memory_step_probe:
        memory_step_probe(args.memory_step_probe, args.steps)
        return

    import torch
    import synth
    from long_context_lm_amd import _lib, attn_decode_paged, attn_fwd
    _lib.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda"

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    pre = synth.prefill_inputs("c4")
    dec = synth.decode_inputs("c5")
    q, k, v = to_dev(pre.q), to_dev(pre.k), to_dev(pre.v)
    pkw = dict(beta=torch.from_numpy(pre.beta).to(dev), null_bias=torch.from_numpy(pre.null_bias).to(dev),
               count_vec=torch.from_numpy(pre.count_vec).to(dev), train_len=pre.train_len,
               flags=pre.flags)
    qd, kc, vc = to_dev(dec.q), to_dev(dec.k_pool), to_dev(dec.v_pool)
    table = torch.from_numpy(dec.page_table).to(dev)
    lens = torch.from_numpy(dec.seq_lens).to(dev)
    dkw = dict(beta=torch.from_numpy(dec.beta).to(dev), null_bias=torch.from_numpy(dec.null_bias).to(dev),
               count_vec=torch.from_numpy(dec.count_vec).to(dev), train_len=dec.train_len,
               flags=dec.flags)
    from long_context_lm_amd import decode_workspace_bytes
    ws = torch.empty(decode_workspace_bytes(dec.Hq, dec.Hkv, dec.B, dec.max_seq_len),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs resident: prefill T={pre.T}, decode B={dec.B} L={dec.max_seq_len}",
          file=sys.stderr, flush=True)

    def step(evs=None):
        if evs:
            evs[0].record()
        attn_fwd(q, k, v, **pkw)
        if evs:
            evs[1].record()
        attn_decode_paged(qd, kc, vc, table, lens, dec.max_seq_len, workspace=ws, **dkw)
        if evs:
            evs[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    t_pre = [e[0].elapsed_time(e[1]) for e in events]
    t_dec = [e[1].elapsed_time(e[2]) for e in events]
    F = prefill_flops(pre.B, pre.T, pre.Hq, pre.d)
    Dbytes = decode_bytes(dec.B, dec.max_seq_len, dec.Hq, dec.Hkv, dec.d, dec.page_size,
                          dec.page_table.shape[1])
    pre_ms = float(np.mean(t_pre))
    dec_ms = float(np.mean(t_dec))
    tflops = F / (pre_ms * 1e-3) / 1e12
    gbs = Dbytes / (dec_ms * 1e-3) / 1e9
    print(f"[bench] prefill mean {pre_ms:.3f} ms (median {np.median(t_pre):.3f}), "
          f"decode mean {dec_ms:.3f} ms (median {np.median(t_dec):.3f})", file=sys.stderr,
          flush=True)
    tr_pre = traffic_record("prefill")
    tr_dec = traffic_record("decode")
    rec = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill B=1 T=65536 Hq=16 Hkv=4 d=64 causal bf16 (T=64K, "
                               "32x train length, 8 needles) + paged decode B=16 L=262144 "
                               "Hq=16 Hkv=4 d=64 page=64 shuffled table (256K KV)",
                   "prefill_ms": round(pre_ms, 4), "decode_ms": round(dec_ms, 4)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": tr_pre},
        "decode": {"value": round(gbs, 1), "unit": "GB/s", "ms": round(dec_ms, 4),
                   "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                "traffic": tr_dec}},
    }
    rec["variants"] = measure_variants(dev, q, k, v, pkw, pre, max(1, args.steps // 4),
                                       min(args.warmup, 2), not args.no_cpu_baseline)
    rec["paged"] = measure_paged(dev, pre, max(1, args.steps // 2), min(args.warmup, 2),
                                 not args.no_cpu_baseline)
    del q, k, v, qd, kc, vc, table, lens, ws
    torch.cuda.empty_cache()
    rec["decode_b1"] = measure_decode_b1(dev, args.steps, min(args.warmup, 2),
                                         not args.no_cpu_baseline)
    torch.cuda.empty_cache()
    rec["backward"] = measure_backward(dev, max(1, args.steps // 2), args.warmup,
                                       not args.no_cpu_baseline)
    rec["memory_step"] = measure_memory_step(dev, args.steps, args.warmup,
                                             not args.no_cpu_baseline)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on bounded samples", file=sys.stderr, flush=True)
        rec["cpu_baseline"] = cpu_baseline(pre, dec)
        for job in CPU_JOBS:
            job()
    else:
        rec["cpu_baseline"] = None
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

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
forward count); ``backward.variant`` times the same for the 512-key window + RoPE arm.

Besides the headline pair, the JSON line carries one object per further leg, each with its
own roofline and, unless ``--no-cpu-baseline``, the oracle timed beside it: the forward at
the 2K training shape and at 16K (``prefill_c2``, ``prefill_c3``), the variant modes, the
paged chunk, the one-sequence decode, the backward, the memory step and the memory stream
over whole sequences (``memory_sequence``, fp32 TFLOP/s of 7 d^2 per token and head).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                       [--legs all|LEG,LEG...]  (a subset of the extra legs, for profiling)
       python bench.py --copy-probe BYTES   (plain device copy, for counter calibration)
       python bench.py --memory-step-probe fused|ref --steps K
                                            (one form of the memory step, for counters)
       python bench.py --memory-sequence-probe --steps K
                                            (the memory-stream launch alone, for counters)
       python bench.py --counter-summary DIR  (profiles/ summaries from a rocprofv3 run)
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
PEAK_FP32_TFLOPS = 157.3        # MI355X fp32 vector (published; counts packed fp32 FMA)


# Sources each timed kernel is built from; a counter record stays valid while these are unchanged.
_PREFILL_SRC = ["polar_prefill.hip", "polar_mfma.h", "polar_kernels.h", "polar_rope.h"]
_DECODE_SRC = ["polar_decode.hip", "polar_mfma.h", "polar_kernels.h"]
KERNEL_SOURCES = {
    "prefill": _PREFILL_SRC,
    "prefill_c2": _PREFILL_SRC,
    "prefill_c3": _PREFILL_SRC,
    "decode": _DECODE_SRC,
    "decode_b1": _DECODE_SRC,
    "backward": ["polar_backward.hip", "polar_mfma.h", "polar_kernels.h", "polar_rope.h"],
    "variant": _PREFILL_SRC,            # key rotation + variant prefill, full causal range
    "variant_window": _PREFILL_SRC,     # key rotation + variant prefill, 4096-key window
    "paged": _PREFILL_SRC,
    "append": ["polar_paged.hip", "polar_kernels.h"],
    "memory_step": ["polar_delta.hip", "polar_kernels.h"],
    "memory_sequence": ["polar_delta.hip", "polar_kernels.h"],
    "fwd_train": _PREFILL_SRC,          # the training forward beside the backward
    # the window + RoPE arm: rotations, windowed training forward, windowed backward kernels
    "backward_variant": ["polar_backward.hip", "polar_prefill.hip", "polar_mfma.h",
                         "polar_kernels.h", "polar_rope.h"],
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


def cpu_model() -> str:
    """The host CPU's model name (the oracle's machine)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


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
            "kind": "oracle", "cpu": cpu_model(),
            "sample": f"prefill rows {len(rows)} evenly spaced of T=65536, all 16 heads "
                      f"({t_pre:.1f} s)",
            "decode": {"value": dbytes / t_dec / 1e9, "unit": "GB/s",
                       "sample": f"decode, all {len(batches)} sequences ({t_dec:.1f} s)"}}


def warm_up(fn, calls: int, min_ms: float = 100.0):
    """``calls`` warmup calls, then more until the GPU has run this call for ``min_ms`` of
    wall time: a GPU that sat idle while the host drew a leg's inputs runs its first
    launches at a lower clock, and short legs would otherwise time that ramp."""
    import torch
    for _ in range(calls):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()


def measure_prefill_cfg(dev, name: str, steps: int, warmup: int, with_cpu: bool):
    """The causal forward on another of the pages' shapes: "c2" (B=8, T=2048, the training
    length, 5% planted near-copy keys) or "c3" (B=1, T=16384, 8x the training length, one
    needle per head), with the oracle timed on all of C2 or on 1024 rows of C3."""
    import torch
    import synth
    from long_context_lm_amd import attn_fwd
    p = synth.prefill_inputs(name)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = to_dev(p.q), to_dev(p.k), to_dev(p.v)
    kw = dict(beta=torch.from_numpy(p.beta).to(dev), null_bias=torch.from_numpy(p.null_bias).to(dev),
              count_vec=torch.from_numpy(p.count_vec).to(dev), train_len=p.train_len, flags=p.flags)
    warm_up(lambda: attn_fwd(q, k, v, **kw), warmup)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        attn_fwd(q, k, v, **kw)
        e[1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    F = prefill_flops(p.B, p.T, p.Hq, p.d)
    tf = F / (ms * 1e-3) / 1e12
    print(f"[bench] prefill {name} B={p.B} T={p.T}: {ms:.4f} ms ({tf:.1f} TFLOP/s)",
          file=sys.stderr, flush=True)
    rec = {"workload": f"prefill B={p.B} T={p.T} Hq=16 Hkv=4 d=64 causal bf16 "
                       + ("(2K training length, 5% planted near-copy keys)" if name == "c2"
                          else "(16K, 8x train length, one needle per head)"),
           "value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                        "traffic": traffic_record("prefill_" + name)},
           "cpu_baseline": None}
    if with_cpu:
        def job():
            import oracle
            rows = None if name == "c2" else np.linspace(0, p.T - 1, 1024).astype(np.int64)
            t0 = time.perf_counter()
            oracle.polar_prefill(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.beta,
                                 p.null_bias, p.count_vec, p.train_len, p.flags, rows=rows)
            t = time.perf_counter() - t0
            r = np.arange(p.T) if rows is None else rows
            fl = 4.0 * p.d * p.B * p.Hq * float((r + 1).sum())
            rec["cpu_baseline"] = {
                "value": fl / t / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
                "kind": "oracle", "cpu": cpu_model(),
                "sample": ("the whole workload, all 8 sequences" if rows is None else
                           "1024 rows evenly spaced of T=16384, all 16 heads") + f" ({t:.1f} s)"}
        CPU_JOBS.append(job)
    return rec


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
    warm_up(lambda: (attn_fwd_train(q, k, v, **kw), attn_bwd(q, k, v, fwd, cot, workspace=ws, **kw)),
            warmup)
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
    rec["variant"] = measure_backward_variant(dev, steps, warmup, q, k, v, kw, cot, p)
    if with_cpu:
        def job():
            import oracle
            t0 = time.perf_counter()
            oracle.polar_prefill_grad(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), cot_np,
                                      p.beta, p.null_bias, p.count_vec, p.train_len, p.flags)
            t = time.perf_counter() - t0
            rec["cpu_baseline"] = {
                "value": round(backward_flops(p.B, p.T, p.Hq, p.d) / t / 1e12, 5),
                "unit": "TFLOP/s", "cores": int(torch.get_num_threads()), "kind": "oracle", "cpu": cpu_model(),
                "sample": f"float64 autograd backward of the whole workload, all 8 sequences "
                          f"({t:.1f} s)"}
        CPU_JOBS.append(job)
    return rec


def measure_backward_variant(dev, steps: int, warmup: int, q, k, v, kw, cot, p,
                             window: int = 512, theta: float = 10000.0):
    """Training forward + backward of the window + RoPE arm at the same 2K shape: the
    rotations of q and k and the windowed kernels (which turn dq and dk back)."""
    import torch
    from long_context_lm_amd import attn_bwd, attn_fwd_train, bwd_workspace_bytes
    from long_context_lm_amd import train_variant_workspace_bytes
    vw = dict(window=window, rope_theta=theta)
    wf = torch.empty(train_variant_workspace_bytes(p.Hq, p.Hkv, p.B, p.T, **vw),
                     dtype=torch.uint8, device=dev)
    wb = torch.empty(bwd_workspace_bytes(p.Hq, p.Hkv, p.B, p.T, **vw), dtype=torch.uint8,
                     device=dev)
    fwd = attn_fwd_train(q, k, v, workspace=wf, **vw, **kw)
    warm_up(lambda: (attn_fwd_train(q, k, v, workspace=wf, **vw, **kw),
                     attn_bwd(q, k, v, fwd, cot, workspace=wb, **vw, **kw)), warmup)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        fwd = attn_fwd_train(q, k, v, workspace=wf, **vw, **kw)
        e[1].record()
        attn_bwd(q, k, v, fwd, cot, workspace=wb, **vw, **kw)
        e[2].record()
    torch.cuda.synchronize()
    f_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    b_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    Fb = 2.5 * 4.0 * p.d * p.B * p.Hq * visible_pairs(p.T, window)
    tf = Fb / (b_ms * 1e-3) / 1e12
    print(f"[bench] backward, window {window} + RoPE: {b_ms:.3f} ms ({tf:.1f} TFLOP/s), "
          f"training forward {f_ms:.3f} ms", file=sys.stderr, flush=True)
    return {"workload": f"backward of the {window}-key window + RoPE (theta {theta:g}) "
                        "prefill at the same shape, the rotation of q and k included (the "
                        "kernels turn dq and dk back as they store them)",
            "value": round(tf, 2), "unit": "TFLOP/s", "bwd_ms": round(b_ms, 4),
            "fwd_train_ms": round(f_ms, 4),
            "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                         "traffic": traffic_record("backward_variant")}}


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
        warm_up(lambda: attn_fwd_variant(q, k, v, **var, **pkw), warmup)
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
                                     pre.flags, rows=rows, window=window, rope_theta=theta,
                                     rope_bf16=True)
                dt = time.perf_counter() - t0
                vis = np.minimum(rows + 1, window) if window else rows + 1
                fl = 4.0 * pre.d * pre.Hq * float(vis.sum())
                r["cpu_baseline"] = {
                    "value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": blas_threads(),
                    "kind": "oracle", "cpu": cpu_model(),
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
    warm_up(f, warmup)
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
                                   "kind": "oracle", "cpu": cpu_model(),
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
    warm_up(lambda: (kv_append(kn, vn, kc, vc, table, sp, ci.max_seq_len),
                     attn_prefill_paged(qn, kc, vc, table, sp, ci.max_seq_len, **kw)), warmup)
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
                                   "cores": blas_threads(), "kind": "oracle", "cpu": cpu_model(),
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
        warm_up(fn, warmup)
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
                                   "cores": 1, "kind": "oracle", "cpu": cpu_model(),
                                   "sample": f"float64 step of all 256 x 16 states ({t:.1f} s)"}
        CPU_JOBS.append(job)
    return rec


SEQ_SHAPE = dict(B=32, T=2048, H=16)       # 32 training sequences of 2K tokens, 16 heads


def delta_seq_flops(B, T, H, d=64):
    """Algorithmic fp32 work of the memory stream: per (token, head) S k and S q (2 d^2
    flops each) and S' = alpha S + u k^T (3 d^2), 7 d^2 in all."""
    return 7.0 * d * d * B * T * H


def _delta_seq_setup(dev):
    import torch
    import synth
    d = synth.delta_seq_inputs(**SEQ_SHAPE, num_slots=64, dtype="bf16")

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    return d, (torch.from_numpy(d.pool).to(dev), torch.from_numpy(d.slots).to(dev), bf(d.q),
               bf(d.k), bf(d.v), torch.from_numpy(d.alpha).to(dev), torch.from_numpy(d.beta).to(dev))


def measure_memory_sequence(dev, steps: int, warmup: int, with_cpu: bool = False):
    """The memory stream over 32 sequences x 2048 tokens x 16 heads in one launch, and the
    same tokens as 2048 chained one-step launches beside it."""
    import torch
    from long_context_lm_amd import delta_sequence, delta_step
    d, (pool, sl, q, k, v, al, be) = _delta_seq_setup(dev)
    B, T, H = SEQ_SHAPE["B"], SEQ_SHAPE["T"], SEQ_SHAPE["H"]
    warm_up(lambda: delta_sequence(pool, sl, q, k, v, al, be), warmup)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        delta_sequence(pool, sl, q, k, v, al, be)
        e[1].record()
    torch.cuda.synchronize()
    ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    # The same work as T step launches on per-token slices laid out beforehand.
    qt, kt, vt = (x.transpose(0, 1).contiguous() for x in (q, k, v))
    at, bt = al.transpose(0, 1).contiguous(), be.transpose(0, 1).contiguous()
    delta_step(pool, sl, qt[0], kt[0], vt[0], at[0], bt[0])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for t in range(T):
        delta_step(pool, sl, qt[t], kt[t], vt[t], at[t], bt[t])
    e1.record()
    torch.cuda.synchronize()
    chained_ms = e0.elapsed_time(e1)
    del qt, kt, vt, at, bt
    fl = delta_seq_flops(B, T, H)
    tf = fl / (ms * 1e-3) / 1e12
    print(f"[bench] memory sequence: {ms:.3f} ms ({tf:.1f} TFLOP/s, "
          f"{B * T / (ms * 1e-3) / 1e6:.1f} M tokens/s), {T} chained steps {chained_ms:.2f} ms",
          file=sys.stderr, flush=True)
    rec = {"workload": f"gated-delta memory stream over {B} sequences x {T} tokens x {H} heads, "
                       "64x64 fp32 states in a 64-slot pool, bf16 q/k/v",
           "value": round(tf, 2), "unit": "TFLOP/s", "ms": round(ms, 4),
           "tokens_per_s": round(B * T / (ms * 1e-3), 0),
           "chained_steps_ms": round(chained_ms, 3),
           "roofline": {"bound": "alu", "achieved": round(tf, 2), "peak": PEAK_FP32_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / PEAK_FP32_TFLOPS, 4),
                        "traffic": traffic_record("memory_sequence")}}
    if with_cpu:
        def job():
            import oracle
            import synth
            nb = 4
            q1, k1, v1 = (synth.bf16_bits_to_f32(x[:nb]) for x in (d.q, d.k, d.v))
            t0 = time.perf_counter()
            oracle.delta_sequence_pool(d.pool, d.slots[:nb], q1, k1, v1, d.alpha[:nb],
                                       d.beta[:nb])
            t = time.perf_counter() - t0
            rec["cpu_baseline"] = {"value": round(delta_seq_flops(nb, T, H) / t / 1e12, 6),
                                   "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
                                   "cpu": cpu_model(),
                                   "sample": f"float64 stream of {nb} of the {B} sequences, all "
                                             f"{T} tokens and {H} heads ({t:.1f} s)"}
        CPU_JOBS.append(job)
    return rec


def memory_sequence_probe(steps: int):
    """Run only the memory-stream launch (for per-launch HBM counters)."""
    import torch
    from long_context_lm_amd import _lib, delta_sequence
    _lib.load()
    d, (pool, sl, q, k, v, al, be) = _delta_seq_setup("cuda")
    torch.cuda.synchronize()
    for _ in range(steps):
        delta_sequence(pool, sl, q, k, v, al, be)
    torch.cuda.synchronize()
    print(json.dumps({"memory_sequence_probe": True, "steps": steps}))


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


# ------------------------------------------------------------------ counter summaries
# Which dispatches make up each leg: (kernel-name pattern, grid size or None, duration
# class).  Dispatches of one kernel and grid are split into classes where their sorted
# durations jump by more than 1.6x (the 2K and 16K forwards share a grid, as do the full
# and windowed variants); class -1 is the longest, 0 the shortest.
LEG_KERNELS = {
    "prefill": [(r"polar_prefill_kernel<Bf16, 1, 8, 0,", 2097152, -1)],
    "decode": [(r"polar_decode_split_kernel<Bf16>", 262144, -1),
               (r"polar_decode_combine_kernel", 262144, -1)],
    "variant": [(r"polar_rope_keys_kernel<unsigned short>", None, -1),
                (r"polar_prefill_kernel<Bf16, 1, 8, 2,", 2097152, -1)],
    "variant_window": [(r"polar_rope_keys_kernel<unsigned short>", None, -1),
                       (r"polar_prefill_kernel<Bf16, 1, 8, 2,", 2097152, 0)],
    "paged": [(r"polar_prefill_kernel<Bf16, 1, 16, 3,", None, -1)],
    "append": [(r"polar_kv_append_kernel", None, -1)],
    "prefill_c2": [(r"polar_prefill_kernel<Bf16, 1, 8, 0,", 524288, 0)],
    "prefill_c3": [(r"polar_prefill_kernel<Bf16, 1, 8, 0,", 524288, -1)],
    "decode_b1": [(r"polar_decode_split_kernel<Bf16>", 131072, -1),
                  (r"polar_decode_combine_kernel", 16384, -1)],
    "backward": [(r"polar_bwd_prep_kernel", None, -1),
                 (r"polar_bwd_dq_kernel<8, false>", None, -1),
                 (r"polar_bwd_dkv_kernel<4, 1, false, false>", None, -1),
                 (r"polar_bwd_dkv_add_kernel", None, -1),
                 (r"polar_bwd_param_kernel", None, -1),
                 (r"polar_bwd_param_final_kernel", None, -1)],
    "fwd_train": [(r"polar_prefill_kernel<Bf16, 1, 8, 1,", None, -1)],
    "backward_variant": [(r"polar_rope_qk_kernel<unsigned short>", None, -1),
                         (r"polar_prefill_kernel<Bf16, 1, 8, 6,", None, -1),
                         (r"polar_bwd_dq_kernel<8, true>", None, -1),
                         (r"polar_bwd_dkv_kernel<4, 1, true, true>", None, -1)],
    "memory_step": [(r"polar_delta_step_kernel<unsigned short, 4>", 262144, -1)],
    "memory_sequence": [(r"polar_delta_seq_kernel<unsigned short,", None, -1)],
}
LEG_WORKLOAD = {
    "prefill": "causal prefill B=1 T=65536 Hq=16 Hkv=4 d=64 bf16",
    "decode": "paged decode B=16 L=262144 Hq=16 Hkv=4 d=64 page 64",
    "variant": "RoPE + softmax-output variant prefill, T=65536 (key rotation included)",
    "variant_window": "the same with a 4096-key window",
    "paged": "last 4096-token chunk of T=65536 from 64-token pages",
    "append": "KV append of that 4096-token chunk",
    "prefill_c2": "causal prefill B=8 T=2048 (training shape)",
    "prefill_c3": "causal prefill B=1 T=16384",
    "decode_b1": "paged decode B=1 L=262144",
    "backward": "backward B=8 T=2048, all cotangents, parameter gradients",
    "fwd_train": "training forward B=8 T=2048 (saves lse, S, Q for the backward)",
    "backward_variant": "window 512 + RoPE arm at B=8 T=2048: q/k rotation, windowed "
                        "training forward, windowed dq and dk/dv turning dq and dk back "
                        "(the prep, partial-add and parameter kernels are the backward "
                        "leg's)",
    "memory_step": "gated-delta step, 256 sequences x 16 heads",
    "memory_sequence": "gated-delta stream, 32 sequences x 2048 tokens x 16 heads",
}
# Algorithmic bf16 flops of the legs whose MFMA counters are summarised.
LEG_FLOPS = {"prefill": lambda: prefill_flops(1, 65536, 16, 64),
             "prefill_c2": lambda: prefill_flops(8, 2048, 16, 64),
             "prefill_c3": lambda: prefill_flops(1, 16384, 16, 64),
             "fwd_train": lambda: prefill_flops(8, 2048, 16, 64),
             "backward": lambda: backward_flops(8, 2048, 16, 64)}
N_SIMD = 1024                    # 256 CUs x 4 SIMDs
NOMINAL_GHZ = 2.4


def _kernel_short(name: str) -> str:
    """Demangled kernel name without namespaces and without the parameter list."""
    name = name.replace("polar::(anonymous namespace)::", "").replace("polar::", "")
    name = name.replace("void ", "")
    depth = 0
    for i in range(len(name) - 1, -1, -1):
        if name[i] == ")":
            depth += 1
        elif name[i] == "(":
            depth -= 1
            if depth == 0:
                return name[:i]
    return name


def _read_dispatches(path: str):
    """{dispatch id: {"name", "grid", "ns", counter: value}} from a rocprofv3 CSV (kernel
    trace or counter collection)."""
    import csv
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["Dispatch_Id"])
            if "Grid_Size" in r:
                grid = int(r["Grid_Size"])
            else:
                grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
            e = out.setdefault(d, {"name": _kernel_short(r["Kernel_Name"]), "grid": grid,
                                   "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
            if "Counter_Name" in r:
                e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _leg_dispatches(disp, pattern: str, grid, cls: int):
    """Dispatch ids of one (kernel, grid, duration class), in dispatch order."""
    import re
    cand = sorted((e["ns"], d) for d, e in disp.items()
                  if re.match(pattern, e["name"]) and (grid is None or e["grid"] == grid))
    if not cand:
        return []
    # The first dispatch of a kernel in the process runs cold (up to twice as long) and is
    # always a warmup: it is left out before the duration classes are formed.
    if len(cand) > 2:
        first = min(d for _, d in cand)
        cand = [c for c in cand if c[1] != first]
    classes = [[cand[0]]]
    for item in cand[1:]:
        if item[0] > 1.6 * classes[-1][-1][0]:
            classes.append([item])
        else:
            classes[-1].append(item)
    return sorted(d for _, d in classes[cls])


def _mean(vals):
    vals = list(vals)
    return sum(vals) / len(vals) if vals else float("nan")


def counter_summary(indir: str, outdir: str) -> None:
    """Write the profiles/ summaries from one counter-collection directory: subfolders kt
    (kernel trace), fetch, write, cfetch, cwrite (FETCH_SIZE / WRITE_SIZE of the run and of
    a 1 GiB copy) and mfma1, mfma2 (MFMA, VALU, LDS and wait counters)."""
    def csv_of(sub, kind):
        hits = glob.glob(os.path.join(indir, sub, f"*_{kind}.csv"))
        if len(hits) != 1:
            raise SystemExit(f"expected one *_{kind}.csv under {indir}/{sub}, found {hits}")
        return hits[0]
    kt = _read_dispatches(csv_of("kt", "kernel_trace"))
    fetch = _read_dispatches(csv_of("fetch", "counter_collection"))
    write = _read_dispatches(csv_of("write", "counter_collection"))
    cf = _read_dispatches(csv_of("cfetch", "counter_collection"))
    cw = _read_dispatches(csv_of("cwrite", "counter_collection"))
    m1 = _read_dispatches(csv_of("mfma1", "counter_collection"))
    m2 = _read_dispatches(csv_of("mfma2", "counter_collection"))
    copy_bytes = float(1 << 30)
    cf_kib = max(e["FETCH_SIZE"] for e in cf.values() if "copyBuffer" in e["name"])
    cw_kib = max(e["WRITE_SIZE"] for e in cw.values() if "copyBuffer" in e["name"])
    f_fac, w_fac = copy_bytes / (cf_kib * 1024), copy_bytes / (cw_kib * 1024)
    bench_cmd = "python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline"
    legs_cmd = bench_cmd + " --legs c2,c3,backward,memory_sequence"
    head = [
        "# rocprofv3 commands (run from /tmp with TMPDIR=/tmp; <R> is the repository, <O> the",
        "# output directory; each --pmc pass is a run of its own):",
        f"#   rocprofv3 --kernel-trace --stats --output-format csv -d <O>/kt -o kt -- {bench_cmd}",
        f"#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <O>/fetch -o fetch -- {bench_cmd}",
        f"#   rocprofv3 --pmc WRITE_SIZE GRBM_GUI_ACTIVE --output-format csv -d <O>/write -o write -- {bench_cmd}",
        "#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <O>/cfetch -o cfetch -- python3 bench.py --copy-probe 1073741824",
        "#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <O>/cwrite -o cwrite -- python3 bench.py --copy-probe 1073741824",
        "#   rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CU_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_MFMA "
        f"SQ_INSTS_VALU SQ_INSTS_VALU_TRANS_F32 GRBM_GUI_ACTIVE --output-format csv -d <O>/mfma1 -o mfma1 -- {legs_cmd}",
        "#   rocprofv3 --pmc SQ_VALU_MFMA_COEXEC_CYCLES SQ_ACTIVE_INST_VALU SQ_WAIT_INST_ANY SQ_WAVE_CYCLES "
        f"SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE GRBM_GUI_ACTIVE --output-format csv -d <O>/mfma2 -o mfma2 -- {legs_cmd}",
        "# summarised by: python3 bench.py --counter-summary <O>",
        "# legs:",
    ] + [f"#   {leg:16s} {desc}" for leg, desc in LEG_WORKLOAD.items()]
    sha = {leg: src_hash(leg) for leg in KERNEL_SOURCES}
    head += [f"# {leg} kernel sources sha256: {h}" for leg, h in sha.items()]

    # Kernel trace: per leg and kernel, the dispatches' mean duration (the first dispatch of
    # each class, a warmup, left out when there are more).
    lines = head + ["", "# kernel trace: mean duration per launch over each leg's timed dispatches",
                    f"{'leg':16s} {'kernel':52s} {'grid':>9s} {'n':>3s} {'mean_us':>10s} "
                    f"{'min_us':>9s} {'max_us':>9s}"]
    trace_us = {}
    for leg, spec in LEG_KERNELS.items():
        for pat, grid, cls in spec:
            ids = _leg_dispatches(kt, pat, grid, cls)
            if not ids:
                continue
            timed = ids[1:] if len(ids) > 1 else ids
            ns = [kt[d]["ns"] for d in timed]
            name = kt[ids[0]]["name"]
            trace_us[(leg, name)] = _mean(ns) / 1e3
            lines.append(f"{leg:16s} {name:52s} {kt[ids[0]]['grid']:9d} {len(timed):3d} "
                         f"{_mean(ns) / 1e3:10.1f} {min(ns) / 1e3:9.1f} {max(ns) / 1e3:9.1f}")
    with open(os.path.join(outdir, "kernel_trace_all_legs.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")

    # HBM traffic per leg (per launch of the leg's timed call).
    lines = head + ["", f"plain copy of 1 GiB (__amd_rocclr_copyBuffer): FETCH_SIZE {cf_kib:.1f} KiB, "
                        f"WRITE_SIZE {cw_kib:.1f} KiB",
                    f"scale factors (true bytes / counter bytes): fetch {f_fac:.4f}, write {w_fac:.4f}",
                    "", f"{'leg':16s} {'kernel':52s} {'FETCH_KiB':>12s} {'WRITE_KiB':>12s} "
                        f"{'HBM_bytes_scaled':>16s} {'clock_GHz':>9s}"]
    traffic = {"fetch_factor": f_fac, "write_factor": w_fac,
               "source": "profiles/hbm_counters_all_legs.txt"}
    for leg, spec in LEG_KERNELS.items():
        fb = wb = 0.0
        names = []
        for pat, grid, cls in spec:
            fi = _leg_dispatches(fetch, pat, grid, cls)
            wi = _leg_dispatches(write, pat, grid, cls)
            if not fi or not wi:
                continue
            fk = _mean(fetch[d]["FETCH_SIZE"] for d in fi)
            wk = _mean(write[d]["WRITE_SIZE"] for d in wi)
            ghz = _mean(write[d]["GRBM_GUI_ACTIVE"] / 8 / write[d]["ns"] for d in wi)
            names.append(fetch[fi[0]]["name"])
            fb += fk * 1024
            wb += wk * 1024
            lines.append(f"{leg:16s} {names[-1]:52s} {fk:12.1f} {wk:12.1f} "
                         f"{fk * 1024 * f_fac + wk * 1024 * w_fac:16.4e} {ghz:9.3f}")
        if names and leg in KERNEL_SOURCES:
            traffic[leg] = {"src_sha256": sha[leg], "kernels": names, "fetch_bytes": fb,
                            "write_bytes": wb}
            lines.append(f"{leg:16s} {'(per launch of the leg)':52s} {fb / 1024:12.1f} "
                         f"{wb / 1024:12.1f} {fb * f_fac + wb * w_fac:16.4e}")
    lines.append("")
    lines.append("# clock_GHz: GRBM_GUI_ACTIVE (summed over the 8 XCDs) / 8 / the dispatch's duration;")
    lines.append("# the counter window exceeds a dispatch of a few tens of microseconds, so the")
    lines.append("# figure is only meaningful for the long kernels.")
    with open(os.path.join(outdir, "hbm_counters_all_legs.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    with open(os.path.join(outdir, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)

    # MFMA / VALU utilisation of the compute-bound kernels.
    lines = head + [
        "",
        "# per SIMD per active cycle: cycles = GRBM_GUI_ACTIVE / 8 (one XCD's busy cycles) over",
        f"# the dispatch, {N_SIMD} SIMDs.  mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x cycles);",
        "# valu_busy = 4 SQ_ACTIVE_INST_VALU / (SIMDs x cycles) (the counter ticks per quad-cycle);",
        "# coexec = SQ_VALU_MFMA_COEXEC_CYCLES / (SIMDs x cycles); wait = SQ_WAIT_INST_ANY /",
        "# SQ_WAVE_CYCLES (share of wave time stalled on a dependency); flops = 512 x",
        "# SQ_INSTS_VALU_MFMA_MOPS_BF16.  frac_at_clock = flops / (duration x SIMDs x clock x",
        "# 1024 bf16 flops per SIMD-cycle); frac_nominal = the same at 2.4 GHz (2.5 PF/s).",
        "# The clock (and every per-cycle figure) is only meaningful for dispatches longer",
        "# than some tens of microseconds.",
        "",
        f"{'leg':12s} {'kernel':44s} {'us':>8s} {'GHz':>6s} {'flops':>10s} {'algo':>10s} "
        f"{'fr_nom':>6s} {'fr_clk':>6s} {'mfma':>6s} {'valu':>6s} {'coex':>6s} {'trans%':>6s} "
        f"{'wait':>6s} {'lds_cf':>7s}"]
    for leg in ("prefill", "prefill_c2", "prefill_c3", "fwd_train", "backward", "decode",
                "memory_sequence"):
        for pat, grid, cls in LEG_KERNELS[leg]:
            i1 = _leg_dispatches(m1, pat, grid, cls)
            i2 = _leg_dispatches(m2, pat, grid, cls)
            if not i1 or not i2:
                continue
            i1 = i1[1:] if len(i1) > 1 else i1
            i2 = i2[1:] if len(i2) > 1 else i2
            us = _mean(m1[d]["ns"] for d in i1) / 1e3
            cyc1 = _mean(m1[d]["GRBM_GUI_ACTIVE"] / 8 for d in i1)
            cyc2 = _mean(m2[d]["GRBM_GUI_ACTIVE"] / 8 for d in i2)
            ghz = cyc1 / (us * 1e3)
            fl = 512.0 * _mean(m1[d]["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in i1)
            busy = _mean(m1[d]["SQ_VALU_MFMA_BUSY_CYCLES"] for d in i1) / (N_SIMD * cyc1)
            valu = 4 * _mean(m2[d]["SQ_ACTIVE_INST_VALU"] for d in i2) / (N_SIMD * cyc2)
            coex = _mean(m2[d]["SQ_VALU_MFMA_COEXEC_CYCLES"] for d in i2) / (N_SIMD * cyc2)
            trans = _mean(m1[d]["SQ_INSTS_VALU_TRANS_F32"] / max(m1[d]["SQ_INSTS_VALU"], 1)
                          for d in i1)
            wait = _mean(m2[d]["SQ_WAIT_INST_ANY"] / max(m2[d]["SQ_WAVE_CYCLES"], 1) for d in i2)
            cf = _mean(m2[d]["SQ_LDS_BANK_CONFLICT"] / max(m2[d]["SQ_LDS_IDX_ACTIVE"], 1)
                       for d in i2)
            algo = LEG_FLOPS[leg]() if leg in LEG_FLOPS and len(LEG_KERNELS[leg]) == 1 else float("nan")
            fr_nom = fl / (us * 1e-6) / 2.5e15
            fr_clk = fl / (us * 1e-6 * N_SIMD * ghz * 1e9 * 1024)
            lines.append(f"{leg:12s} {m1[i1[0]]['name'][:44]:44s} {us:8.1f} {ghz:6.3f} {fl:10.3e} "
                         f"{algo:10.3e} {fr_nom:6.3f} {fr_clk:6.3f} {busy:6.3f} {valu:6.3f} "
                         f"{coex:6.3f} {100 * trans:6.1f} {wait:6.3f} {cf:7.4f}")
    with open(os.path.join(outdir, "mfma_valu_counters_prefill_backward_memory.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote the summaries of {indir} to {outdir}")


EXTRA_LEGS = ("c2", "c3", "variants", "paged", "decode_b1", "backward", "memory_step",
              "memory_sequence")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--legs", default="all",
                    help="comma list of extra legs to run beside the headline pair: "
                         + ",".join(EXTRA_LEGS))
    ap.add_argument("--copy-probe", type=int, default=0)
    ap.add_argument("--memory-step-probe", choices=("fused", "ref"), default=None)
    ap.add_argument("--memory-sequence-probe", action="store_true")
    ap.add_argument("--counter-summary", default=None,
                    help="summarise a rocprofv3 collection directory into profiles/")
    args = ap.parse_args()
    if args.counter_summary:
        counter_summary(args.counter_summary, os.path.join(ROOT, "profiles"))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the Polar Attention path here is a single-GPU "
              "kernel library (one shard of a sharded job is one GPU at its real shape); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.memory_step_probe:
        memory_step_probe(args.memory_step_probe, args.steps)
        return
    if args.memory_sequence_probe:
        memory_sequence_probe(args.steps)
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
    legs = EXTRA_LEGS if args.legs == "all" else tuple(x for x in args.legs.split(",") if x)
    unknown = [x for x in legs if x not in EXTRA_LEGS]
    if unknown:
        print(f"unknown legs {unknown}; choose from {EXTRA_LEGS}", file=sys.stderr)
        sys.exit(2)
    cpu = not args.no_cpu_baseline
    if "variants" in legs:
        rec["variants"] = measure_variants(dev, q, k, v, pkw, pre, max(1, args.steps // 4),
                                           min(args.warmup, 2), cpu)
    if "paged" in legs:
        rec["paged"] = measure_paged(dev, pre, max(1, args.steps // 2), min(args.warmup, 2), cpu)
    del q, k, v, qd, kc, vc, table, lens, ws
    torch.cuda.empty_cache()
    for name in ("c2", "c3"):
        if name in legs:
            rec["prefill_" + name] = measure_prefill_cfg(dev, name, args.steps, args.warmup, cpu)
    torch.cuda.empty_cache()
    if "decode_b1" in legs:
        rec["decode_b1"] = measure_decode_b1(dev, args.steps, min(args.warmup, 2), cpu)
        torch.cuda.empty_cache()
    if "backward" in legs:
        rec["backward"] = measure_backward(dev, max(1, args.steps // 2), args.warmup, cpu)
    if "memory_step" in legs:
        rec["memory_step"] = measure_memory_step(dev, args.steps, args.warmup, cpu)
    if "memory_sequence" in legs:
        torch.cuda.empty_cache()
        rec["memory_sequence"] = measure_memory_sequence(dev, args.steps, args.warmup, cpu)
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

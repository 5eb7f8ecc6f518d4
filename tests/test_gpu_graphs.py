"""Library calls captured in a HIP graph (how bench.py times the short legs, and how a
caller would remove launch latency) give the eager results on every replay.

Each case captures one call, then alternates replays with eager calls of its own and with
synchronisations, and compares every replay with the eager result bit for bit (the kernels
are deterministic).  The large prefill case takes row blocks by ticket, so its replays
also check that each launch leaves its counters at zero for the next one."""
import numpy as np
import pytest
import torch

import synth
from long_context_lm_amd import (attn_bwd, attn_decode_paged, attn_fwd, attn_fwd_train,
                                 bwd_workspace_bytes, decode_workspace_bytes, delta_sequence)
from parity import to_dev

pytestmark = pytest.mark.gpu


def _capture(fn):
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


def _same(a: dict, b: dict):
    for k, v in a.items():
        if v is not None:
            assert torch.equal(v, b[k]), k


@pytest.mark.parametrize("B,T", [(2, 1000), (4, 16384)])
def test_prefill_replays(gpu_lib, B, T):
    print(f"[case] graph prefill B={B} T={T}", flush=True)
    p = synth.prefill_inputs("c3" if T > 8192 else "c2", B=B, T=T)
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    kw = dict(beta=torch.from_numpy(p.beta).cuda(), null_bias=torch.from_numpy(p.null_bias).cuda(),
              count_vec=torch.from_numpy(p.count_vec).cuda(), train_len=p.train_len, flags=p.flags)
    eager = attn_fwd(q, k, v, **kw)
    g, out = _capture(lambda: attn_fwd(q, k, v, **kw))
    for _ in range(3):
        for t in out.values():
            if t is not None:
                t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _same(eager, out)
        again = attn_fwd(q, k, v, **kw)          # eager work between the replays
        torch.cuda.synchronize()
        _same(eager, again)


def test_backward_replays(gpu_lib):
    p = synth.prefill_inputs("c2", B=2, T=300)
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    kw = dict(beta=torch.from_numpy(p.beta).cuda(), null_bias=torch.from_numpy(p.null_bias).cuda(),
              count_vec=torch.from_numpy(p.count_vec).cuda(), train_len=p.train_len, flags=p.flags)
    cot = {n: torch.from_numpy(x).cuda()
           for n, x in synth.cotangents(p.B, p.T, p.Hq, p.d).as_dict().items()}
    ws = torch.empty(bwd_workspace_bytes(p.Hq, p.Hkv, p.B, p.T), dtype=torch.uint8, device="cuda")
    fwd = attn_fwd_train(q, k, v, **kw)
    eager = attn_bwd(q, k, v, fwd, cot, workspace=ws, **kw)
    g, out = _capture(lambda: attn_bwd(q, k, v, fwd, cot, workspace=ws, **kw))
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        _same(eager, out)
        attn_fwd(q, k, v, **kw)
        torch.cuda.synchronize()


def test_variant_backward_replays(gpu_lib):
    """The window + RoPE arm's training forward and backward (rotation, windowed kernels,
    inverse rotation) captured together."""
    from long_context_lm_amd import train_variant_workspace_bytes
    p = synth.prefill_inputs("c2", B=2, T=300)
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    kw = dict(beta=torch.from_numpy(p.beta).cuda(), null_bias=torch.from_numpy(p.null_bias).cuda(),
              count_vec=torch.from_numpy(p.count_vec).cuda(), train_len=p.train_len, flags=p.flags)
    vw = dict(window=96, rope_theta=10000.0)
    cot = {n: torch.from_numpy(x).cuda()
           for n, x in synth.cotangents(p.B, p.T, p.Hq, p.d).as_dict().items()}
    wf = torch.empty(train_variant_workspace_bytes(p.Hq, p.Hkv, p.B, p.T, **vw),
                     dtype=torch.uint8, device="cuda")
    wb = torch.empty(bwd_workspace_bytes(p.Hq, p.Hkv, p.B, p.T, **vw), dtype=torch.uint8,
                     device="cuda")

    def step():
        fwd = attn_fwd_train(q, k, v, workspace=wf, **vw, **kw)
        return {**fwd, **attn_bwd(q, k, v, fwd, cot, workspace=wb, **vw, **kw)}
    eager = step()
    g, out = _capture(step)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        _same(eager, out)
        attn_fwd(q, k, v, **kw)
        torch.cuda.synchronize()


def test_readout_training_replays(gpu_lib):
    """The softmax read-out's training forward (writing u) and its backward (taking u's
    gradient) captured together."""
    p = synth.prefill_inputs("c2", B=2, T=300)
    q, k, v = (to_dev(getattr(p, n), p.dtype) for n in ("q", "k", "v"))
    kw = dict(beta=torch.from_numpy(p.beta).cuda(), null_bias=torch.from_numpy(p.null_bias).cuda(),
              count_vec=torch.from_numpy(p.count_vec).cuda(), train_len=p.train_len, flags=p.flags)
    cot = {n: torch.from_numpy(x).cuda()
           for n, x in synth.cotangents(p.B, p.T, p.Hq, p.d, attn=True).as_dict().items()}
    wb = torch.empty(bwd_workspace_bytes(p.Hq, p.Hkv, p.B, p.T), dtype=torch.uint8, device="cuda")

    def step():
        fwd = attn_fwd_train(q, k, v, want_attn=True, **kw)
        return {**fwd, **attn_bwd(q, k, v, fwd, cot, workspace=wb, **kw)}
    eager = step()
    g, out = _capture(step)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        _same(eager, out)
        attn_fwd(q, k, v, **kw)
        torch.cuda.synchronize()


def test_decode_replays(gpu_lib):
    d = synth.decode_inputs("c5", B=2, L=5000)
    qd, kc, vc = to_dev(d.q, d.dtype), to_dev(d.k_pool, d.dtype), to_dev(d.v_pool, d.dtype)
    table = torch.from_numpy(d.page_table).cuda()
    lens = torch.from_numpy(d.seq_lens).cuda()
    kw = dict(beta=torch.from_numpy(d.beta).cuda(), null_bias=torch.from_numpy(d.null_bias).cuda(),
              count_vec=torch.from_numpy(d.count_vec).cuda(), train_len=d.train_len, flags=d.flags)
    ws = torch.empty(decode_workspace_bytes(d.Hq, d.Hkv, d.B, d.max_seq_len), dtype=torch.uint8,
                     device="cuda")
    call = lambda: attn_decode_paged(qd, kc, vc, table, lens, d.max_seq_len, workspace=ws, **kw)
    eager = call()
    g, out = _capture(call)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        _same(eager, out)
        call()
        torch.cuda.synchronize()


def test_memory_stream_replays(gpu_lib):
    """The stream updates the pool in place: replays on one pool and eager calls on a copy
    walk the same sequence of states."""
    d = synth.delta_seq_inputs(B=3, T=200, H=4, num_slots=5, dtype="bf16")
    pool = torch.from_numpy(d.pool).cuda()
    sl = torch.from_numpy(d.slots).cuda()
    q, k, v = (to_dev(getattr(d, n), d.dtype) for n in ("q", "k", "v"))
    al, be = torch.from_numpy(d.alpha).cuda(), torch.from_numpy(d.beta).cuda()
    pool_e = pool.clone()
    g, out = _capture(lambda: delta_sequence(pool, sl, q, k, v, al, be))
    pool.copy_(pool_e)                           # the capture itself ran nothing
    for _ in range(3):
        g.replay()
        want = delta_sequence(pool_e, sl, q, k, v, al, be)
        torch.cuda.synchronize()
        assert torch.equal(out, want)
        assert torch.equal(pool, pool_e)

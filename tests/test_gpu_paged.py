"""GPU parity of the paged-cache write (KV append: bit-exact) and of chunked prefill over the
paged cache (float tolerances of tests/parity.py) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assert_close, host, select, to_dev
from long_context_lm_amd import attn_prefill_paged, kv_append

pytestmark = pytest.mark.gpu


def _f(a):
    return synth.bf16_bits_to_f32(a).astype(np.float64)


def _setup(ci):
    dt = ci.full.dtype
    kc, vc = to_dev(ci.k_pool, dt), to_dev(ci.v_pool, dt)
    table = torch.from_numpy(ci.page_table).cuda()
    start = torch.from_numpy(ci.start_pos).cuda()
    return kc, vc, table, start


def _append_and_run(ci):
    dt = ci.full.dtype
    kc, vc, table, start = _setup(ci)
    kv_append(to_dev(ci.chunk("k"), dt), to_dev(ci.chunk("v"), dt), kc, vc, table, start,
              ci.max_seq_len)
    p = ci.full
    out = attn_prefill_paged(to_dev(ci.chunk("q"), dt), kc, vc, table, start, ci.max_seq_len,
                             beta=p.beta, null_bias=p.null_bias, count_vec=p.count_vec,
                             train_len=p.train_len, flags=p.flags)
    torch.cuda.synchronize()
    return kc, vc, out


def _oracle(ci, kp, vp, rows=None):
    p = ci.full
    conv = _f if p.dtype == "bf16" else (lambda a: np.asarray(a, np.float64))
    q = conv(ci.chunk("q"))
    return oracle.polar_prefill_paged(q, kp, vp, ci.page_table, ci.start_pos, ci.page_size,
                                      p.beta, p.null_bias, p.count_vec, p.train_len, p.flags,
                                      to_f64=conv)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16) if t.dtype == torch.bfloat16 \
        else t.cpu().numpy()


@pytest.mark.parametrize("B,C,starts,Hq,Hkv", [
    (2, 256, (0, 700), 16, 4),       # a first chunk and a later chunk
    (2, 100, (37, 64), 8, 2),        # ragged chunk, unaligned starts
    (1, 1, (500,), 4, 1),            # one token (the decode case)
    (3, 64, (0, 1, 130), 4, 4),      # no GQA
    (2, 200, (0, 300), 8, 4),        # two heads per block (128-row blocks), split instance
])
def test_append_bit_exact_and_chunked_prefill_parity(gpu_lib, B, C, starts, Hq, Hkv):
    print(f"[case] paged B={B} C={C} starts={starts} {Hq}/{Hkv}", flush=True)
    ci = synth.chunk_inputs("c2", B=B, C=C, starts=starts, Hq=Hq, Hkv=Hkv, train_len=64)
    kc, vc, out = _append_and_run(ci)
    kp, vp = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, ci.start_pos, ci.chunk("k"),
                              ci.chunk("v"), ci.page_size, ci.max_seq_len)
    np.testing.assert_array_equal(_bits(kc), kp)
    np.testing.assert_array_equal(_bits(vc), vp)
    want = _oracle(ci, kp, vp)
    assert_close(out, want, ci.full.count_vec, "bf16", label=f"chunk C={C} starts={starts}")


def test_append_drops_tokens_on_invalid_pages(gpu_lib):
    ci = synth.chunk_inputs("c2", B=1, C=128, starts=(0,), Hq=4, Hkv=1)
    ci.page_table[0, 1] = -1                       # tokens 64..127 have nowhere to go
    kc, vc, table, start = _setup(ci)
    kv_append(to_dev(ci.chunk("k"), "bf16"), to_dev(ci.chunk("v"), "bf16"), kc, vc, table, start,
              ci.max_seq_len)
    torch.cuda.synchronize()
    kp, _ = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, ci.start_pos, ci.chunk("k"),
                             ci.chunk("v"), ci.page_size, ci.max_seq_len)
    np.testing.assert_array_equal(_bits(kc), kp)


def test_out_of_range_starts_are_clamped_alike(gpu_lib):
    """start_pos outside [0, max_seq_len - C] (here -7 and 999, with max_seq_len 264 and
    C = 64): the append kernel and the chunked prefill both clamp it, so the pools match
    the oracle's (which clamps the same way) bit for bit and the rows match its chunked
    prefill at the clamped starts."""
    print("[case] paged clamped starts", flush=True)
    ci = synth.chunk_inputs("c2", B=2, C=64, starts=(0, 200), Hq=8, Hkv=2, train_len=64)
    wild = np.array([-7, 999], np.int32)
    kc, vc, table, _ = _setup(ci)
    start = torch.from_numpy(wild).cuda()
    kv_append(to_dev(ci.chunk("k"), "bf16"), to_dev(ci.chunk("v"), "bf16"), kc, vc, table, start,
              ci.max_seq_len)
    p = ci.full
    out = attn_prefill_paged(to_dev(ci.chunk("q"), "bf16"), kc, vc, table, start, ci.max_seq_len,
                             beta=p.beta, null_bias=p.null_bias, count_vec=p.count_vec,
                             train_len=p.train_len, flags=p.flags)
    torch.cuda.synchronize()
    kp, vp = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, wild, ci.chunk("k"),
                              ci.chunk("v"), ci.page_size, ci.max_seq_len)
    np.testing.assert_array_equal(_bits(kc), kp)
    np.testing.assert_array_equal(_bits(vc), vp)
    want = oracle.polar_prefill_paged(_f(ci.chunk("q")), kp, vp, ci.page_table, wild,
                                      ci.page_size, p.beta, p.null_bias, p.count_vec,
                                      p.train_len, p.flags, to_f64=_f,
                                      max_seq_len=ci.max_seq_len)
    assert_close(out, want, p.count_vec, "bf16", label="clamped starts")


def test_chunked_prefill_float32(gpu_lib):
    ci = synth.chunk_inputs("c1", B=2, C=96, starts=(0, 150), Hq=4, Hkv=2, train_len=64)
    kc, vc, out = _append_and_run(ci)
    kp, vp = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, ci.start_pos, ci.chunk("k"),
                              ci.chunk("v"), ci.page_size, ci.max_seq_len)
    assert_close(out, _oracle(ci, kp, vp), ci.full.count_vec, "f32", label="chunk f32")


def test_last_chunk_of_64k_sequence_sampled(gpu_lib):
    """The final 4096-token chunk of the T=64K workload over a shuffled page pool."""
    print("[case] paged last chunk of C4", flush=True)
    ci = synth.chunk_inputs("c4", B=1, C=4096, starts=(61440,))
    kc, vc, out = _append_and_run(ci)
    kp, vp = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, ci.start_pos, ci.chunk("k"),
                              ci.chunk("v"), ci.page_size, ci.max_seq_len)
    rows = np.array([0, 1, 2047, 4094, 4095])
    p = ci.full
    full = oracle.polar_prefill(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.beta,
                                p.null_bias, p.count_vec, p.train_len, p.flags,
                                rows=rows + 61440)
    assert_close(select(out, rows=rows), full, p.count_vec, "bf16", label="C4 last chunk")


def test_lean_and_split_paged_chunks(gpu_lib):
    """Four 4096-token chunks (16/4 heads): 1024 workgroups choose the lean instance; a
    one-sequence launch (256 workgroups) the split instance, whose two 8-wave halves take
    the two halves of the key range and merge.  Every row of two of the chunks against the
    oracle, from both instances, and the two instances within the bf16 bound of each
    other."""
    print("[case] paged lean and split B=4 C=4096", flush=True)
    ci = synth.chunk_inputs("c2", B=4, C=4096, starts=(0, 1000, 2500, 3000))
    kc, vc, out = _append_and_run(ci)
    p = ci.full
    dt = p.dtype
    q = to_dev(ci.chunk("q"), dt)
    table = torch.from_numpy(ci.page_table).cuda()
    start = torch.from_numpy(ci.start_pos).cuda()
    kp, vp = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, ci.start_pos, ci.chunk("k"),
                              ci.chunk("v"), ci.page_size, ci.max_seq_len)
    for b in (0, 3):
        want = oracle.polar_prefill_paged(
            _f(ci.chunk("q")[b:b + 1]), kp, vp, ci.page_table[b:b + 1],
            ci.start_pos[b:b + 1], ci.page_size, p.beta, p.null_bias, p.count_vec, p.train_len,
            p.flags, to_f64=_f)
        got = {n: out[n][b:b + 1] for n in ("dir", "count", "n_eff", "gate", "lse")}
        assert_close(got, want, p.count_vec, dt, label=f"lean paged b={b}")
        one = attn_prefill_paged(q[b:b + 1], kc, vc, table[b:b + 1], start[b:b + 1],
                                 ci.max_seq_len, beta=p.beta, null_bias=p.null_bias,
                                 count_vec=p.count_vec, train_len=p.train_len, flags=p.flags)
        torch.cuda.synchronize()
        assert_close(one, want, p.count_vec, dt, label=f"split paged b={b}")
        lean_all = {n: host(out[n][b:b + 1]) for n in ("dir", "count", "n_eff", "gate", "lse")}
        assert_close(one, lean_all, p.count_vec, dt, label=f"split vs lean b={b}")


def test_lean_paged_invalid_page_ids_mask_their_keys(gpu_lib):
    """Pages of the cached prefix with ids outside [0, num_pages) (-1, and one past the
    pool) have their keys masked out, while n = pos + 1 still drives tau and the floor.
    Expected values: the oracle's row function over the sequence's keys with that page's
    64 keys removed, with lo = -64 so that the row's key count stays pos + 1.  Lean
    instance (1024 workgroups) and one-sequence launches (the split instance)."""
    print("[case] paged lean invalid page ids B=4 C=4096", flush=True)
    ci = synth.chunk_inputs("c2", B=4, C=4096, starts=(0, 1000, 2500, 3000))
    kc, vc, _ = _append_and_run(ci)
    p, dt = ci.full, ci.full.dtype
    kp, vp = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, ci.start_pos, ci.chunk("k"),
                              ci.chunk("v"), ci.page_size, ci.max_seq_len)
    num_pages = kp.shape[0]
    bad = ci.page_table.copy()
    dropped = {1: (3, -1), 3: (10, num_pages)}      # sequence: (logical page, bad id)
    for b, (pg, bid) in dropped.items():
        assert (pg + 1) * 64 <= ci.start_pos[b]      # a page of the prefix
        bad[b, pg] = bid
    q = to_dev(ci.chunk("q"), dt)
    table = torch.from_numpy(bad).cuda()
    start = torch.from_numpy(ci.start_pos).cuda()
    kw = dict(beta=p.beta, null_bias=p.null_bias, count_vec=p.count_vec, train_len=p.train_len,
              flags=p.flags)
    out = attn_prefill_paged(q, kc, vc, table, start, ci.max_seq_len, **kw)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 63, 64, 2000, 4095])
    G = p.Hq // p.Hkv
    qf = _f(ci.chunk("q"))
    for b, (pg, _) in dropped.items():
        L = int(ci.start_pos[b]) + ci.C
        pos = int(ci.start_pos[b]) + rows
        keep = np.ones(L, bool)
        keep[pg * 64:(pg + 1) * 64] = False
        want = {k: np.zeros((1, len(rows), p.Hq) + ((64,) if k in ("dir", "count") else ()))
                for k in ("dir", "count", "n_eff", "gate", "lse")}
        for g in range(p.Hkv):
            K = _f(oracle.gather_pages(kp, ci.page_table[b], g, L, ci.page_size))[keep]
            V = _f(oracle.gather_pages(vp, ci.page_table[b], g, L, ci.page_size))[keep]
            for h in range(g * G, (g + 1) * G):
                res = oracle.polar_oracle._polar_rows(qf[b, rows, h], K, V, pos + 1 - 64, p.beta[h],
                                         p.null_bias[h], p.count_vec[h], p.train_len, p.flags,
                                         lo=np.full(len(rows), -64))
                for k in want:
                    want[k][0, :, h] = res[k]
        got = {n: out[n][b:b + 1, rows] for n in want}
        assert_close(got, want, p.count_vec, dt, label=f"invalid page b={b}")
        one = attn_prefill_paged(q[b:b + 1], kc, vc, table[b:b + 1], start[b:b + 1],
                                 ci.max_seq_len, **kw)
        torch.cuda.synchronize()
        got1 = {n: one[n][:, rows] for n in want}
        assert_close(got1, want, p.count_vec, dt, label=f"invalid page split b={b}")

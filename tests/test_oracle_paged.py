"""Pins of the chunked-prefill and KV-append oracles.

* after appending the chunk, chunked prefill rows equal the contiguous causal prefill rows
  start..start+C-1 of the same sequence (the page indirection and the prefix split change
  nothing);
* a chunk of one token equals paged decode of that sequence;
* appending into pages and gathering back returns the contiguous keys and values exactly;
  dropped tokens (invalid pages) leave the pool unchanged;
* a start outside [0, max_seq_len - C] behaves exactly like the nearest start inside it, in
  the append and in the chunked prefill alike.
"""
import numpy as np

import oracle
import synth


def _f(a):
    return synth.bf16_bits_to_f32(a).astype(np.float64)


def test_chunked_prefill_equals_contiguous_rows():
    ci = synth.chunk_inputs("c2", B=2, C=40, starts=(0, 77), Hq=8, Hkv=2, train_len=16)
    kp, vp = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, ci.start_pos,
                              ci.chunk("k"), ci.chunk("v"), ci.page_size, ci.max_seq_len)
    p = ci.full
    got = oracle.polar_prefill_paged(_f(ci.chunk("q")), kp, vp, ci.page_table, ci.start_pos,
                                     ci.page_size, p.beta, p.null_bias, p.count_vec,
                                     p.train_len, p.flags, to_f64=_f)
    full = oracle.polar_prefill(p.as_f32("q"), p.as_f32("k"), p.as_f32("v"), p.beta,
                                p.null_bias, p.count_vec, p.train_len, p.flags)
    for b, s in enumerate(ci.start_pos):
        for n in ("dir", "count", "n_eff", "gate", "lse"):
            np.testing.assert_allclose(got[n][b], full[n][b, s:s + ci.C], rtol=1e-12, atol=1e-12)


def test_one_token_chunk_equals_decode():
    ci = synth.chunk_inputs("c2", B=2, C=1, starts=(130, 5), Hq=4, Hkv=1, train_len=16)
    kp, vp = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, ci.start_pos,
                              ci.chunk("k"), ci.chunk("v"), ci.page_size, ci.max_seq_len)
    p = ci.full
    got = oracle.polar_prefill_paged(_f(ci.chunk("q")), kp, vp, ci.page_table, ci.start_pos,
                                     ci.page_size, p.beta, p.null_bias, p.count_vec,
                                     p.train_len, p.flags, to_f64=_f)
    dec = oracle.polar_decode_paged(_f(ci.chunk("q"))[:, 0], kp, vp, ci.page_table,
                                    ci.start_pos + 1, ci.page_size, p.beta, p.null_bias,
                                    p.count_vec, p.train_len, p.flags, to_f64=_f)
    for n in ("dir", "count", "n_eff", "gate", "lse"):
        np.testing.assert_allclose(got[n][:, 0], dec[n], rtol=1e-13, atol=1e-13)


def test_append_then_gather_round_trips():
    ci = synth.chunk_inputs("c2", B=2, C=70, starts=(10, 200), Hq=4, Hkv=2)
    kp, vp = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, ci.start_pos,
                              ci.chunk("k"), ci.chunk("v"), ci.page_size, ci.max_seq_len)
    for b, s in enumerate(ci.start_pos):
        L = int(s) + ci.C
        for g in range(2):
            np.testing.assert_array_equal(
                oracle.gather_pages(kp, ci.page_table[b], g, L, ci.page_size), ci.full.k[b, :L, g])
            np.testing.assert_array_equal(
                oracle.gather_pages(vp, ci.page_table[b], g, L, ci.page_size), ci.full.v[b, :L, g])


def test_append_drops_out_of_range_tokens():
    ci = synth.chunk_inputs("c2", B=1, C=64, starts=(0,), Hq=4, Hkv=1)
    table = ci.page_table.copy()
    table[0, 0] = -1                                       # invalid page: tokens dropped
    kp, vp = oracle.kv_append(ci.k_pool, ci.v_pool, table, ci.start_pos, ci.chunk("k"),
                              ci.chunk("v"), ci.page_size, ci.max_seq_len)
    np.testing.assert_array_equal(kp, ci.k_pool)


def test_chunk_start_clamp_closed_form():
    np.testing.assert_array_equal(oracle.chunk_start([-3, 0, 5, 90, 91, 999], 10, 100),
                                  [0, 0, 5, 90, 90, 90])
    np.testing.assert_array_equal(oracle.chunk_start([-3, 999], 10, None), [-3, 999])


def test_out_of_range_starts_act_like_the_clamped_start():
    """Appending and attending with starts (-7, 999) over max_seq_len = 264, C = 64 is the
    same as with the clamped starts (0, 200): the same pool and the same rows."""
    ci = synth.chunk_inputs("c2", B=2, C=64, starts=(0, 200), Hq=4, Hkv=2, train_len=16)
    assert ci.max_seq_len == 264
    wild = np.array([-7, 999], np.int32)
    args = (ci.chunk("k"), ci.chunk("v"), ci.page_size, ci.max_seq_len)
    kp, vp = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, ci.start_pos, *args)
    kw, vw = oracle.kv_append(ci.k_pool, ci.v_pool, ci.page_table, wild, *args)
    np.testing.assert_array_equal(kw, kp)
    np.testing.assert_array_equal(vw, vp)
    p = ci.full
    common = (ci.page_size, p.beta, p.null_bias, p.count_vec, p.train_len, p.flags)
    want = oracle.polar_prefill_paged(_f(ci.chunk("q")), kp, vp, ci.page_table, ci.start_pos,
                                      *common, to_f64=_f)
    got = oracle.polar_prefill_paged(_f(ci.chunk("q")), kp, vp, ci.page_table, wild, *common,
                                     to_f64=_f, max_seq_len=ci.max_seq_len)
    for n in ("dir", "count", "n_eff", "gate", "lse"):
        np.testing.assert_array_equal(got[n], want[n])

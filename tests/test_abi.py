"""libpolar loads, exports every symbol include/polar.h declares, and validates its
arguments on the host before any HIP call (no GPU needed: no call here launches)."""
import ctypes
import os
import re

import pytest

from long_context_lm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 0x10000            # a 16-byte aligned fake device address (never dereferenced)


def declared_symbols():
    src = open(os.path.join(ROOT, "include", "polar.h")).read()
    return sorted(set(re.findall(r"POLAR_API\s+[\w\s\*]+?\b(polar_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = declared_symbols()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert _lib.polar_abi_version() == 7 == _lib.ABI_VERSION


def test_status_strings():
    for code in range(7):
        assert _lib.polar_status_str(code) not in ("", "unknown status")
    assert _lib.polar_status_str(99) == "unknown status"


def params(**kw):
    d = dict(n_q_heads=16, n_kv_heads=4, head_dim=64, train_len=2048, flags=3, beta=None,
             null_bias=None, count_vec=A)
    d.update(kw)
    return _lib.polar_params(d["n_q_heads"], d["n_kv_heads"], d["head_dim"], d["train_len"],
                             d["flags"], d["beta"], d["null_bias"], d["count_vec"])


def outs(**kw):
    d = dict(dir=A, count=A, n_eff=A, gate=A, lse=A)
    d.update(kw)
    return _lib.polar_outputs(d["dir"], d["count"], d["n_eff"], d["gate"], d["lse"])


def fwd(p=None, dt=1, B=1, T=8, q=A, k=A, v=A, o=None):
    p = params() if p is None else p
    o = outs() if o is None else o
    return _lib.polar_attn_fwd(p, dt, B, T, q, k, v, o, None)


@pytest.mark.parametrize("kw,code", [
    (dict(p=params(head_dim=128)), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(dt=7), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(p=params(n_q_heads=6, n_kv_heads=4)), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(p=params(n_kv_heads=0)), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(p=params(train_len=1)), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(p=params(flags=4)), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(B=-1), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(T=-5), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(q=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(o=outs(dir=None)), _lib.POLAR_ERR_NULL_POINTER),
    (dict(o=outs(n_eff=None)), _lib.POLAR_ERR_NULL_POINTER),
    (dict(p=params(count_vec=None)), _lib.POLAR_ERR_NULL_POINTER),
    (dict(k=A + 4), _lib.POLAR_ERR_MISALIGNED),
    (dict(o=outs(dir=A + 8)), _lib.POLAR_ERR_MISALIGNED),
])
def test_prefill_validation_errors(kw, code):
    assert fwd(**kw) == code
    assert _lib.polar_last_error() != ""


def test_prefill_null_params_and_outputs():
    lib = _lib.load()
    assert lib.polar_attn_fwd(None, 1, 1, 8, A, A, A, ctypes.byref(outs()), None) == \
        _lib.POLAR_ERR_NULL_POINTER
    assert lib.polar_attn_fwd(ctypes.byref(params()), 1, 1, 8, A, A, A, None, None) == \
        _lib.POLAR_ERR_NULL_POINTER


def test_empty_prefill_is_a_valid_no_op():
    # nothing is launched for B == 0 or T == 0, so no GPU is touched
    assert fwd(B=0) == _lib.POLAR_OK
    assert fwd(T=0) == _lib.POLAR_OK
    assert fwd(p=params(count_vec=None), o=outs(count=None, gate=None, lse=None), T=0) == \
        _lib.POLAR_OK
    # empty tensors may come as NULL pointers
    assert fwd(B=0, q=None, k=None, v=None, o=outs(dir=None, n_eff=None)) == _lib.POLAR_OK


def mixed(p=None, dt=1, B=1, T=8, q=A, k=A, v=A, mem=A, mx=A, o=None):
    p = params() if p is None else p
    o = outs(dir=None, count=None) if o is None else o
    return _lib.polar_attn_fwd_mixed(p, dt, B, T, q, k, v, mem, mx, o, None)


@pytest.mark.parametrize("kw,code", [
    (dict(o=outs()), _lib.POLAR_ERR_UNSUPPORTED),                  # dir and count set
    (dict(o=outs(dir=None)), _lib.POLAR_ERR_UNSUPPORTED),          # count set
    (dict(mx=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(mx=A + 8), _lib.POLAR_ERR_MISALIGNED),
    (dict(mem=A + 4), _lib.POLAR_ERR_MISALIGNED),
    (dict(p=params(count_vec=A + 4)), _lib.POLAR_ERR_MISALIGNED),
    (dict(o=outs(dir=None, count=None, n_eff=None)), _lib.POLAR_ERR_NULL_POINTER),
    (dict(dt=7), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(p=params(n_q_heads=6, n_kv_heads=4)), _lib.POLAR_ERR_BAD_SHAPE),
])
def test_mixed_validation_errors(kw, code):
    assert mixed(**kw) == code
    assert _lib.polar_last_error() != ""


def test_mixed_empty_and_optional_memory():
    assert mixed(B=0, q=None, k=None, v=None, mem=None, mx=None) == _lib.POLAR_OK
    assert mixed(T=0, q=None, k=None, v=None, mem=None, mx=None) == _lib.POLAR_OK
    assert _lib.load().polar_attn_fwd_mixed(params(), 1, 1, 8, A, A, A, A, A, None, None) == \
        _lib.POLAR_ERR_NULL_POINTER


def dec(p=None, dt=1, B=2, q=A, kc=A, vc=A, num_pages=10, page=64, table=A, stride=4,
        lens=A, max_len=256, ws=A, ws_bytes=None, o=None):
    p = params() if p is None else p
    o = outs() if o is None else o
    if ws_bytes is None:
        ws_bytes = _lib.polar_decode_workspace_bytes(p, B, max(max_len, 1))
    return _lib.polar_attn_decode_paged(p, dt, B, q, kc, vc, num_pages, page, table, stride,
                                        lens, max_len, ws, ws_bytes, o, None)


def test_workspace_bytes():
    p = params()
    n = _lib.polar_decode_workspace_bytes(p, 16, 262144)
    assert n > 0 and n % 16 == 0
    assert _lib.polar_decode_workspace_bytes(p, 16, 0) == 0
    assert _lib.polar_decode_workspace_bytes(params(n_q_heads=5), 16, 100) == 0
    assert _lib.polar_decode_workspace_bytes(p, 0, 100) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(page=32), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(p=params(head_dim=32)), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(B=-1), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(num_pages=0), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(max_len=0, ws_bytes=1 << 20), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(stride=3), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(table=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(lens=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(ws=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(kc=A + 2), _lib.POLAR_ERR_MISALIGNED),
    (dict(ws=A + 4), _lib.POLAR_ERR_MISALIGNED),
    (dict(ws_bytes=15), _lib.POLAR_ERR_WORKSPACE_TOO_SMALL),
])
def test_decode_validation_errors(kw, code):
    assert dec(**kw) == code
    assert _lib.polar_last_error() != ""


def test_empty_decode_is_a_valid_no_op():
    assert dec(B=0, ws_bytes=0) == _lib.POLAR_OK
    assert dec(B=0, ws_bytes=0, q=None, table=None, lens=None, ws=None,
               o=outs(dir=None, n_eff=None)) == _lib.POLAR_OK


# ------------------------------------------------------------------ training entry points
WS = 0x100000          # 256-byte aligned fake workspace address


def saved(**kw):
    d = dict(u_norm=A, arg_max=A)
    d.update(kw)
    return _lib.polar_saved(d["u_norm"], d["arg_max"])


def cots(**kw):
    d = dict(dir=A, count=A, n_eff=A, gate=A, lse=A, attn=A)
    d.update(kw)
    return _lib.polar_cotangents(d["dir"], d["count"], d["n_eff"], d["gate"], d["lse"],
                                 d["attn"])


def grads(**kw):
    d = dict(dq=A, dk=A, dv=A, d_beta=None, d_null_bias=None, d_count_vec=None)
    d.update(kw)
    return _lib.polar_grads(d["dq"], d["dk"], d["dv"], d["d_beta"], d["d_null_bias"],
                            d["d_count_vec"])


def bwd(p=None, dt=1, B=1, T=100, q=A, k=A, v=A, o=None, s=None, c=None, g=None, ws=WS,
        ws_bytes=None):
    p = params() if p is None else p
    if ws_bytes is None:
        ws_bytes = _lib.polar_bwd_workspace_bytes(p, max(B, 1), max(T, 1))
    return _lib.polar_attn_bwd(p, dt, B, T, q, k, v, outs() if o is None else o,
                               saved() if s is None else s, cots() if c is None else c,
                               grads() if g is None else g, ws, ws_bytes, None)


def test_bwd_workspace_bytes():
    p = params()
    n = _lib.polar_bwd_workspace_bytes(p, 8, 2048)
    assert n >= 8 * 2048 * 16 * (64 * 2 + 3 * 16) and n % 256 == 0   # du, row records
    assert _lib.polar_bwd_workspace_bytes(p, 0, 2048) == 0
    assert _lib.polar_bwd_workspace_bytes(p, 8, 0) == 0
    assert _lib.polar_bwd_workspace_bytes(params(n_q_heads=6), 8, 64) == 0
    assert _lib.polar_bwd_workspace_bytes(p, 1, 1 << 30) == 0       # 32-bit offsets


@pytest.mark.parametrize("kw,code", [
    (dict(dt=0), _lib.POLAR_ERR_UNSUPPORTED),                        # bf16 only
    (dict(p=params(head_dim=128)), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(T=-1), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(g=grads(dq=None)), _lib.POLAR_ERR_NULL_POINTER),
    (dict(g=grads(dv=None)), _lib.POLAR_ERR_NULL_POINTER),
    (dict(s=saved(arg_max=None)), _lib.POLAR_ERR_NULL_POINTER),
    (dict(o=outs(lse=None)), _lib.POLAR_ERR_NULL_POINTER),
    (dict(o=outs(gate=None)), _lib.POLAR_ERR_NULL_POINTER),
    (dict(p=params(count_vec=None), o=outs(count=None)), _lib.POLAR_ERR_NULL_POINTER),
    (dict(ws=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(ws=WS + 16), _lib.POLAR_ERR_MISALIGNED),
    (dict(g=grads(dk=A + 4)), _lib.POLAR_ERR_MISALIGNED),
    (dict(c=cots(dir=A + 8)), _lib.POLAR_ERR_MISALIGNED),
    (dict(c=cots(attn=A + 4)), _lib.POLAR_ERR_MISALIGNED),
    (dict(ws_bytes=1024), _lib.POLAR_ERR_WORKSPACE_TOO_SMALL),
])
def test_bwd_validation_errors(kw, code):
    assert bwd(**kw) == code
    assert _lib.polar_last_error() != ""


def test_bwd_null_structs():
    lib = _lib.load()
    p = params()
    n = _lib.polar_bwd_workspace_bytes(p, 1, 100)
    assert lib.polar_attn_bwd(ctypes.byref(p), 1, 1, 100, A, A, A, ctypes.byref(outs()), None,
                              ctypes.byref(cots()), ctypes.byref(grads()), WS, n, None) == \
        _lib.POLAR_ERR_NULL_POINTER


def test_empty_bwd_without_parameter_grads_is_a_no_op():
    assert bwd(B=0, q=None, k=None, v=None, ws=None, ws_bytes=0) == _lib.POLAR_OK
    assert bwd(T=0, g=grads(dq=None, dk=None, dv=None), ws=None, ws_bytes=0) == _lib.POLAR_OK


def test_fwd_train_validation():
    lib = _lib.load()
    p = params()
    assert lib.polar_attn_fwd_train(ctypes.byref(p), 1, 1, 8, A, A, A, ctypes.byref(outs()),
                                    None, None) == _lib.POLAR_ERR_NULL_POINTER
    assert _lib.polar_attn_fwd_train(p, 1, 1, 8, A, A, A, outs(), saved(u_norm=None),
                                     None) == _lib.POLAR_ERR_NULL_POINTER
    assert _lib.polar_attn_fwd_train(p, 1, 1, 8, A, A, A, outs(gate=None), saved(),
                                     None) == _lib.POLAR_ERR_NULL_POINTER
    assert _lib.polar_attn_fwd_train(p, 1, 0, 8, A, A, A, outs(), saved(), None) == _lib.POLAR_OK


# ------------------------------------------------------------------ variant modes
def var_fwd(window=0, theta=0.0, attn=None, ws=None, ws_bytes=0, dt=1, **kw):
    return _lib.polar_attn_fwd_variant(params(),
                                       _lib.polar_variant(window, theta, attn, ws, ws_bytes),
                                       dt, kw.get("B", 1), kw.get("T", 8), A, A, A, outs(), None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=-1), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(theta=-2.0), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(theta=0.5), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(theta=float("inf")), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(theta=float("nan")), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(attn=A + 4), _lib.POLAR_ERR_MISALIGNED),
    (dict(theta=10000.0, ws=A + 8, ws_bytes=1 << 20), _lib.POLAR_ERR_MISALIGNED),
    # 1 x 8 keys x 4 KV heads x 64 dims x 2 bytes = 4096 bytes needed (8192 for fp32)
    (dict(theta=10000.0, ws=A, ws_bytes=4095), _lib.POLAR_ERR_WORKSPACE_TOO_SMALL),
    (dict(theta=10000.0, ws=A, ws_bytes=8191, dt=0), _lib.POLAR_ERR_WORKSPACE_TOO_SMALL),
])
def test_variant_validation_errors(kw, code):
    assert var_fwd(**kw) == code
    assert _lib.polar_last_error() != ""


def test_variant_workspace_bytes():
    # B * T * Hkv * d * element size; the workspace is only read with rope_theta > 0
    assert _lib.polar_variant_workspace_bytes(params(), 1, 3, 100) == 3 * 100 * 4 * 64 * 2
    assert _lib.polar_variant_workspace_bytes(params(), 0, 3, 100) == 3 * 100 * 4 * 64 * 4
    assert _lib.polar_variant_workspace_bytes(params(), 1, 0, 100) == 0
    assert _lib.polar_variant_workspace_bytes(params(), 7, 3, 100) == 0
    assert _lib.load().polar_variant_workspace_bytes(None, 1, 3, 100) == 0


def test_variant_empty_calls():
    assert var_fwd(window=16, theta=10000.0, attn=A, B=0) == _lib.POLAR_OK
    assert _lib.polar_attn_fwd_variant(params(), None, 1, 1, 0, A, A, A, outs(), None) == \
        _lib.POLAR_OK


# ------------------------------------------------------------------ variant training + backward
def train_var(window=0, theta=0.0, attn=None, ws=None, ws_bytes=0, dt=1, B=1, T=8, s=None,
              o=None, q=A):
    return _lib.polar_attn_fwd_train_variant(params(),
                                             _lib.polar_variant(window, theta, attn, ws,
                                                                ws_bytes),
                                             dt, B, T, q, A, A, outs() if o is None else o,
                                             saved() if s is None else s, None)


@pytest.mark.parametrize("kw,code", [
    (dict(window=-3), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(theta=0.9), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(attn=A + 4), _lib.POLAR_ERR_MISALIGNED),          # the read-out, misaligned
    (dict(theta=10000.0, ws=A, ws_bytes=1 << 20, attn=A + 8), _lib.POLAR_ERR_MISALIGNED),
    (dict(window=4, o=outs(lse=None)), _lib.POLAR_ERR_NULL_POINTER),
    (dict(theta=10000.0), _lib.POLAR_ERR_NULL_POINTER),     # RoPE needs the workspace
    (dict(theta=10000.0, ws=A + 8, ws_bytes=1 << 20), _lib.POLAR_ERR_MISALIGNED),
    # q and k rotated: 1 x 8 x (16 + 4) x 64 x 2 bytes = 20480
    (dict(theta=10000.0, ws=A, ws_bytes=20479), _lib.POLAR_ERR_WORKSPACE_TOO_SMALL),
    (dict(theta=10000.0, ws=A, ws_bytes=1 << 20, q=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(theta=10000.0, ws=A, ws_bytes=1 << 20, dt=9), _lib.POLAR_ERR_UNSUPPORTED),
])
def test_train_variant_validation_errors(kw, code):
    assert train_var(**kw) == code
    assert _lib.polar_last_error() != ""


def test_train_variant_null_saved_and_empty():
    assert _lib.load().polar_attn_fwd_train_variant(
        ctypes.byref(params()), None, 1, 1, 8, A, A, A, ctypes.byref(outs()), None, None) == \
        _lib.POLAR_ERR_NULL_POINTER
    assert train_var(window=4, theta=10000.0, B=0) == _lib.POLAR_OK
    assert train_var(attn=A, T=0) == _lib.POLAR_OK          # the read-out, empty call


def test_train_variant_workspace_bytes():
    var = lambda w, t: _lib.polar_variant(w, t, None, None, 0)
    f = _lib.polar_train_variant_workspace_bytes
    assert f(params(), var(0, 10000.0), 1, 2, 100) == 2 * 100 * 20 * 64 * 2
    assert f(params(), var(16, 10000.0), 0, 2, 100) == 2 * 100 * 20 * 64 * 4
    assert f(params(), var(16, 0.0), 1, 2, 100) == 0          # no rotation, no workspace
    assert f(params(), var(-1, 10000.0), 1, 2, 100) == 0
    assert f(params(), var(0, 10000.0), 4, 2, 100) == 0


def test_bwd_variant_workspace_bytes():
    var = lambda w, t: _lib.polar_variant(w, t, None, None, 0)
    f = _lib.polar_bwd_variant_workspace_bytes
    base = _lib.polar_bwd_workspace_bytes(params(), 2, 300)
    assert f(params(), var(64, 0.0), 2, 300) == base
    assert f(params(), None, 2, 300) == base
    rot = f(params(), var(0, 500.0), 2, 300)
    q_bytes, k_bytes = 2 * 300 * 16 * 64 * 2, 2 * 300 * 4 * 64 * 2
    assert rot >= base + q_bytes + k_bytes and rot <= base + q_bytes + k_bytes + 512
    assert f(params(), var(0, 0.5), 2, 300) == 0
    assert f(params(), var(0, 500.0), 0, 300) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(var=_lib.polar_variant(-1, 0.0, None, None, 0)), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(var=_lib.polar_variant(0, 1.0, None, None, 0)), _lib.POLAR_ERR_BAD_SHAPE),
    # the read-out's gradient comes in cot.attn, never var.attn
    (dict(var=_lib.polar_variant(8, 0.0, A, None, 0)), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(var=_lib.polar_variant(0, 500.0, None, None, 0), dt=0), _lib.POLAR_ERR_UNSUPPORTED),
    # the base workspace is not enough once q and k are rotated into it
    (dict(var=_lib.polar_variant(0, 500.0, None, None, 0), base_ws=True),
     _lib.POLAR_ERR_WORKSPACE_TOO_SMALL),
    (dict(var=_lib.polar_variant(16, 500.0, None, None, 0), g=grads(dq=None)),
     _lib.POLAR_ERR_NULL_POINTER),
])
def test_bwd_variant_validation_errors(kw, code):
    var = kw["var"]
    p = params()
    n = (_lib.polar_bwd_workspace_bytes(p, 1, 100) if kw.get("base_ws")
         else _lib.polar_bwd_variant_workspace_bytes(p, var, 1, 100))
    assert _lib.polar_attn_bwd_variant(p, var, kw.get("dt", 1), 1, 100, A, A, A, outs(),
                                       saved(), cots(), kw.get("g", grads()), WS, n,
                                       None) == code
    assert _lib.polar_last_error() != ""


# ------------------------------------------------------------------ paged append / chunks
def app(p=None, dt=1, B=2, C=16, kn=A, vn=A, kc=A, vc=A, num_pages=10, page=64, table=A,
        stride=4, start=A, max_len=256):
    return _lib.polar_kv_append(params() if p is None else p, dt, B, C, kn, vn, kc, vc,
                                num_pages, page, table, stride, start, max_len, None)


@pytest.mark.parametrize("kw,code", [
    (dict(page=32), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(dt=5), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(p=params(head_dim=32)), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(C=-1), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(num_pages=0), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(max_len=8), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(stride=3), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(table=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(start=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(kc=A + 8), _lib.POLAR_ERR_MISALIGNED),
])
def test_append_validation_errors(kw, code):
    assert app(**kw) == code
    assert _lib.polar_last_error() != ""


def chunk(p=None, dt=1, B=2, C=16, q=A, kc=A, vc=A, num_pages=10, page=64, table=A, stride=4,
          start=A, max_len=256, o=None):
    return _lib.polar_attn_prefill_paged(params() if p is None else p, dt, B, C, q, kc, vc,
                                         num_pages, page, table, stride, start, max_len,
                                         outs() if o is None else o, None)


@pytest.mark.parametrize("kw,code", [
    (dict(page=16), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(p=params(n_q_heads=5)), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(C=-2), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(max_len=4), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(stride=2), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(start=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(q=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(o=outs(dir=None)), _lib.POLAR_ERR_NULL_POINTER),
    (dict(kc=A + 2), _lib.POLAR_ERR_MISALIGNED),
])
def test_chunked_prefill_validation_errors(kw, code):
    assert chunk(**kw) == code
    assert _lib.polar_last_error() != ""


def test_empty_append_and_chunk():
    assert app(C=0, kn=None, vn=None) == _lib.POLAR_OK
    assert chunk(B=0, q=None) == _lib.POLAR_OK


# ------------------------------------------------------------------ gated-delta memory step
def dstep(H=4, dk=64, dv=64, flags=1, dt=1, B=3, pool=A, num_slots=8, slots=A, q=A, k=A, v=A,
          al=A, be=A, out=A):
    prm = _lib.polar_delta_params(H, dk, dv, flags)
    return _lib.polar_delta_step(prm, dt, B, pool, num_slots, slots, q, k, v, al, be, out, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dk=32), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(dv=128), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(flags=2), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(dt=3), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(H=0), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(B=-1), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(num_slots=0), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(slots=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(be=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(pool=A + 4), _lib.POLAR_ERR_MISALIGNED),
    (dict(out=A + 8), _lib.POLAR_ERR_MISALIGNED),
])
def test_delta_step_validation_errors(kw, code):
    assert dstep(**kw) == code
    assert _lib.polar_last_error() != ""


def test_delta_step_empty_and_null_params():
    assert dstep(B=0, pool=None, slots=None, q=None) == _lib.POLAR_OK
    lib = _lib.load()
    assert lib.polar_delta_step(None, 1, 1, A, 1, A, A, A, A, A, A, A, None) == \
        _lib.POLAR_ERR_NULL_POINTER


def dseq(H=4, dk=64, dv=64, flags=1, dt=1, B=3, T=100, pool=A, num_slots=8, slots=A, q=A, k=A,
         v=A, al=A, be=A, out=A):
    prm = _lib.polar_delta_params(H, dk, dv, flags)
    return _lib.polar_delta_sequence(prm, dt, B, T, pool, num_slots, slots, q, k, v, al, be, out,
                                     None)


@pytest.mark.parametrize("kw,code", [
    (dict(dk=32), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(dv=128), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(flags=2), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(dt=3), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(H=0), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(B=-1), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(T=-1), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(num_slots=0), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(B=1 << 30, H=4), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(slots=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(k=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(al=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(pool=A + 4), _lib.POLAR_ERR_MISALIGNED),
    (dict(v=A + 8), _lib.POLAR_ERR_MISALIGNED),
    (dict(out=A + 8), _lib.POLAR_ERR_MISALIGNED),
])
def test_delta_sequence_validation_errors(kw, code):
    assert dseq(**kw) == code
    assert _lib.polar_last_error() != ""


def test_delta_sequence_empty_and_null_params():
    assert dseq(B=0, pool=None, slots=None, q=None) == _lib.POLAR_OK
    assert dseq(T=0, pool=None, slots=None, q=None) == _lib.POLAR_OK
    lib = _lib.load()
    assert lib.polar_delta_sequence(None, 1, 1, 1, A, 1, A, A, A, A, A, A, A, None) == \
        _lib.POLAR_ERR_NULL_POINTER


def dec_noalloc(p=None, dt=1, B=2, q=A, kc=A, vc=A, num_pages=10, page=64, table=A, stride=4,
                lens=A, max_len=256, o=None):
    p = params() if p is None else p
    o = outs() if o is None else o
    return _lib.polar_attn_decode_paged_noalloc(p, dt, B, q, kc, vc, num_pages, page, table,
                                                stride, lens, max_len, o, None)


@pytest.mark.parametrize("kw,code", [
    (dict(page=32), _lib.POLAR_ERR_UNSUPPORTED),
    (dict(B=-1), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(q=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(table=None), _lib.POLAR_ERR_NULL_POINTER),
    (dict(stride=3), _lib.POLAR_ERR_BAD_SHAPE),
    (dict(kc=A + 8), _lib.POLAR_ERR_MISALIGNED),
    # 4096 sequences of 256K keys need 17.8 MB of split partials: more than the scratch
    (dict(B=4096, max_len=262144, stride=4096, num_pages=1 << 20), _lib.POLAR_ERR_WORKSPACE_TOO_SMALL),
])
def test_noalloc_decode_validation(kw, code):
    """The allocation-free decode validates like the workspace one, and refuses a decode
    whose partials exceed its static scratch, all before any HIP call."""
    assert dec_noalloc(**kw) == code
    if code == _lib.POLAR_ERR_WORKSPACE_TOO_SMALL:
        assert "static scratch" in _lib.polar_last_error()
        p = params()
        assert _lib.polar_decode_workspace_bytes(p, 4096, 262144) > _lib.POLAR_NOALLOC_SCRATCH_BYTES


def test_noalloc_decode_empty_batch_launches_nothing():
    assert dec_noalloc(B=0, q=None, kc=None, vc=None, table=None, lens=None) == _lib.POLAR_OK

"""torch-facing wrappers over libpolar: allocate outputs, pass pointers and the stream.

Nothing here computes: shapes are read, buffers allocated with torch, and the C entry
points of include/polar.h are called on torch's current HIP stream.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import _lib

_DT = {torch.bfloat16: _lib.POLAR_DTYPE_BF16, torch.float32: _lib.POLAR_DTYPE_F32}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _params(Hq, Hkv, d, beta, null_bias, count_vec, train_len, flags):
    return _lib.polar_params(Hq, Hkv, d, train_len, flags, _ptr(beta), _ptr(null_bias),
                             _ptr(count_vec))


def _device_f32(x, device, numel=None, name="parameter"):
    """A per-head parameter as a contiguous float32 tensor on ``device`` (copied there if
    needed), holding exactly ``numel`` values: the kernels index it by head."""
    if x is None:
        return None
    t = torch.as_tensor(x, dtype=torch.float32, device=device).contiguous()
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} values (got {t.numel()})")
    return t


def _head_params(beta, null_bias, count_vec, Hq, d, dev):
    return (_device_f32(beta, dev, Hq, "beta"), _device_f32(null_bias, dev, Hq, "null_bias"),
            _device_f32(count_vec, dev, Hq * d, "count_vec"))


def _check_input(t: torch.Tensor, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in _DT:
        raise ValueError(f"{name} has dtype {t.dtype}; bfloat16 or float32 expected")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_aux(t, name: str, device, dtype, shape=None) -> None:
    """A tensor the kernels read or write beside q, k and v (tables, positions, slots, saved
    residuals, workspaces): it must sit on the inputs' GPU, since the library takes a bare
    device pointer, and be contiguous, since the only row strides the C calls know are the
    ones their arguments state."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.device != torch.device(device):
        raise ValueError(f"{name} must be on {device} (got {t.device})")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def _outputs(lead, Hq, d, device, want_count, want_gate, want_lse):
    o = dict(dir=torch.empty(*lead, Hq, d, device=device, dtype=torch.float32),
             n_eff=torch.empty(*lead, Hq, device=device, dtype=torch.float32))
    o["count"] = (torch.empty(*lead, Hq, d, device=device, dtype=torch.float32)
                  if want_count else None)
    o["gate"] = torch.empty(*lead, Hq, device=device, dtype=torch.float32) if want_gate else None
    o["lse"] = torch.empty(*lead, Hq, device=device, dtype=torch.float32) if want_lse else None
    c = _lib.polar_outputs(_ptr(o["dir"]), _ptr(o["count"]), _ptr(o["n_eff"]), _ptr(o["gate"]),
                           _ptr(o["lse"]))
    return o, c


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta=None, null_bias=None,
             count_vec=None, train_len: int = 2048,
             flags: int = _lib.POLAR_FLAG_LENGTH_TEMP | _lib.POLAR_FLAG_NULL_FLOOR,
             want_gate: bool = True, want_lse: bool = True, stream=None) -> dict:
    """Causal Polar Attention prefill.  q [B,T,Hq,d], k and v [B,T,Hkv,d] on the GPU."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_input(t, n)
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, T, Hkv, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [B,T,Hkv,d] with q's dtype")
    dev = q.device
    beta, null_bias, count_vec = _head_params(beta, null_bias, count_vec, Hq, d, dev)
    prm = _params(Hq, Hkv, d, beta, null_bias, count_vec, train_len, flags)
    out, cout = _outputs((B, T), Hq, d, dev, count_vec is not None, want_gate, want_lse)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    _lib.check(_lib.polar_attn_fwd(prm, _DT[q.dtype], B, T, q.data_ptr(), k.data_ptr(),
                                   v.data_ptr(), cout, s))
    return out


def attn_fwd_mixed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   memory: Optional[torch.Tensor] = None, beta=None, null_bias=None,
                   count_vec=None, train_len: int = 2048,
                   flags: int = _lib.POLAR_FLAG_LENGTH_TEMP | _lib.POLAR_FLAG_NULL_FLOOR,
                   want_gate: bool = True, want_lse: bool = True, stream=None) -> dict:
    """The three streams summed (see polar_attn_fwd_mixed): "mixed" [B,T,Hq,d] = dir + count
    + memory, plus the scalar outputs.  ``memory`` is the memory stream's output [B,T,Hq,d]
    float32 (e.g. from :func:`delta_sequence` with Hq heads), or None."""
    prm, keep, (B, T, Hq, Hkv, d) = _prefill_args(q, k, v, beta, null_bias, count_vec,
                                                  train_len, flags)
    dev = q.device
    if memory is not None:
        _check_aux(memory, "memory", dev, torch.float32, (B, T, Hq, d))
    out = dict(mixed=torch.empty(B, T, Hq, d, device=dev, dtype=torch.float32),
               n_eff=torch.empty(B, T, Hq, device=dev, dtype=torch.float32))
    out["gate"] = torch.empty(B, T, Hq, device=dev, dtype=torch.float32) if want_gate else None
    out["lse"] = torch.empty(B, T, Hq, device=dev, dtype=torch.float32) if want_lse else None
    cout = _lib.polar_outputs(None, None, _ptr(out["n_eff"]), _ptr(out["gate"]),
                              _ptr(out["lse"]))
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    _lib.check(_lib.polar_attn_fwd_mixed(prm, _DT[q.dtype], B, T, q.data_ptr(), k.data_ptr(),
                                         v.data_ptr(), _ptr(memory), out["mixed"].data_ptr(),
                                         cout, s))
    return out


def _prefill_args(q, k, v, beta, null_bias, count_vec, train_len, flags):
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_input(t, n)
    B, T, Hq, d = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, T, Hkv, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [B,T,Hkv,d] with q's dtype")
    dev = q.device
    beta, null_bias, count_vec = _head_params(beta, null_bias, count_vec, Hq, d, dev)
    prm = _params(Hq, Hkv, d, beta, null_bias, count_vec, train_len, flags)
    return prm, (beta, null_bias, count_vec), (B, T, Hq, Hkv, d)


def attn_fwd_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, beta=None,
                   null_bias=None, count_vec=None, train_len: int = 2048,
                   flags: int = _lib.POLAR_FLAG_LENGTH_TEMP | _lib.POLAR_FLAG_NULL_FLOOR,
                   window: int = 0, rope_theta: float = 0.0, want_attn: bool = False,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Prefill that also returns the residuals of the backward pass ("u_norm", "arg_max").

    ``window`` and ``rope_theta`` select the variant modes (polar_attn_fwd_train_variant);
    with RoPE, q and k are rotated into ``workspace`` (a uint8 device tensor of at least
    train_variant_workspace_bytes(...) bytes, allocated here when None).  ``want_attn``
    adds the plain softmax read-out "attn" [B,T,Hq,d]."""
    prm, keep, (B, T, Hq, Hkv, d) = _prefill_args(q, k, v, beta, null_bias, count_vec,
                                                  train_len, flags)
    dev = q.device
    out, cout = _outputs((B, T), Hq, d, dev, keep[2] is not None, True, True)
    out["u_norm"] = torch.empty(B, T, Hq, device=dev, dtype=torch.float32)
    out["arg_max"] = torch.empty(B, T, Hq, device=dev, dtype=torch.int32)
    saved = _lib.polar_saved(_ptr(out["u_norm"]), _ptr(out["arg_max"]))
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    if window == 0 and rope_theta == 0.0 and not want_attn:
        _lib.check(_lib.polar_attn_fwd_train(prm, _DT[q.dtype], B, T, q.data_ptr(),
                                             k.data_ptr(), v.data_ptr(), cout, saved, s))
        return out
    if want_attn:
        out["attn"] = torch.empty(B, T, Hq, d, device=dev, dtype=torch.float32)
    attn = _ptr(out.get("attn"))
    var = _lib.polar_variant(window, rope_theta, attn, None, 0)
    need = _lib.polar_train_variant_workspace_bytes(prm, var, _DT[q.dtype], B, T)
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _check_aux(workspace, "workspace", dev, None)
        var = _lib.polar_variant(window, rope_theta, attn, workspace.data_ptr(),
                                 workspace.numel() * workspace.element_size())
    _lib.check(_lib.polar_attn_fwd_train_variant(prm, var, _DT[q.dtype], B, T, q.data_ptr(),
                                                 k.data_ptr(), v.data_ptr(), cout, saved, s))
    return out


def train_variant_workspace_bytes(Hq: int, Hkv: int, B: int, T: int, window: int = 0,
                                  rope_theta: float = 0.0, dtype=torch.bfloat16,
                                  d: int = 64) -> int:
    prm = _lib.polar_params(Hq, Hkv, d, 2048, 0, None, None, None)
    var = _lib.polar_variant(window, rope_theta, None, None, 0)
    return _lib.polar_train_variant_workspace_bytes(prm, var, _DT[dtype], B, T)


def attn_fwd_variant(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, window: int = 0,
                     rope_theta: float = 0.0, want_attn: bool = True, beta=None,
                     null_bias=None, count_vec=None, train_len: int = 2048,
                     flags: int = _lib.POLAR_FLAG_LENGTH_TEMP | _lib.POLAR_FLAG_NULL_FLOOR,
                     rotate_keys_once: bool = True, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> dict:
    """Prefill with the variant modes: sliding ``window``, RoPE on load (``rope_theta``) and
    the plain softmax output ("attn", when ``want_attn``).

    With RoPE and ``rotate_keys_once``, the keys are rotated once into ``workspace`` (a
    uint8 device tensor of at least variant_workspace_bytes(...) bytes, allocated here when
    None) before the attention kernel; otherwise every workgroup rotates the keys it
    stages.  Both give bit-identical results."""
    prm, keep, (B, T, Hq, Hkv, d) = _prefill_args(q, k, v, beta, null_bias, count_vec,
                                                  train_len, flags)
    dev = q.device
    out, cout = _outputs((B, T), Hq, d, dev, keep[2] is not None, True, True)
    out["attn"] = (torch.empty(B, T, Hq, d, device=dev, dtype=torch.float32)
                   if want_attn else None)
    ws_ptr, ws_bytes = None, 0
    if rope_theta > 0 and rotate_keys_once:
        need = _lib.polar_variant_workspace_bytes(prm, _DT[q.dtype], B, T)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        _check_aux(workspace, "workspace", dev, None)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    var = _lib.polar_variant(window, rope_theta, _ptr(out["attn"]), ws_ptr, ws_bytes)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    _lib.check(_lib.polar_attn_fwd_variant(prm, var, _DT[q.dtype], B, T, q.data_ptr(),
                                           k.data_ptr(), v.data_ptr(), cout, s))
    return out


def variant_workspace_bytes(Hq: int, Hkv: int, B: int, T: int, dtype=torch.bfloat16,
                            d: int = 64) -> int:
    prm = _lib.polar_params(Hq, Hkv, d, 2048, 0, None, None, None)
    return _lib.polar_variant_workspace_bytes(prm, _DT[dtype], B, T)


def bwd_workspace_bytes(Hq: int, Hkv: int, B: int, T: int, d: int = 64, window: int = 0,
                        rope_theta: float = 0.0) -> int:
    prm = _lib.polar_params(Hq, Hkv, d, 2048, 0, None, None, None)
    if window == 0 and rope_theta == 0.0:
        return _lib.polar_bwd_workspace_bytes(prm, B, T)
    var = _lib.polar_variant(window, rope_theta, None, None, 0)
    return _lib.polar_bwd_variant_workspace_bytes(prm, var, B, T)


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, fwd: dict, cot: dict,
             beta=None, null_bias=None, count_vec=None, train_len: int = 2048,
             flags: int = _lib.POLAR_FLAG_LENGTH_TEMP | _lib.POLAR_FLAG_NULL_FLOOR,
             param_grads: bool = True, workspace: Optional[torch.Tensor] = None,
             window: int = 0, rope_theta: float = 0.0, stream=None) -> dict:
    """Backward of the causal prefill.

    ``fwd`` is what attn_fwd_train returned for the same arguments (``window`` and
    ``rope_theta`` included: they select polar_attn_bwd_variant); ``cot`` maps output
    names ("dir", "count", "n_eff", "gate", "lse", and "attn" for the softmax read-out) to
    float32 upstream gradients (missing names are zero).  Returns float32 dq, dk, dv and, with ``param_grads``, d_beta,
    d_null_bias and d_count_vec.
    """
    prm, keep, (B, T, Hq, Hkv, d) = _prefill_args(q, k, v, beta, null_bias, count_vec,
                                                  train_len, flags)
    dev = q.device
    f32t = torch.float32
    for name, dt, shp in (("dir", f32t, (B, T, Hq, d)), ("n_eff", f32t, (B, T, Hq)),
                          ("gate", f32t, (B, T, Hq)), ("lse", f32t, (B, T, Hq)),
                          ("u_norm", f32t, (B, T, Hq)), ("arg_max", torch.int32, (B, T, Hq))):
        _check_aux(fwd.get(name), f"fwd[{name!r}]", dev, dt, shp)
    cts = {}
    for name in _lib.COTANGENTS:
        c = cot.get(name)
        cts[name] = None if c is None else torch.as_tensor(
            c, dtype=torch.float32, device=dev).contiguous()
        if c is not None:
            want = (B, T, Hq, d) if name in ("dir", "count", "attn") else (B, T, Hq)
            _check_aux(cts[name], f"cot[{name!r}]", dev, f32t, want)
    f32 = dict(device=dev, dtype=torch.float32)
    g = dict(dq=torch.empty(B, T, Hq, d, **f32), dk=torch.empty(B, T, Hkv, d, **f32),
             dv=torch.empty(B, T, Hkv, d, **f32))
    if param_grads:
        g.update(d_beta=torch.empty(Hq, **f32), d_null_bias=torch.empty(Hq, **f32),
                 d_count_vec=torch.empty(Hq, d, **f32))
    variant = window != 0 or rope_theta != 0.0
    var = _lib.polar_variant(window, rope_theta, None, None, 0) if variant else None
    need = (_lib.polar_bwd_variant_workspace_bytes(prm, var, B, T) if variant
            else _lib.polar_bwd_workspace_bytes(prm, B, T))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check_aux(workspace, "workspace", dev, None)
    fo = _lib.polar_outputs(_ptr(fwd["dir"]), None, _ptr(fwd["n_eff"]), _ptr(fwd["gate"]),
                            _ptr(fwd["lse"]))
    sv = _lib.polar_saved(_ptr(fwd["u_norm"]), _ptr(fwd["arg_max"]))
    co = _lib.polar_cotangents(*(_ptr(cts[n]) for n in _lib.COTANGENTS))
    go = _lib.polar_grads(_ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g.get("d_beta")),
                          _ptr(g.get("d_null_bias")), _ptr(g.get("d_count_vec")))
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    nbytes = workspace.numel() * workspace.element_size()
    if variant:
        _lib.check(_lib.polar_attn_bwd_variant(prm, var, _DT[q.dtype], B, T, q.data_ptr(),
                                               k.data_ptr(), v.data_ptr(), fo, sv, co, go,
                                               workspace.data_ptr(), nbytes, s))
    else:
        _lib.check(_lib.polar_attn_bwd(prm, _DT[q.dtype], B, T, q.data_ptr(), k.data_ptr(),
                                       v.data_ptr(), fo, sv, co, go, workspace.data_ptr(),
                                       nbytes, s))
    return g


def decode_workspace_bytes(Hq: int, Hkv: int, B: int, max_seq_len: int, d: int = 64) -> int:
    prm = _lib.polar_params(Hq, Hkv, d, 2048, 0, None, None, None)
    return _lib.polar_decode_workspace_bytes(prm, B, max_seq_len)


def attn_decode_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                      page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                      beta=None, null_bias=None, count_vec=None, train_len: int = 2048,
                      flags: int = _lib.POLAR_FLAG_LENGTH_TEMP | _lib.POLAR_FLAG_NULL_FLOOR,
                      workspace: Optional[torch.Tensor] = None, want_gate: bool = True,
                      want_lse: bool = True, no_alloc: bool = False, stream=None) -> dict:
    """GQA paged decode.  q [B,Hq,d]; caches [num_pages,Hkv,page,d]; table [B,stride] int32.

    With ``no_alloc`` the call goes to polar_attn_decode_paged_noalloc, whose split partials
    live in the library's static scratch: no workspace is passed (``workspace`` must be
    None) and the C call allocates nothing; the outputs are still allocated here."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _check_input(t, n)
    B, Hq, d = q.shape
    num_pages, Hkv, page, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [num_pages,Hkv,page,d] matching q")
    dev = q.device
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B,stride]")
    _check_aux(page_table, "page_table", dev, torch.int32)
    _check_aux(seq_lens, "seq_lens", dev, torch.int32, (B,))
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _check_aux(t, n, dev, q.dtype)
    beta, null_bias, count_vec = _head_params(beta, null_bias, count_vec, Hq, d, dev)
    prm = _params(Hq, Hkv, d, beta, null_bias, count_vec, train_len, flags)
    if no_alloc and workspace is not None:
        raise ValueError("the allocation-free decode takes no workspace")
    if not no_alloc:
        need = _lib.polar_decode_workspace_bytes(prm, B, max_seq_len)
        if workspace is None:
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
        _check_aux(workspace, "workspace", dev, None)
    out, cout = _outputs((B,), Hq, d, dev, count_vec is not None, want_gate, want_lse)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    if no_alloc:
        _lib.check(_lib.polar_attn_decode_paged_noalloc(
            prm, _DT[q.dtype], B, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
            num_pages, page, page_table.data_ptr(), page_table.shape[1], seq_lens.data_ptr(),
            max_seq_len, cout, s))
        return out
    _lib.check(_lib.polar_attn_decode_paged(
        prm, _DT[q.dtype], B, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), num_pages,
        page, page_table.data_ptr(), page_table.shape[1], seq_lens.data_ptr(), max_seq_len,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(), cout, s))
    return out


def _paged_args(k_cache, v_cache, page_table, start_pos, B, dev):
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _check_input(t, n)
        _check_aux(t, n, dev, None)
    num_pages, Hkv, page, d = k_cache.shape
    if v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("caches must match")
    if page_table.dim() != 2 or page_table.shape[0] != B:
        raise ValueError("page_table must be [B,stride]")
    _check_aux(page_table, "page_table", dev, torch.int32)
    _check_aux(start_pos, "start_pos", dev, torch.int32, (B,))
    return num_pages, Hkv, page, d


def kv_append(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
              v_cache: torch.Tensor, page_table: torch.Tensor, start_pos: torch.Tensor,
              max_seq_len: int, stream=None) -> None:
    """Write k_new, v_new [B,C,Hkv,d] into the page pools in place (see polar_kv_append)."""
    for t, n in ((k_new, "k_new"), (v_new, "v_new")):
        _check_input(t, n)
    B, C, Hkv, d = k_new.shape
    num_pages, Hkv2, page, d2 = _paged_args(k_cache, v_cache, page_table, start_pos, B,
                                            k_new.device)
    if (Hkv2, d2) != (Hkv, d) or v_new.shape != k_new.shape or k_new.dtype != k_cache.dtype:
        raise ValueError("k_new/v_new must be [B,C,Hkv,d] matching the pools")
    prm = _lib.polar_params(Hkv, Hkv, d, 2048, 0, None, None, None)
    s = torch.cuda.current_stream(k_new.device).cuda_stream if stream is None else stream
    _lib.check(_lib.polar_kv_append(prm, _DT[k_new.dtype], B, C, k_new.data_ptr(),
                                    v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                    num_pages, page, page_table.data_ptr(), page_table.shape[1],
                                    start_pos.data_ptr(), max_seq_len, s))


def attn_prefill_paged(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                       page_table: torch.Tensor, start_pos: torch.Tensor, max_seq_len: int,
                       beta=None, null_bias=None, count_vec=None, train_len: int = 2048,
                       flags: int = _lib.POLAR_FLAG_LENGTH_TEMP | _lib.POLAR_FLAG_NULL_FLOOR,
                       want_gate: bool = True, want_lse: bool = True, stream=None) -> dict:
    """Chunked prefill over the paged cache.  q [B,C,Hq,d]: row t is the token at position
    start_pos[b] + t; its keys come from the pools (append the chunk first)."""
    _check_input(q, "q")
    B, C, Hq, d = q.shape
    num_pages, Hkv, page, d2 = _paged_args(k_cache, v_cache, page_table, start_pos, B, q.device)
    if d2 != d or k_cache.dtype != q.dtype:
        raise ValueError("caches must match q's head_dim and dtype")
    dev = q.device
    beta, null_bias, count_vec = _head_params(beta, null_bias, count_vec, Hq, d, dev)
    prm = _params(Hq, Hkv, d, beta, null_bias, count_vec, train_len, flags)
    out, cout = _outputs((B, C), Hq, d, dev, count_vec is not None, want_gate, want_lse)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    _lib.check(_lib.polar_attn_prefill_paged(
        prm, _DT[q.dtype], B, C, q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), num_pages,
        page, page_table.data_ptr(), page_table.shape[1], start_pos.data_ptr(), max_seq_len,
        cout, s))
    return out


def delta_step(state_pool: torch.Tensor, slots: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
               v: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
               normalize_qk: bool = True, stream=None) -> torch.Tensor:
    """In-place gated-delta memory step (see polar_delta_step): updates
    state_pool[slots[b]] for every sequence b and returns o [B,H,d_v] (float32)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_input(t, n)
    dev = q.device
    _check_aux(state_pool, "state_pool", dev, torch.float32)
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [num_slots,H,d_v,d_k]")
    num_slots, H, dv, dk = state_pool.shape
    B = q.shape[0]
    if q.shape != (B, H, dk) or k.shape != q.shape or v.shape != (B, H, dv):
        raise ValueError("q, k must be [B,H,d_k] and v [B,H,d_v] matching the pool")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    _check_aux(slots, "slots", dev, torch.int32, (B,))
    alpha = torch.as_tensor(alpha, dtype=torch.float32, device=dev).contiguous()
    beta = torch.as_tensor(beta, dtype=torch.float32, device=dev).contiguous()
    _check_aux(alpha, "alpha", dev, torch.float32, (B, H))
    _check_aux(beta, "beta", dev, torch.float32, (B, H))
    out = torch.empty(B, H, dv, device=dev, dtype=torch.float32)
    prm = _lib.polar_delta_params(H, dk, dv, _lib.POLAR_DELTA_NORMALIZE_QK if normalize_qk else 0)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    _lib.check(_lib.polar_delta_step(prm, _DT[q.dtype], B, state_pool.data_ptr(), num_slots,
                                     slots.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     alpha.data_ptr(), beta.data_ptr(), out.data_ptr(), s))
    return out


def delta_sequence(state_pool: torch.Tensor, slots: torch.Tensor, q: torch.Tensor,
                   k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor, beta: torch.Tensor,
                   normalize_qk: bool = True, stream=None) -> torch.Tensor:
    """The memory stream over T tokens (see polar_delta_sequence): runs the gated-delta step
    for t = 0..T-1 on state_pool[slots[b]] in place and returns o [B,T,H,d_v] (float32).
    q, k [B,T,H,d_k]; v [B,T,H,d_v]; alpha, beta [B,T,H]."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _check_input(t, n)
    dev = q.device
    _check_aux(state_pool, "state_pool", dev, torch.float32)
    if state_pool.dim() != 4:
        raise ValueError("state_pool must be [num_slots,H,d_v,d_k]")
    num_slots, H, dv, dk = state_pool.shape
    if q.dim() != 4:
        raise ValueError("q must be [B,T,H,d_k]")
    B, T = q.shape[:2]
    if q.shape != (B, T, H, dk) or k.shape != q.shape or v.shape != (B, T, H, dv):
        raise ValueError("q, k must be [B,T,H,d_k] and v [B,T,H,d_v] matching the pool")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    _check_aux(slots, "slots", dev, torch.int32, (B,))
    alpha = torch.as_tensor(alpha, dtype=torch.float32, device=dev).contiguous()
    beta = torch.as_tensor(beta, dtype=torch.float32, device=dev).contiguous()
    _check_aux(alpha, "alpha", dev, torch.float32, (B, T, H))
    _check_aux(beta, "beta", dev, torch.float32, (B, T, H))
    out = torch.empty(B, T, H, dv, device=dev, dtype=torch.float32)
    prm = _lib.polar_delta_params(H, dk, dv, _lib.POLAR_DELTA_NORMALIZE_QK if normalize_qk else 0)
    s = torch.cuda.current_stream(dev).cuda_stream if stream is None else stream
    _lib.check(_lib.polar_delta_sequence(prm, _DT[q.dtype], B, T, state_pool.data_ptr(),
                                         num_slots, slots.data_ptr(), q.data_ptr(), k.data_ptr(),
                                         v.data_ptr(), alpha.data_ptr(), beta.data_ptr(),
                                         out.data_ptr(), s))
    return out

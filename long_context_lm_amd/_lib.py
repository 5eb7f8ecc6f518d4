"""ctypes binding of libpolar (include/polar.h): argument marshalling only.

Every step of the computation runs in the HIP kernels of libpolar.so.  torch is used for
device memory and for the current HIP stream.  There is no fallback: if the library is
missing or no GPU is present, calls fail loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpolar.so")

POLAR_OK = 0
POLAR_ERR_NULL_POINTER = 1
POLAR_ERR_BAD_SHAPE = 2
POLAR_ERR_UNSUPPORTED = 3
POLAR_ERR_MISALIGNED = 4
POLAR_ERR_WORKSPACE_TOO_SMALL = 5
POLAR_ERR_HIP = 6

POLAR_DTYPE_F32 = 0
POLAR_DTYPE_BF16 = 1

POLAR_FLAG_LENGTH_TEMP = 1
POLAR_FLAG_NULL_FLOOR = 2
POLAR_DELTA_NORMALIZE_QK = 1

EXPORTS = ("polar_attn_fwd", "polar_attn_fwd_mixed", "polar_decode_workspace_bytes", "polar_attn_decode_paged",
           "polar_attn_decode_paged_noalloc",
           "polar_attn_fwd_train", "polar_bwd_workspace_bytes", "polar_attn_bwd",
           "polar_attn_fwd_variant", "polar_variant_workspace_bytes", "polar_kv_append",
           "polar_attn_prefill_paged",
           "polar_delta_step", "polar_delta_sequence",
           "polar_train_variant_workspace_bytes", "polar_attn_fwd_train_variant",
           "polar_bwd_variant_workspace_bytes", "polar_attn_bwd_variant",
           "polar_status_str", "polar_last_error", "polar_abi_version")


ABI_VERSION = 7                            # POLAR_ABI_VERSION of include/polar.h


class polar_params(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("train_len", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("beta", ctypes.c_void_p),
                ("null_bias", ctypes.c_void_p), ("count_vec", ctypes.c_void_p)]


class polar_outputs(ctypes.Structure):
    _fields_ = [("dir", ctypes.c_void_p), ("count", ctypes.c_void_p),
                ("n_eff", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("lse", ctypes.c_void_p)]


class polar_delta_params(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("key_dim", ctypes.c_int32),
                ("value_dim", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class polar_variant(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("rope_theta", ctypes.c_float),
                ("attn", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class polar_saved(ctypes.Structure):
    _fields_ = [("u_norm", ctypes.c_void_p), ("arg_max", ctypes.c_void_p)]


class polar_cotangents(ctypes.Structure):
    _fields_ = [("dir", ctypes.c_void_p), ("count", ctypes.c_void_p),
                ("n_eff", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("attn", ctypes.c_void_p)]


COTANGENTS = tuple(name for name, _ in polar_cotangents._fields_)


class polar_grads(ctypes.Structure):
    _fields_ = [("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
                ("d_beta", ctypes.c_void_p), ("d_null_bias", ctypes.c_void_p),
                ("d_count_vec", ctypes.c_void_p)]


class PolarError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"libpolar status {status}: {detail}")
        self.status = status
        self.detail = detail


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpolar.so once and declare its signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with "
                                "`python -m long_context_lm_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    lib.polar_attn_fwd.restype = I32
    lib.polar_attn_fwd.argtypes = [P(polar_params), I32, I32, I32, VP, VP, VP, P(polar_outputs),
                                   VP]
    lib.polar_decode_workspace_bytes.restype = SZ
    lib.polar_decode_workspace_bytes.argtypes = [P(polar_params), I32, I32]
    lib.polar_attn_decode_paged.restype = I32
    lib.polar_attn_decode_paged.argtypes = [P(polar_params), I32, I32, VP, VP, VP, I32, I32, VP,
                                            I32, VP, I32, VP, SZ, P(polar_outputs), VP]
    lib.polar_attn_decode_paged_noalloc.restype = I32
    lib.polar_attn_decode_paged_noalloc.argtypes = [P(polar_params), I32, I32, VP, VP, VP, I32,
                                                    I32, VP, I32, VP, I32, P(polar_outputs), VP]
    lib.polar_attn_fwd_train.restype = I32
    lib.polar_attn_fwd_train.argtypes = [P(polar_params), I32, I32, I32, VP, VP, VP,
                                         P(polar_outputs), P(polar_saved), VP]
    lib.polar_bwd_workspace_bytes.restype = SZ
    lib.polar_bwd_workspace_bytes.argtypes = [P(polar_params), I32, I32]
    lib.polar_attn_bwd.restype = I32
    lib.polar_attn_bwd.argtypes = [P(polar_params), I32, I32, I32, VP, VP, VP, P(polar_outputs),
                                   P(polar_saved), P(polar_cotangents), P(polar_grads), VP, SZ,
                                   VP]
    lib.polar_attn_fwd_variant.restype = I32
    lib.polar_attn_fwd_variant.argtypes = [P(polar_params), P(polar_variant), I32, I32, I32, VP,
                                           VP, VP, P(polar_outputs), VP]
    lib.polar_variant_workspace_bytes.restype = SZ
    lib.polar_variant_workspace_bytes.argtypes = [P(polar_params), I32, I32, I32]
    lib.polar_train_variant_workspace_bytes.restype = SZ
    lib.polar_train_variant_workspace_bytes.argtypes = [P(polar_params), P(polar_variant), I32,
                                                        I32, I32]
    lib.polar_attn_fwd_train_variant.restype = I32
    lib.polar_attn_fwd_train_variant.argtypes = [P(polar_params), P(polar_variant), I32, I32,
                                                 I32, VP, VP, VP, P(polar_outputs),
                                                 P(polar_saved), VP]
    lib.polar_bwd_variant_workspace_bytes.restype = SZ
    lib.polar_bwd_variant_workspace_bytes.argtypes = [P(polar_params), P(polar_variant), I32,
                                                      I32]
    lib.polar_attn_bwd_variant.restype = I32
    lib.polar_attn_bwd_variant.argtypes = [P(polar_params), P(polar_variant), I32, I32, I32, VP,
                                           VP, VP, P(polar_outputs), P(polar_saved),
                                           P(polar_cotangents), P(polar_grads), VP, SZ, VP]
    lib.polar_kv_append.restype = I32
    lib.polar_kv_append.argtypes = [P(polar_params), I32, I32, I32, VP, VP, VP, VP, I32, I32, VP,
                                    I32, VP, I32, VP]
    lib.polar_attn_prefill_paged.restype = I32
    lib.polar_attn_prefill_paged.argtypes = [P(polar_params), I32, I32, I32, VP, VP, VP, I32, I32,
                                             VP, I32, VP, I32, P(polar_outputs), VP]
    lib.polar_delta_step.restype = I32
    lib.polar_delta_step.argtypes = [P(polar_delta_params), I32, I32, VP, I32, VP, VP, VP, VP, VP,
                                     VP, VP, VP]
    lib.polar_delta_sequence.restype = I32
    lib.polar_delta_sequence.argtypes = [P(polar_delta_params), I32, I32, I32, VP, I32, VP, VP, VP,
                                         VP, VP, VP, VP, VP]
    lib.polar_attn_fwd_mixed.restype = I32
    lib.polar_attn_fwd_mixed.argtypes = [P(polar_params), I32, I32, I32, VP, VP, VP, VP, VP,
                                         P(polar_outputs), VP]
    lib.polar_status_str.restype = ctypes.c_char_p
    lib.polar_status_str.argtypes = [I32]
    lib.polar_last_error.restype = ctypes.c_char_p
    lib.polar_last_error.argtypes = []
    lib.polar_abi_version.restype = I32
    lib.polar_abi_version.argtypes = []
    if lib.polar_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has C ABI version {lib.polar_abi_version()}, the binding "
                           f"declares version {ABI_VERSION}: rebuild it")
    _lib = lib
    return lib


# ----------------------------------------------------------------- raw C names
def polar_abi_version() -> int:
    return load().polar_abi_version()


def polar_status_str(status: int) -> str:
    return load().polar_status_str(status).decode()


def polar_last_error() -> str:
    return load().polar_last_error().decode()


def polar_attn_fwd(params, dtype, B, T, q, k, v, outputs, stream) -> int:
    """Direct call of the C entry point (pointers as ints); returns the status code."""
    return load().polar_attn_fwd(ctypes.byref(params), dtype, B, T, q, k, v,
                                 ctypes.byref(outputs), stream)


def polar_decode_workspace_bytes(params, B, max_seq_len) -> int:
    return load().polar_decode_workspace_bytes(ctypes.byref(params), B, max_seq_len)


def polar_attn_decode_paged(params, dtype, B, q, k_cache, v_cache, num_pages, page_size,
                            page_table, page_table_stride, seq_lens, max_seq_len, workspace,
                            workspace_bytes, outputs, stream) -> int:
    return load().polar_attn_decode_paged(ctypes.byref(params), dtype, B, q, k_cache, v_cache,
                                          num_pages, page_size, page_table, page_table_stride,
                                          seq_lens, max_seq_len, workspace, workspace_bytes,
                                          ctypes.byref(outputs), stream)


POLAR_NOALLOC_SCRATCH_BYTES = 16 << 20    # include/polar.h


def polar_attn_decode_paged_noalloc(params, dtype, B, q, k_cache, v_cache, num_pages,
                                    page_size, page_table, page_table_stride, seq_lens,
                                    max_seq_len, outputs, stream) -> int:
    return load().polar_attn_decode_paged_noalloc(ctypes.byref(params), dtype, B, q, k_cache,
                                                  v_cache, num_pages, page_size, page_table,
                                                  page_table_stride, seq_lens, max_seq_len,
                                                  ctypes.byref(outputs), stream)


def polar_attn_fwd_train(params, dtype, B, T, q, k, v, outputs, saved, stream) -> int:
    return load().polar_attn_fwd_train(ctypes.byref(params), dtype, B, T, q, k, v,
                                       ctypes.byref(outputs), ctypes.byref(saved), stream)


def polar_attn_fwd_variant(params, variant, dtype, B, T, q, k, v, outputs, stream) -> int:
    return load().polar_attn_fwd_variant(ctypes.byref(params),
                                         None if variant is None else ctypes.byref(variant),
                                         dtype, B, T, q, k, v, ctypes.byref(outputs), stream)


def polar_kv_append(params, dtype, B, C, k_new, v_new, k_cache, v_cache, num_pages, page_size,
                    page_table, stride, start_pos, max_seq_len, stream) -> int:
    return load().polar_kv_append(ctypes.byref(params), dtype, B, C, k_new, v_new, k_cache,
                                  v_cache, num_pages, page_size, page_table, stride, start_pos,
                                  max_seq_len, stream)


def polar_attn_prefill_paged(params, dtype, B, C, q, k_cache, v_cache, num_pages, page_size,
                             page_table, stride, start_pos, max_seq_len, outputs, stream) -> int:
    return load().polar_attn_prefill_paged(ctypes.byref(params), dtype, B, C, q, k_cache,
                                           v_cache, num_pages, page_size, page_table, stride,
                                           start_pos, max_seq_len, ctypes.byref(outputs), stream)


def polar_delta_step(params, dtype, B, state_pool, num_slots, slots, q, k, v, alpha, beta, out,
                     stream) -> int:
    return load().polar_delta_step(ctypes.byref(params), dtype, B, state_pool, num_slots, slots,
                                   q, k, v, alpha, beta, out, stream)


def polar_attn_fwd_mixed(params, dtype, B, T, q, k, v, memory, mixed, outputs, stream) -> int:
    return load().polar_attn_fwd_mixed(ctypes.byref(params), dtype, B, T, q, k, v, memory, mixed,
                                       ctypes.byref(outputs), stream)


def polar_delta_sequence(params, dtype, B, T, state_pool, num_slots, slots, q, k, v, alpha, beta,
                         out, stream) -> int:
    return load().polar_delta_sequence(ctypes.byref(params), dtype, B, T, state_pool, num_slots,
                                       slots, q, k, v, alpha, beta, out, stream)


def polar_variant_workspace_bytes(params, dtype, B, T) -> int:
    return load().polar_variant_workspace_bytes(ctypes.byref(params), dtype, B, T)


def polar_bwd_workspace_bytes(params, B, T) -> int:
    return load().polar_bwd_workspace_bytes(ctypes.byref(params), B, T)


def polar_attn_bwd(params, dtype, B, T, q, k, v, fwd, saved, cot, grads, workspace,
                   workspace_bytes, stream) -> int:
    return load().polar_attn_bwd(ctypes.byref(params), dtype, B, T, q, k, v, ctypes.byref(fwd),
                                 ctypes.byref(saved), ctypes.byref(cot), ctypes.byref(grads),
                                 workspace, workspace_bytes, stream)


def _var_ref(variant):
    return None if variant is None else ctypes.byref(variant)


def polar_train_variant_workspace_bytes(params, variant, dtype, B, T) -> int:
    return load().polar_train_variant_workspace_bytes(ctypes.byref(params), _var_ref(variant),
                                                      dtype, B, T)


def polar_attn_fwd_train_variant(params, variant, dtype, B, T, q, k, v, outputs, saved,
                                 stream) -> int:
    return load().polar_attn_fwd_train_variant(ctypes.byref(params), _var_ref(variant), dtype,
                                               B, T, q, k, v, ctypes.byref(outputs),
                                               ctypes.byref(saved), stream)


def polar_bwd_variant_workspace_bytes(params, variant, B, T) -> int:
    return load().polar_bwd_variant_workspace_bytes(ctypes.byref(params), _var_ref(variant), B, T)


def polar_attn_bwd_variant(params, variant, dtype, B, T, q, k, v, fwd, saved, cot, grads,
                           workspace, workspace_bytes, stream) -> int:
    return load().polar_attn_bwd_variant(ctypes.byref(params), _var_ref(variant), dtype, B, T, q,
                                         k, v, ctypes.byref(fwd), ctypes.byref(saved),
                                         ctypes.byref(cot), ctypes.byref(grads), workspace,
                                         workspace_bytes, stream)


def check(status: int) -> None:
    if status != POLAR_OK:
        raise PolarError(status, f"{polar_status_str(status)}: {polar_last_error()}")

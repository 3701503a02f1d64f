"""ctypes binding of ``libmla.so``: argument marshalling only.

Each function has the name and argument order of the C entry point in
``include/mla.h``.  Tensors are torch tensors on the GPU (torch provides
device memory and the current stream); sizes are read from their shapes and
passed through unchanged.  Every step of the computation runs in the HIP
library: if it is not built, importing works but the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla.so")

FP32, BF16, FP8_E4M3, FP8_E4M3_PO2 = 0, 1, 2, 3
FLAG_GENERIC_DECODE = 1
FLAG_VALIDATE = 2

OK = 0
ERR_INVALID_ARGUMENT = -1
ERR_UNSUPPORTED = -2
ERR_WORKSPACE_TOO_SMALL = -3
ERR_HIP = -4

EXPORTS = ("mla_abi_version", "mla_last_error", "mla_device_cu_count",
           "mla_cache_append_workspace_size", "mla_cache_append",
           "mla_decode_workspace_size", "mla_decode", "mla_decode_combine", "mla_out_proj",
           "mla_decode_combine_out_proj", "mla_query_absorb", "mla_cache_append_query_absorb",
           "mla_linear_workspace_size",
           "mla_linear", "mla_decode_noalloc", "mla_prefill_workspace_size", "mla_prefill")
NOALLOC_SCRATCH_BYTES = 64 << 20


class MlaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"mla error {code}: {msg}")
        self.code = code


class mla_dims(ctypes.Structure):
    _fields_ = [
        ("num_heads", ctypes.c_int32),
        ("d_latent", ctypes.c_int32),
        ("d_rope", ctypes.c_int32),
        ("d_nope", ctypes.c_int32),
        ("d_v", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("cache_dtype", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("rope_base", ctypes.c_float),
        ("flags", ctypes.c_int32),
    ]


def make_dims(num_heads, d_latent, d_rope, d_nope, d_v, block_size, cache_dtype, act_dtype,
              softmax_scale=0.0, rope_base=0.0, flags=0) -> mla_dims:
    return mla_dims(num_heads, d_latent, d_rope, d_nope, d_v, block_size, cache_dtype, act_dtype,
                    softmax_scale, rope_base, flags)


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def lib():
    """Load libmla.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mla_latent_kv_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        D = ctypes.POINTER(mla_dims)
        L.mla_abi_version.restype = ctypes.c_int
        L.mla_last_error.restype = ctypes.c_char_p
        L.mla_device_cu_count.restype = ctypes.c_int
        L.mla_cache_append_workspace_size.argtypes = [D, _I, _I]
        L.mla_cache_append_workspace_size.restype = ctypes.c_size_t
        L.mla_cache_append.argtypes = [D, _P, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P, _P,
                                       ctypes.c_size_t, _P]
        L.mla_decode_workspace_size.argtypes = [D, _I, _I, _I]
        L.mla_decode_workspace_size.restype = ctypes.c_size_t
        L.mla_decode.argtypes = [D, _P, _I, _I, _P, _P, _P, _I, _P, _I, _P, ctypes.c_size_t, _P]
        L.mla_decode_combine.argtypes = [D, _P, ctypes.c_size_t, _I, _I, _P, _I, _P, _P, _P]
        L.mla_out_proj.argtypes = [D, _P, _I, _P, _P, _P]
        L.mla_decode_combine_out_proj.argtypes = [D, _P, ctypes.c_size_t, _I, _I, _P, _I, _P, _P,
                                                  _P, _P, _P]
        L.mla_query_absorb.argtypes = [D, _P, _P, _P, _P, _I, _P]
        L.mla_cache_append_query_absorb.argtypes = [D, _P, _I, _I, _P, _P, _P, _P, _P, _I, _P, _P,
                                                    _P, ctypes.c_size_t, _P, _P, _P, _P, _I, _P]
        L.mla_linear_workspace_size.argtypes = [D, _I, _I, _I]
        L.mla_linear_workspace_size.restype = ctypes.c_size_t
        L.mla_linear.argtypes = [D, _P, _I, _I, _P, _I, _P, _P, ctypes.c_size_t, _P]
        L.mla_decode_noalloc.argtypes = [D, _P, _I, _I, _P, _P, _P, _I, _P, _I, _P, _P, _P]
        L.mla_prefill_workspace_size.argtypes = [D, _I, _I]
        L.mla_prefill_workspace_size.restype = ctypes.c_size_t
        L.mla_prefill.argtypes = [D, _P, _I, _P, _P, _P, _I, _P, _P, _P, _P, ctypes.c_size_t, _P]
        for f in ("mla_cache_append", "mla_decode", "mla_decode_combine", "mla_out_proj",
                  "mla_decode_combine_out_proj", "mla_query_absorb", "mla_cache_append_query_absorb",
                  "mla_linear", "mla_decode_noalloc", "mla_prefill"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(rc: int):
    if rc != OK:
        raise MlaError(rc, lib().mla_last_error().decode())


def mla_abi_version() -> int:
    return lib().mla_abi_version()


def mla_device_cu_count() -> int:
    return lib().mla_device_cu_count()


def mla_cache_append_workspace_size(dims, n_tokens: int, d_model: int) -> int:
    return lib().mla_cache_append_workspace_size(ctypes.byref(dims), n_tokens, d_model)


def mla_cache_append(dims, h, w_dkv, w_kr, seq_ids, positions, page_table, cache,
                     cache_scales=None, workspace=None, stream=None):
    """h [T, d_model]; page_table [B, max_blocks]; cache [num_blocks, bs, D];
    workspace: a device tensor of mla_cache_append_workspace_size bytes (or None if 0)."""
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_cache_append(ctypes.byref(dims), _ptr(h), h.shape[0], h.shape[1], _ptr(w_dkv),
                                  _ptr(w_kr), _ptr(seq_ids), _ptr(positions), _ptr(page_table),
                                  page_table.shape[1], _ptr(cache), _ptr(cache_scales),
                                  _ptr(workspace), wsb, _stream(stream)))


def mla_decode_workspace_size(dims, batch: int, n_q: int, num_partitions: int = 0) -> int:
    return lib().mla_decode_workspace_size(ctypes.byref(dims), batch, n_q, num_partitions)


def mla_decode(dims, q, cache, cache_scales, page_table, seq_lens, workspace,
               num_partitions: int = 0, stream=None):
    """q [B, n_q, H, D]; workspace a uint8 tensor of mla_decode_workspace_size bytes."""
    _check(lib().mla_decode(ctypes.byref(dims), _ptr(q), q.shape[0], q.shape[1], _ptr(cache),
                            _ptr(cache_scales), _ptr(page_table), page_table.shape[1],
                            _ptr(seq_lens), num_partitions, _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream(stream)))


def mla_decode_combine(dims, workspace, seq_lens, u_out, lse_out=None, num_partitions: int = 0,
                       stream=None):
    """u_out [B, n_q, H, d_latent]; lse_out [B, n_q, H] fp32 or None."""
    _check(lib().mla_decode_combine(ctypes.byref(dims), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(),
                                    u_out.shape[0], u_out.shape[1], _ptr(seq_lens),
                                    num_partitions, _ptr(u_out), _ptr(lse_out), _stream(stream)))


def mla_decode_combine_out_proj(dims, workspace, seq_lens, w_uv, out, batch: int, n_q: int,
                                u_out=None, lse_out=None, num_partitions: int = 0, stream=None):
    """out [B*n_q, H, d_v]; u_out [B, n_q, H, d_latent] or None; lse_out [B, n_q, H] or None."""
    _check(lib().mla_decode_combine_out_proj(ctypes.byref(dims), _ptr(workspace),
                                             workspace.numel() * workspace.element_size(),
                                             batch, n_q, _ptr(seq_lens), num_partitions,
                                             _ptr(w_uv), _ptr(out), _ptr(u_out), _ptr(lse_out),
                                             _stream(stream)))


def mla_out_proj(dims, u, w_uv, out, stream=None):
    """u [rows, H, d_latent]; w_uv [H, d_v, d_latent]; out [rows, H, d_v]."""
    _check(lib().mla_out_proj(ctypes.byref(dims), _ptr(u), u.shape[0], _ptr(w_uv), _ptr(out),
                              _stream(stream)))


def mla_query_absorb(dims, q_in, positions, w_uk, q_out, stream=None):
    """q_in [rows, H, d_nope + d_rope] (any leading shape whose product is rows);
    positions [rows] int32; w_uk [H, d_nope, d_latent]; q_out [rows, H, d_latent + d_rope]."""
    rows = q_in.numel() // (dims.num_heads * (dims.d_nope + dims.d_rope))
    _check(lib().mla_query_absorb(ctypes.byref(dims), _ptr(q_in), _ptr(positions), _ptr(w_uk),
                                  _ptr(q_out), rows, _stream(stream)))


def mla_cache_append_query_absorb(dims, h, w_dkv, w_kr, seq_ids, positions, page_table, cache,
                                  cache_scales, workspace, q_in, q_positions, w_uk, q_out, stream=None):
    """mla_cache_append(dims, h, ..., workspace) then mla_query_absorb(dims, q_in,
    q_positions, w_uk, q_out), with the arguments of those two calls."""
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rows = q_in.numel() // (dims.num_heads * (dims.d_nope + dims.d_rope))
    _check(lib().mla_cache_append_query_absorb(
        ctypes.byref(dims), _ptr(h), h.shape[0], h.shape[1], _ptr(w_dkv), _ptr(w_kr), _ptr(seq_ids),
        _ptr(positions), _ptr(page_table), page_table.shape[1], _ptr(cache), _ptr(cache_scales),
        _ptr(workspace), wsb, _ptr(q_in), _ptr(q_positions), _ptr(w_uk), _ptr(q_out), rows,
        _stream(stream)))


def mla_linear_workspace_size(dims, rows: int, n: int, k: int) -> int:
    return lib().mla_linear_workspace_size(ctypes.byref(dims), rows, n, k)


def mla_linear(dims, x, w, y, workspace=None, stream=None):
    """y = x W^T: x [rows, k] (any leading shape whose product is rows); w [n, k];
    y [rows, n]; workspace a device tensor of mla_linear_workspace_size bytes
    (or None if that is 0)."""
    k = x.shape[-1]
    rows = x.numel() // k
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mla_linear(ctypes.byref(dims), _ptr(x), rows, k, _ptr(w), w.shape[0], _ptr(y),
                            _ptr(workspace), wsb, _stream(stream)))


def mla_decode_noalloc(dims, q, cache, cache_scales, page_table, seq_lens, u_out, lse_out=None,
                       num_partitions: int = 0, stream=None):
    """mla_decode + mla_decode_combine with the library's static scratch as the
    workspace.  q [B, n_q, H, D]; u_out [B, n_q, H, d_latent]; lse_out [B, n_q, H] or None."""
    _check(lib().mla_decode_noalloc(ctypes.byref(dims), _ptr(q), q.shape[0], q.shape[1], _ptr(cache),
                                    _ptr(cache_scales), _ptr(page_table), page_table.shape[1],
                                    _ptr(seq_lens), num_partitions, _ptr(u_out), _ptr(lse_out),
                                    _stream(stream)))


def mla_prefill_workspace_size(dims, n_tokens: int, seq_len: int) -> int:
    return lib().mla_prefill_workspace_size(ctypes.byref(dims), n_tokens, seq_len)


def mla_prefill(dims, q_in, cache, page_table_row, seq_len: int, w_uk, w_uv, out, workspace, stream=None,
                cache_scales=None):
    """q_in [C, H, d_nope + d_rope] (q^R not rotated); page_table_row [max_blocks] int32;
    out [C, H, d_v]; workspace a uint8 tensor of mla_prefill_workspace_size bytes;
    cache_scales [nblk, bs, 5] fp32 for an e4m3 cache."""
    _check(lib().mla_prefill(ctypes.byref(dims), _ptr(q_in), q_in.shape[0], _ptr(cache), _ptr(cache_scales),
                             _ptr(page_table_row), seq_len, _ptr(w_uk), _ptr(w_uv), _ptr(out), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream)))

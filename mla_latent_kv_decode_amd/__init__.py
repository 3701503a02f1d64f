"""MI355X (gfx950) MLA decode over a paged latent cache.

The computation lives in the HIP library ``libmla.so`` (sources in
``csrc/``, C ABI in ``include/mla.h``); this package is its thin ctypes
binding.  Build the library with ``python -m mla_latent_kv_decode_amd.build``.
"""
from ._lib import (  # noqa: F401
    BF16, EXPORTS, FLAG_GENERIC_DECODE, FLAG_VALIDATE, FP32, FP8_E4M3, FP8_E4M3_PO2, LIB_PATH, MlaError, lib, make_dims,
    mla_abi_version, mla_cache_append, mla_cache_append_workspace_size, mla_decode,
    mla_decode_combine, mla_decode_combine_out_proj, mla_decode_workspace_size,
    mla_device_cu_count, mla_dims, mla_linear, mla_linear_workspace_size, mla_out_proj,
    mla_query_absorb,
    mla_cache_append_query_absorb, mla_decode_noalloc, NOALLOC_SCRATCH_BYTES,
    mla_prefill, mla_prefill_workspace_size,
)

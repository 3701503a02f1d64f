"""Host-side checks of the C ABI: the library loads, exports every entry point
declared in include/mla.h, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from mla_latent_kv_decode_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from mla_latent_kv_decode_amd import build
        build.build()
    return _lib


def declared_functions():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_hot_path_calls():
    names = declared_functions()
    for n in ["mla_cache_append", "mla_decode", "mla_decode_combine", "mla_out_proj"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    lib = L.lib()
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} not exported"
    assert set(declared_functions()) == set(L.EXPORTS)
    assert L.mla_abi_version() == 1


def _dims(L, **kw):
    base = dict(num_heads=128, d_latent=512, d_rope=64, d_nope=128, d_v=128, block_size=64,
                cache_dtype=L.BF16, act_dtype=L.BF16)
    base.update(kw)
    return L.make_dims(**base)


FAKE = 1 << 20  # aligned, non-null, never dereferenced: validation fails first


def test_decode_validation_errors(L):
    lib = L.lib()
    d = _dims(L)
    ws = L.mla_decode_workspace_size(d, 4, 1, 8)
    assert ws > 0
    call = lambda dims, q=FAKE, batch=4, n_q=1, ws_bytes=ws, seq=FAKE, sc=None, G=8: lib.mla_decode(
        dims, q, batch, n_q, FAKE, sc, FAKE, 16, seq, G, FAKE, ws_bytes, None)
    assert call(None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), n_q=0) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), q=None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), seq=None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), q=FAKE + 1) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), ws_bytes=ws - 1) == L.ERR_WORKSPACE_TOO_SMALL
    assert "workspace" in lib.mla_last_error().decode()
    assert call(ctypes.byref(d), sc=FAKE) == L.ERR_INVALID_ARGUMENT   # scales for a bf16 cache
    d8 = _dims(L, cache_dtype=L.FP8_E4M3)
    assert call(ctypes.byref(d8)) == L.ERR_INVALID_ARGUMENT            # fp8 without scales
    bad = _dims(L, d_rope=63)
    assert call(ctypes.byref(bad)) == L.ERR_INVALID_ARGUMENT
    bad = _dims(L, act_dtype=L.FP8_E4M3)
    assert call(ctypes.byref(bad)) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), batch=0) == L.OK                       # nothing to do
    assert call(ctypes.byref(d), G=(1 << 20) + 1) == L.ERR_INVALID_ARGUMENT  # partition cap
    assert L.mla_decode_workspace_size(d, 4, 1, (1 << 20) + 1) == 0
    assert L.mla_decode_workspace_size(d, 4, 1, 1 << 20) > 0
    big = _dims(L, d_latent=1024, flags=L.FLAG_GENERIC_DECODE)
    ws_big = L.mla_decode_workspace_size(big, 4, 1, 8)
    assert lib.mla_decode(ctypes.byref(big), FAKE, 4, 1, FAKE, None, FAKE, 16, FAKE, 8, FAKE,
                          ws_big, None) == L.ERR_UNSUPPORTED


def test_workspace_size_closed_form(L):
    d = _dims(L)
    B, n_q, G, H, dc = 64, 1, 256, 128, 512
    slots = B + G
    o = slots * n_q * H * dc * 2          # partials are stored in the bf16 activation dtype
    lse = slots * n_q * H * 4
    up = lambda x: (x + 255) // 256 * 256
    tab = B * 2 * 4                       # first slot and piece count per sequence
    want = up(up(up(o) + lse) + tab)
    assert L.mla_decode_workspace_size(d, B, n_q, G) == want
    assert L.mla_decode_workspace_size(d, B, 0, G) == 0


def test_other_entry_points_validate(L):
    lib = L.lib()
    d = _dims(L)
    assert lib.mla_decode_combine(ctypes.byref(d), FAKE, 10, 4, 1, FAKE, 8, FAKE, None, None) \
        == L.ERR_WORKSPACE_TOO_SMALL
    assert lib.mla_decode_combine(ctypes.byref(d), None, 10, 4, 1, FAKE, 8, FAKE, None, None) \
        == L.ERR_INVALID_ARGUMENT
    assert lib.mla_decode_combine(ctypes.byref(d), FAKE, 1 << 40, 4, 1, FAKE, (1 << 20) + 1, FAKE,
                                  None, None) == L.ERR_INVALID_ARGUMENT
    assert lib.mla_out_proj(ctypes.byref(d), FAKE, -1, FAKE, FAKE, None) == L.ERR_INVALID_ARGUMENT
    assert lib.mla_out_proj(ctypes.byref(d), None, 4, FAKE, FAKE, None) == L.ERR_INVALID_ARGUMENT
    assert lib.mla_out_proj(ctypes.byref(d), FAKE, 0, FAKE, FAKE, None) == L.OK
    ap = lambda dims, T=4, dm=7168, sc=None, ws=FAKE, wsb=1 << 30: lib.mla_cache_append(
        dims, FAKE, T, dm, FAKE, FAKE, FAKE, FAKE, FAKE, 16, FAKE, sc, ws, wsb, None)
    assert ap(ctypes.byref(d), sc=FAKE) == L.ERR_INVALID_ARGUMENT           # scales on bf16
    need = L.mla_cache_append_workspace_size(d, 4, 7168)
    assert need > 0
    assert ap(ctypes.byref(d), wsb=need - 1) == L.ERR_WORKSPACE_TOO_SMALL
    assert ap(ctypes.byref(d), ws=None) == L.ERR_WORKSPACE_TOO_SMALL
    f32 = _dims(L, d_latent=100, act_dtype=L.FP32, cache_dtype=L.FP32)       # VALU path
    assert L.mla_cache_append_workspace_size(f32, 4, 64) == 0
    assert ap(ctypes.byref(f32), dm=64, ws=None, wsb=0) == L.ERR_UNSUPPORTED  # RoPE straddles tiles
    assert ap(ctypes.byref(d), T=0) == L.OK


def test_combine_out_proj_validates(L):
    lib = L.lib()
    d = _dims(L)
    ws = L.mla_decode_workspace_size(d, 4, 1, 8)
    call = lambda dims, ws_ptr=FAKE, ws_bytes=ws, w=FAKE, out=FAKE, u=None, G=8: \
        lib.mla_decode_combine_out_proj(dims, ws_ptr, ws_bytes, 4, 1, FAKE, G, w, out, u, None, None)
    assert call(None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), ws_ptr=None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), out=None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), ws_bytes=ws - 1) == L.ERR_WORKSPACE_TOO_SMALL
    assert call(ctypes.byref(d), G=(1 << 20) + 1) == L.ERR_INVALID_ARGUMENT
    odd = _dims(L, d_v=100)  # no fused kernel for d_v % 32 != 0, and no u_out to fall back on
    ws_odd = L.mla_decode_workspace_size(odd, 4, 1, 8)
    assert call(ctypes.byref(odd), ws_bytes=ws_odd) == L.ERR_UNSUPPORTED
    assert "u_out" in lib.mla_last_error().decode()


def test_query_absorb_validates(L):
    lib = L.lib()
    d = _dims(L)
    call = lambda dims, q=FAKE, pos=FAKE, w=FAKE, out=FAKE * 4, rows=2: \
        lib.mla_query_absorb(dims, q, pos, w, out, rows, None)
    assert call(None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), q=None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), pos=None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), w=None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), out=None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), rows=-1) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), rows=0) == L.OK          # nothing to do, nothing touched
    assert call(ctypes.byref(d), q=FAKE + 1) == L.ERR_INVALID_ARGUMENT  # misaligned bf16
    # q_out overlapping q_in
    assert call(ctypes.byref(d), out=FAKE + 256) == L.ERR_INVALID_ARGUMENT
    assert "overlap" in lib.mla_last_error().decode()
    no_nope = _dims(L, d_nope=0, softmax_scale=0.1)
    assert call(ctypes.byref(no_nope)) == L.ERR_INVALID_ARGUMENT


def test_append_query_absorb_validates_both_halves(L):
    """The one-call form rejects what either of its two calls rejects, before
    launching anything, and does nothing when both halves are empty."""
    lib = L.lib()
    d = _dims(L)
    need = L.mla_cache_append_workspace_size(d, 4, 7168)
    call = lambda T=4, sc=None, ws=FAKE, wsb=need, q=FAKE * 64, out=FAKE * 128, rows=2: \
        lib.mla_cache_append_query_absorb(ctypes.byref(d), FAKE, T, 7168, FAKE, FAKE, FAKE, FAKE, FAKE, 16,
                                          FAKE, sc, ws, wsb, q, FAKE, FAKE, out, rows, None)
    assert call(sc=FAKE) == L.ERR_INVALID_ARGUMENT                 # the append half: scales on bf16
    assert call(wsb=need - 1) == L.ERR_WORKSPACE_TOO_SMALL
    assert call(T=-1) == L.ERR_INVALID_ARGUMENT
    assert call(rows=-1) == L.ERR_INVALID_ARGUMENT                 # the query half
    assert call(q=None) == L.ERR_INVALID_ARGUMENT
    assert call(out=FAKE * 64 + 256) == L.ERR_INVALID_ARGUMENT      # q_out overlapping q_in
    assert "overlap" in lib.mla_last_error().decode()
    assert call(T=0, rows=0) == L.OK
    assert call(T=0, rows=-1) == L.ERR_INVALID_ARGUMENT


def test_linear_validates_and_sizes_its_workspace(L):
    lib = L.lib()
    d = _dims(L)
    # the weight-streaming shapes of the decode step's neighbours: W^DQ and W^O
    # split k (fp32 partials in the workspace), the wide W^UQ|W^QR does not
    assert L.mla_linear_workspace_size(d, 64, 1536, 7168) == 7 * 64 * 1536 * 4
    assert L.mla_linear_workspace_size(d, 64, 7168, 16384) == 4 * 64 * 7168 * 4
    assert L.mla_linear_workspace_size(d, 64, 128 * 192, 1536) == 0
    assert L.mla_linear_workspace_size(d, 64, 100, 7168) == 0          # n % 32: VALU form
    assert L.mla_linear_workspace_size(d, 64, 128, 7000) == 0          # k % 512: VALU form
    assert L.mla_linear_workspace_size(_dims(L, act_dtype=L.FP32), 64, 1536, 7168) == 0
    assert L.mla_linear_workspace_size(d, -1, 64, 512) == 0
    X, W, Y = FAKE, FAKE * 64, FAKE * 128
    ws = L.mla_linear_workspace_size(d, 64, 1536, 7168)
    call = lambda dims, x=X, rows=64, k=7168, w=W, n=1536, y=Y, wsp=FAKE * 256, wsb=ws: \
        lib.mla_linear(dims, x, rows, k, w, n, y, wsp, wsb, None)
    assert call(None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), x=None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), w=None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), y=None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), rows=-1) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), k=0) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), n=0) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), rows=0) == L.OK
    assert call(ctypes.byref(d), x=X + 1) == L.ERR_INVALID_ARGUMENT       # misaligned bf16
    assert call(ctypes.byref(d), y=X + 64) == L.ERR_INVALID_ARGUMENT      # y overlaps x
    assert "overlap" in lib.mla_last_error().decode()
    assert call(ctypes.byref(d), wsb=ws - 1) == L.ERR_WORKSPACE_TOO_SMALL
    assert call(ctypes.byref(d), wsp=None) == L.ERR_WORKSPACE_TOO_SMALL


def test_prefill_validates(L):
    """mla_prefill rejects bad lengths and pointers before launching anything,
    including a cached length whose expanded keys would pass 2 GiB per head."""
    lib = L.lib()
    d = _dims(L)
    call = lambda dims, n=4, seq=100, q=FAKE, sc=None, ws_bytes=1 << 40: lib.mla_prefill(
        dims, q, n, FAKE, sc, FAKE, seq, FAKE, FAKE, FAKE * 2, FAKE, ws_bytes, None)
    assert call(None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), n=-1) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), n=5, seq=4) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), n=0, seq=4) == L.OK       # nothing to do
    assert call(ctypes.byref(d), q=None) == L.ERR_INVALID_ARGUMENT
    assert call(ctypes.byref(d), sc=FAKE) == L.ERR_INVALID_ARGUMENT  # scales for a bf16 cache
    limit = 1 << 23
    assert call(ctypes.byref(d), seq=limit) == L.ERR_INVALID_ARGUMENT
    assert "seq_len" in lib.mla_last_error().decode()
    assert call(ctypes.byref(d), ws_bytes=16) == L.ERR_WORKSPACE_TOO_SMALL
    odd = _dims(L, num_heads=64)
    assert call(ctypes.byref(odd)) == L.ERR_UNSUPPORTED

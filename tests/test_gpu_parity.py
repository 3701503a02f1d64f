"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (from the stated tolerances of the method): bf16 inputs with fp32
accumulation -> relative L2 <= 1e-2 and max-abs <= 2e-2; fp8-e4m3 caches ->
relative L2 <= 5e-2; fp32 workloads are additionally held to 1e-5 relative L2.
Index and placement work (page tables, slots) is checked bit for bit.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import mla_workloads as W
from oracle import mla_oracle as O
from tests.cases import (DT, FP8, DecodeCase, append_workspace, compare_sampled, dims_of, fp8_score_bound,
                         max_abs, rel_l2, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_decode_amd as M
    M.lib()  # raises if the HIP library is missing: no fallback exists
    return M


def _t(x, dtype, dev="cuda"):
    return torch.as_tensor(np.asarray(x)).to(dev).to(dtype)


# --------------------------------------------------------------------------
# tiny fp32 workload, end to end: append -> decode -> combine -> out_proj
# --------------------------------------------------------------------------
def test_tiny_end_to_end_fp32():
    import mla_latent_kv_decode_amd as M
    cfg = W.CONFIGS["tiny"]
    d = cfg.dims
    dm, H = d.d_model, d.num_heads
    w_dkv = W.weight(d.d_latent, dm, 1).numpy()
    w_kr = W.weight(d.d_rope, dm, 2).numpy()
    w_q = W.weight(H * (d.d_nope + d.d_rope), dm, 3).numpy()
    w_uk = W.normal((H, d.d_nope, d.d_latent), 4, std=1 / math.sqrt(d.d_latent)).numpy()
    w_uv = W.normal((H, d.d_v, d.d_latent), 5, std=1 / math.sqrt(d.d_latent)).numpy()
    h = W.normal((65, dm), 6).numpy()          # positions 0..63 prior, 64 = query token
    pos = np.arange(65, dtype=np.int32)
    # oracle
    rows = O.kv_rows(h, w_dkv, w_kr, pos)
    q, _, _ = O.query_from_hidden(h[64], w_q, w_uk, 64, H, d.d_nope, d.d_rope)
    scale = O.softmax_scale(d.d_nope, d.d_rope)
    u_ref, lse_ref = O.attend_absorbed(q[None], rows, 1, d.d_latent, scale)
    o_ref = O.out_proj(u_ref, w_uv)
    # GPU: contiguous cache = identity page table over 2 blocks of 64
    dims = dims_of(cfg)
    # query: projection W^Q h, absorption and q-RoPE, all on the GPU
    q_full = torch.empty(1, H, d.d_nope + d.d_rope, device="cuda")
    M.mla_linear(dims, _t(h[64:65], torch.float32), _t(w_q, torch.float32), q_full)
    q_gpu = torch.empty(1, H, d.row, device="cuda")
    M.mla_query_absorb(dims, q_full, torch.tensor([64], dtype=torch.int32, device="cuda"),
                       _t(w_uk, torch.float32), q_gpu)
    cache = torch.full((2, 64, d.row), float("nan"), device="cuda")
    table = torch.tensor([[0, 1]], dtype=torch.int32, device="cuda")
    M.mla_cache_append(dims, _t(h, torch.float32), _t(w_dkv, torch.float32),
                       _t(w_kr, torch.float32), torch.zeros(65, dtype=torch.int32, device="cuda"),
                       _t(pos, torch.int32), table, cache)
    lens = torch.tensor([65], dtype=torch.int32, device="cuda")
    ws = torch.empty(M.mla_decode_workspace_size(dims, 1, 1, 0), dtype=torch.uint8, device="cuda")
    qd = q_gpu.view(1, 1, H, d.row)
    M.mla_decode(dims, qd, cache, None, table, lens, ws)
    u = torch.empty(1, 1, H, d.d_latent, device="cuda")
    lse = torch.empty(1, 1, H, device="cuda")
    M.mla_decode_combine(dims, ws, lens, u, lse)
    o = torch.empty(1, H, d.d_v, device="cuda")
    M.mla_out_proj(dims, u.view(1, H, d.d_latent), _t(w_uv, torch.float32), o)
    torch.cuda.synchronize()
    got_rows = cache.view(-1, d.row)[:65].cpu().numpy().astype(np.float64)
    assert rel_l2(got_rows, rows) <= 1e-6
    assert rel_l2(q_gpu.cpu().numpy()[0].astype(np.float64), q) <= 1e-6
    assert rel_l2(u.cpu().numpy()[0], u_ref) <= 1e-5
    assert max_abs(lse.cpu().numpy()[0], lse_ref) <= 1e-5
    assert rel_l2(o.cpu().numpy(), o_ref) <= 1e-5
    assert max_abs(o.cpu().numpy(), o_ref) <= 2e-2
    assert torch.isnan(cache.view(-1, d.row)[65:]).all(), "slots past the sequence were written"


# --------------------------------------------------------------------------
# dense layers (mla_linear): the low-rank query path and W^O
# --------------------------------------------------------------------------
LINEAR_SHAPES = [   # (rows, n, k)
    (64, 1536, 7168),       # W^DQ at B = 64: k split in 7 ranges, partials summed in order
    (64, 128 * 192, 1536),  # [W^UQ_i ; W^QR_i] head by head: one k range, direct bf16 store
    (64, 7168, 16384),      # W^O: k split in 4, two column blocks per workgroup
    (1, 32, 512),           # one row, one stage, one workgroup
    (33, 96, 1536),         # two row blocks, the second ragged; three stages
    (100, 64, 8192),        # two row tiles, the second ragged; k split in 4
    (7, 64, 1000),          # k % 512 != 0: the VALU form in bf16
    (150, 192, 1024),       # three row tiles x three column tiles: 9 workgroups over 8 XCDs
]


def _linear(M, dims, x, w, y):
    rows, k = x.shape[0], x.shape[-1]
    nws = M.mla_linear_workspace_size(dims, rows, w.shape[0], k)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    M.mla_linear(dims, x, w, y, ws)


@pytest.mark.parametrize("shape", LINEAR_SHAPES)
def test_linear_bf16_matches_oracle(shape):
    import mla_latent_kv_decode_amd as M
    rows, n, k = shape
    dims = dims_of(W.CONFIGS["v3"])
    x = W.normal((rows, k), 200 + rows, device="cuda", dtype=torch.bfloat16)
    w = W.weight(n, k, 300 + n, dtype=torch.bfloat16, device="cuda")
    y = torch.full((rows, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    _linear(M, dims, x, w, y)
    torch.cuda.synchronize()
    got, ref = to_f64(y), O.linear(to_f64(x), to_f64(w))
    assert np.all(np.isfinite(got))
    assert rel_l2(got, ref) <= 1e-2 and max_abs(got, ref) <= 2e-2
    # fp32 accumulation, one round-to-nearest-even bf16 store
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-4)


def test_linear_generic_fp32_tight():
    import mla_latent_kv_decode_amd as M
    dims = dims_of(W.CONFIGS["tiny"])
    x = W.normal((7, 300), 210, device="cuda")
    w = W.weight(96, 300, 211, device="cuda")
    y = torch.empty(7, 96, device="cuda")
    _linear(M, dims, x, w, y)
    torch.cuda.synchronize()
    assert rel_l2(y.cpu().numpy().astype(np.float64), O.linear(to_f64(x), to_f64(w))) <= 1e-6


def test_linear_mfma_agrees_with_generic_and_is_deterministic():
    import mla_latent_kv_decode_amd as M
    x = W.normal((40, 4096), 220, device="cuda", dtype=torch.bfloat16)
    w = W.weight(320, 4096, 221, dtype=torch.bfloat16, device="cuda")
    outs = []
    for flags in (0, 0, M.FLAG_GENERIC_DECODE):
        y = torch.empty(40, 320, dtype=torch.bfloat16, device="cuda")  # k split in 4
        _linear(M, dims_of(W.CONFIGS["v3"], flags), x, w, y)
        outs.append(y)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "the split-k sum order is fixed"
    # same products summed in another order: at most a bf16 rounding apart
    assert rel_l2(to_f64(outs[0]), to_f64(outs[2])) <= 2e-3


def test_query_path_low_rank_v3():
    """The decoding section's step 2 and 3 at B = 64 on the GPU: c^Q = W^DQ h,
    [q^C ; q^R] per head from the head-by-head stacked [W^UQ_i ; W^QR_i] (one
    call), then absorption and q-RoPE."""
    import mla_latent_kv_decode_amd as M
    d, rows = W.V3, 64
    H, dn, dr, dq = d.num_heads, d.d_nope, d.d_rope, d.d_q
    dims = dims_of(W.CONFIGS["v3"])
    bf = torch.bfloat16
    h = W.normal((rows, d.d_model), 230, device="cuda", dtype=bf)
    w_dq = W.weight(dq, d.d_model, 231, dtype=bf, device="cuda")
    w_uq = W.weight(H * dn, dq, 232, dtype=bf, device="cuda")
    w_qr = W.weight(H * dr, dq, 233, dtype=bf, device="cuda")
    w_uk = W.normal((H, dn, d.d_latent), 234, std=1 / math.sqrt(d.d_latent), device="cuda", dtype=bf)
    pos = np.random.default_rng(235).integers(0, 131072, size=rows).astype(np.int32)
    # weight layout, once per model: rows of head i are [W^UQ_i ; W^QR_i]
    w_uqr = torch.cat([w_uq.view(H, dn, dq), w_qr.view(H, dr, dq)], 1).reshape(H * (dn + dr), dq).contiguous()
    c_q = torch.empty(rows, dq, dtype=bf, device="cuda")
    q_in = torch.empty(rows, H, dn + dr, dtype=bf, device="cuda")
    q = torch.empty(rows, H, d.row, dtype=bf, device="cuda")
    _linear(M, dims, h, w_dq, c_q)
    _linear(M, dims, c_q, w_uqr, q_in)
    M.mla_query_absorb(dims, q_in, torch.from_numpy(pos).cuda(), w_uk, q)
    torch.cuda.synchronize()
    # each stage against the oracle from the stored bf16 values it was given
    # (one bf16 rounding each: the element bar holds per stage) ...
    f = {k: to_f64(t) for k, t in dict(h=h, w_dq=w_dq, w_uq=w_uq, w_qr=w_qr, w_uk=w_uk,
                                       c_q=c_q, q_in=q_in, q=q).items()}
    stages = [(f["c_q"], O.linear(f["h"], f["w_dq"])),
              (f["q_in"][..., :dn], O.linear(f["c_q"], f["w_uq"]).reshape(rows, H, dn)),
              (f["q_in"][..., dn:], O.linear(f["c_q"], f["w_qr"]).reshape(rows, H, dr)),
              (f["q"], O.absorb_query(f["q_in"][..., :dn], f["q_in"][..., dn:], f["w_uk"], pos))]
    for got, ref in stages:
        assert rel_l2(got, ref) <= 1e-2 and max_abs(got, ref) <= 2e-2
    # ... and the whole path against the page's unrounded form (three bf16
    # roundings on the way: c^Q, q_in, q)
    q_c, q_r = O.query_lowrank(f["h"], f["w_dq"], f["w_uq"], f["w_qr"], H, dn, dr)
    assert rel_l2(f["q"], O.absorb_query(q_c, q_r, f["w_uk"], pos)) <= 1e-2


def test_output_projection_v3():
    """The module's last step at B = 64: the per-head outputs laid end to end,
    then W^O [d_model, H d_v]."""
    import mla_latent_kv_decode_amd as M
    d, rows = W.V3, 64
    dims = dims_of(W.CONFIGS["v3"])
    v = W.normal((rows, d.num_heads, d.d_v), 240, device="cuda", dtype=torch.bfloat16)
    w_o = W.weight(d.d_model, d.num_heads * d.d_v, 241, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(rows, d.d_model, dtype=torch.bfloat16, device="cuda")
    _linear(M, dims, v.view(rows, -1), w_o, out)
    torch.cuda.synchronize()
    ref = O.output_projection(to_f64(v), to_f64(w_o))
    assert rel_l2(to_f64(out), ref) <= 1e-2 and max_abs(to_f64(out), ref) <= 2e-2


# --------------------------------------------------------------------------
# query absorption + q-RoPE (mla_query_absorb)
# --------------------------------------------------------------------------
def _query_case(H, d_nope, d_rope, d_latent, rows, seed, dtype):
    q_in = W.normal((rows, H, d_nope + d_rope), seed, device="cuda").to(dtype)
    w_uk = W.normal((H, d_nope, d_latent), seed + 1, std=1 / math.sqrt(d_latent), device="cuda").to(dtype)
    pos = np.random.default_rng(seed + 2).integers(0, 131072, size=rows).astype(np.int32)
    pos[0] = 0
    pos[-1] = 131071   # long-context angles: the fp64 angle matters here
    ref = O.absorb_query(to_f64(q_in[..., :d_nope]), to_f64(q_in[..., d_nope:]), to_f64(w_uk), pos)
    return q_in, w_uk, torch.from_numpy(pos).cuda(), ref


@pytest.mark.parametrize("rows", [1, 64, 70, 300, 512])  # 300: three row splits, the last ragged
def test_query_absorb_v3_bf16(rows):
    import mla_latent_kv_decode_amd as M
    d = W.V3
    dims = dims_of(W.CONFIGS["v3"])
    q_in, w_uk, pos, ref = _query_case(d.num_heads, d.d_nope, d.d_rope, d.d_latent, rows, 40 + rows,
                                       torch.bfloat16)
    out = torch.full((rows, d.num_heads, d.row), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.mla_query_absorb(dims, q_in, pos, w_uk, out)
    torch.cuda.synchronize()
    got = to_f64(out)
    assert np.all(np.isfinite(got))
    assert rel_l2(got, ref) <= 1e-2 and max_abs(got, ref) <= 2e-2
    # the rotation itself: bf16 in, fp32 arithmetic, one bf16 rounding out
    assert rel_l2(got[..., d.d_latent:], ref[..., d.d_latent:]) <= 4e-3


def test_query_absorb_mfma_rope_width_48():
    """d_R = 48: 24 rotation pairs, which do not divide the workgroup's 256
    threads (each thread's pairs have different frequencies)."""
    import mla_latent_kv_decode_amd as M
    H, dn, dr, dl, rows = 16, 128, 48, 512, 40
    q_in, w_uk, pos, ref = _query_case(H, dn, dr, dl, rows, 90, torch.bfloat16)
    outs = []
    for flags in (0, M.FLAG_GENERIC_DECODE):
        dims = M.make_dims(H, dl, dr, dn, 128, 64, M.BF16, M.BF16, flags=flags)
        out = torch.full((rows, H, dl + dr), float("nan"), dtype=torch.bfloat16, device="cuda")
        M.mla_query_absorb(dims, q_in, pos, w_uk, out)
        outs.append(to_f64(out))
    torch.cuda.synchronize()
    got = outs[0]
    assert np.all(np.isfinite(got))
    assert rel_l2(got, ref) <= 1e-2 and max_abs(got, ref) <= 2e-2
    assert rel_l2(got[..., dl:], ref[..., dl:]) <= 4e-3
    assert rel_l2(got[..., dl:], outs[1][..., dl:]) <= 1e-4


def test_query_absorb_generic_fp32_tight():
    import mla_latent_kv_decode_amd as M
    d = W.TINY
    dims = dims_of(W.CONFIGS["tiny"])
    q_in, w_uk, pos, ref = _query_case(d.num_heads, d.d_nope, d.d_rope, d.d_latent, 37, 60, torch.float32)
    out = torch.empty(37, d.num_heads, d.row, device="cuda")
    M.mla_query_absorb(dims, q_in, pos, w_uk, out)
    torch.cuda.synchronize()
    assert rel_l2(out.cpu().numpy().astype(np.float64), ref) <= 1e-6


def test_query_absorb_mfma_agrees_with_generic():
    import mla_latent_kv_decode_amd as M
    d = W.V3
    q_in, w_uk, pos, _ = _query_case(d.num_heads, d.d_nope, d.d_rope, d.d_latent, 50, 70, torch.bfloat16)
    outs = []
    for flags in (0, M.FLAG_GENERIC_DECODE):
        out = torch.empty(50, d.num_heads, d.row, dtype=torch.bfloat16, device="cuda")
        M.mla_query_absorb(dims_of(W.CONFIGS["v3"], flags), q_in, pos, w_uk, out)
        outs.append(to_f64(out))
    torch.cuda.synchronize()
    # same products, summed in another order: at most a bf16 rounding apart
    assert rel_l2(outs[0], outs[1]) <= 2e-3
    # the RoPE part is the same arithmetic on both paths (up to fma contraction)
    assert rel_l2(outs[0][..., d.d_latent:], outs[1][..., d.d_latent:]) <= 1e-4


# --------------------------------------------------------------------------
# append: placement is bit-exact (identity projection), values match the oracle
# --------------------------------------------------------------------------
@pytest.mark.parametrize("cache_dtype", ["fp32", "bf16", "fp8", "fp8p2"])
def test_append_identity_projection_bit_exact(cache_dtype):
    import mla_latent_kv_decode_amd as M
    d_c, d_r, bs = 512, 64, 64
    D = d_c + d_r
    act = "fp32" if cache_dtype == "fp32" else "bf16"
    tdt = torch.float32 if act == "fp32" else torch.bfloat16
    rng = np.random.default_rng(7)
    lens = np.array([130, 64, 300], np.int32)
    table, nblk = W.page_table(lens, bs, seed=7, guard_blocks=2)
    # 40 tokens at distinct positions; several at position 0
    toks = []
    for b, L in enumerate(lens):
        for p in rng.choice(L, size=13 + b, replace=False):
            toks.append((b, int(p)))
    toks += [(0, 0), (2, 0)]
    toks = list(dict.fromkeys(toks))
    seq_ids = np.array([t[0] for t in toks], np.int32)
    positions = np.array([t[1] for t in toks], np.int32)
    T = len(toks)
    h = W.normal((T, D), 8).to(tdt)
    h64 = to_f64(h)
    w_dkv = np.concatenate([np.eye(d_c), np.zeros((d_c, d_r))], 1)
    w_kr = np.concatenate([np.zeros((d_r, d_c)), np.eye(d_r)], 1)
    cfg = W.Config("ident", W.Dims(1, d_c, d_r, 128, 128, D), 3, 1, 0, cache_dtype, act, None)
    dims = dims_of(cfg)
    if cache_dtype in FP8:
        cache = torch.full((nblk, bs, D), 0x7F, dtype=torch.uint8, device="cuda")
        scales = torch.full((nblk, bs, 5), float("nan"), device="cuda")
    else:
        cache = torch.full((nblk, bs, D), float("nan"), dtype=tdt, device="cuda")
        scales = None
    before = cache.clone()
    M.mla_cache_append(dims, h.cuda(), _t(w_dkv, tdt), _t(w_kr, tdt), _t(seq_ids, torch.int32),
                       _t(positions, torch.int32), _t(table, torch.int32), cache, scales,
                       append_workspace(dims, T, D))
    torch.cuda.synchronize()
    pool = {"dtype": cache_dtype, "data": None}
    written = np.zeros((nblk, bs), bool)
    for i in range(T):
        blk, off = O.slot_of(table, int(seq_ids[i]), int(positions[i]), bs)
        written[blk, off] = True
        want = O.kv_rows(h64[i:i + 1], w_dkv, w_kr, positions[i:i + 1])[0].astype(np.float32)
        if cache_dtype in FP8:
            codes, sc = O.quantize_fp8_rows(want[None], pow2_scales=cache_dtype == "fp8p2")
            codes, sc = codes[0], sc[0]
            got_c = cache[blk, off].cpu().numpy()
            got_s = scales[blk, off].cpu().numpy()
            # latent tiles: exact inputs -> the same fp32 decisions -> identical bytes
            assert np.array_equal(got_c[:d_c], codes[:d_c]), (i, positions[i])
            assert np.array_equal(got_s[:4], sc[:4])
            if positions[i] == 0:
                assert np.array_equal(got_c, codes) and np.array_equal(got_s, sc)
            dec = O.dequantize_fp8_rows(got_c[None], got_s[None])[0]
            assert rel_l2(dec[d_c:], want[d_c:]) <= 5e-2
        else:
            got = to_f64(cache[blk, off])
            assert np.array_equal(got[:d_c], h64[i, :d_c]), "latent part must be copied exactly"
            if positions[i] == 0:
                assert np.array_equal(got, h64[i]), "RoPE at position 0 is the identity"
            # rotated part: fp32 rotation on the device vs float64 here
            if cache_dtype == "fp32":
                bound = 1e-6 * np.maximum(np.abs(want[d_c:]), 1.0)
            else:
                bound = 2.0 ** -8 * np.maximum(np.abs(want[d_c:]), 0.01)
            assert np.all(np.abs(got[d_c:] - want[d_c:]) <= bound)
    untouched = torch.from_numpy(~written).cuda()
    a, b = cache[untouched], before[untouched]
    if cache_dtype in FP8:
        assert torch.equal(a, b)
        assert torch.isnan(scales[untouched]).all()
    else:
        assert torch.equal(a.view(torch.int16 if act == "bf16" else torch.int32),
                           b.view(torch.int16 if act == "bf16" else torch.int32))


def test_append_v3_random_weights_bf16():
    import mla_latent_kv_decode_amd as M
    d = W.V3
    T = 64
    h = W.normal((T, d.d_model), 11).to(torch.bfloat16)
    w_dkv = W.weight(d.d_latent, d.d_model, 12, dtype=torch.bfloat16)
    w_kr = W.weight(d.d_rope, d.d_model, 13, dtype=torch.bfloat16)
    lens = np.full(T, 4096, np.int32)
    table, nblk = W.page_table(lens, 64, seed=5)
    positions = np.full(T, 4095, np.int32)
    seq_ids = np.arange(T, dtype=np.int32)
    cfg = W.CONFIGS["v3"]
    dims = dims_of(cfg)
    cache = torch.zeros((nblk, 64, d.row), dtype=torch.bfloat16, device="cuda")
    M.mla_cache_append(dims, h.cuda(), w_dkv.cuda(), w_kr.cuda(), _t(seq_ids, torch.int32),
                       _t(positions, torch.int32), _t(table, torch.int32), cache,
                       workspace=append_workspace(dims, T, d.d_model))
    torch.cuda.synchronize()
    want = O.kv_rows(to_f64(h), to_f64(w_dkv), to_f64(w_kr), positions)
    got = np.stack([to_f64(cache[table[b, 63], 63]) for b in range(T)])
    assert rel_l2(got, want) <= 4e-3
    assert max_abs(got, want) <= 2e-2


@pytest.mark.parametrize("T", [1, 33, 512])
def test_append_v3_fp8_random_weights(T):
    """fp8 cache: the device quantises its own fp32 rows; compare the decoded
    values with the oracle's rows (fp8 bar) and check every code's tile
    scale is amax/448 of what was stored."""
    import mla_latent_kv_decode_amd as M
    d = W.V3
    h = W.normal((T, d.d_model), 14).to(torch.bfloat16)
    w_dkv = W.weight(d.d_latent, d.d_model, 15, dtype=torch.bfloat16)
    w_kr = W.weight(d.d_rope, d.d_model, 16, dtype=torch.bfloat16)
    lens = np.full(T, 300, np.int32)
    table, nblk = W.page_table(lens, 64, seed=6, guard_blocks=1)
    positions = np.random.default_rng(T).integers(0, 300, T).astype(np.int32)
    seq_ids = np.arange(T, dtype=np.int32)
    dims = dims_of(W.CONFIGS["fp8"])
    cache = torch.zeros((nblk, 64, d.row), dtype=torch.uint8, device="cuda")
    scales = torch.zeros((nblk, 64, 5), device="cuda")
    M.mla_cache_append(dims, h.cuda(), w_dkv.cuda(), w_kr.cuda(), _t(seq_ids, torch.int32),
                       _t(positions, torch.int32), _t(table, torch.int32), cache, scales,
                       append_workspace(dims, T, d.d_model))
    torch.cuda.synchronize()
    want = O.kv_rows(to_f64(h), to_f64(w_dkv), to_f64(w_kr), positions)
    got = []
    for i in range(T):
        blk, off = O.slot_of(table, i, int(positions[i]), 64)
        c, sc = cache[blk, off].cpu().numpy(), scales[blk, off].cpu().numpy()
        dec = O.dequantize_fp8_rows(c[None], sc[None])[0]
        for k, (lo, hi) in enumerate(O.fp8_tiles(d.row)):
            assert np.max(np.abs(c[lo:hi] & 0x7F)) == 0x7E  # the tile max encodes to 448
        got.append(dec)
    assert rel_l2(np.stack(got), want) <= 5e-2


@pytest.mark.parametrize("cache_dtype,act,flags,T,rows", [
    ("bf16", "bf16", 0, 64, 64),   # one shared launch
    ("fp8", "bf16", 0, 33, 70),    # 165 append units: the last workgroup's second half is idle
    ("fp32", "bf16", 0, 1, 300),
    ("bf16", "bf16", 0, 0, 5),     # no tokens: the query half alone
    ("fp8", "bf16", 0, 7, 0),      # no query rows: the append half alone
    ("fp8p2", "bf16", 0, 33, 70),  # power-of-two tile scales
    ("fp32", "fp32", 0, 5, 3),     # VALU forms, two launches
    ("bf16", "bf16", 1, 9, 9),     # VALU query form beside the matrix-core append
])
def test_append_query_absorb_one_call_matches_two_calls(cache_dtype, act, flags, T, rows):
    """mla_cache_append_query_absorb writes the cache rows, fp8 scales and
    absorbed queries of mla_cache_append followed by mla_query_absorb, bit for
    bit (those two calls are held to the oracle above)."""
    import mla_latent_kv_decode_amd as M
    d = W.V3
    cfg = dataclasses.replace(W.CONFIGS["v3"], cache_dtype=cache_dtype, act_dtype=act)
    dims = dims_of(cfg, flags)
    adt = torch.bfloat16 if act == "bf16" else torch.float32
    cdt = {"bf16": torch.bfloat16, "fp32": torch.float32, "fp8": torch.uint8, "fp8p2": torch.uint8}[cache_dtype]
    h = W.normal((T, d.d_model), 70 + T, device="cuda").to(adt)
    w_dkv = W.weight(d.d_latent, d.d_model, 71, dtype=adt, device="cuda")
    w_kr = W.weight(d.d_rope, d.d_model, 72, dtype=adt, device="cuda")
    lens = np.full(max(T, 1), 300, np.int32)
    table, nblk = W.page_table(lens, 64, seed=7, guard_blocks=1)
    positions = _t(np.random.default_rng(T).integers(0, 300, T).astype(np.int32), torch.int32)
    seq_ids = torch.arange(T, dtype=torch.int32, device="cuda")
    table_t = _t(table, torch.int32)
    q_in = W.normal((rows, d.num_heads, d.d_nope + d.d_rope), 73 + rows, device="cuda").to(adt)
    w_uk = W.normal((d.num_heads, d.d_nope, d.d_latent), 74, std=1 / math.sqrt(d.d_latent),
                    device="cuda").to(adt)
    q_pos = _t(np.random.default_rng(rows).integers(0, 131072, rows).astype(np.int32), torch.int32)
    ws = append_workspace(dims, max(T, 1), d.d_model)

    def run(one_call):
        cache = torch.zeros((nblk, 64, d.row), dtype=cdt, device="cuda")
        scales = torch.zeros((nblk, 64, 5), device="cuda") if cache_dtype in FP8 else None
        q_out = torch.full((rows, d.num_heads, d.row), float("nan"), dtype=adt, device="cuda")
        if one_call:
            M.mla_cache_append_query_absorb(dims, h, w_dkv, w_kr, seq_ids, positions, table_t, cache, scales,
                                            ws, q_in, q_pos, w_uk, q_out)
        else:
            M.mla_cache_append(dims, h, w_dkv, w_kr, seq_ids, positions, table_t, cache, scales, ws)
            M.mla_query_absorb(dims, q_in, q_pos, w_uk, q_out)
        torch.cuda.synchronize()
        out = [cache.view(torch.uint8), q_out.view(torch.uint8)]
        return out + ([scales.view(torch.uint8)] if scales is not None else [])

    two, one = run(False), run(True)
    for a, b in zip(two, one):
        assert torch.equal(a, b)
    assert torch.isfinite(one[1].view(adt).float()).all()
    if T:
        assert bool(one[0].any())


# --------------------------------------------------------------------------
# decode + combine
# --------------------------------------------------------------------------
SMALL = [
    ("bf16", 1, W.scaled(W.CONFIGS["v3"], batch=3, seq_len=333)),
    ("bf16", 2, W.scaled(W.CONFIGS["ragged"], batch=5, len_lo=2, len_hi=400)),
    ("fp8", 1, W.scaled(W.CONFIGS["fp8"], batch=3, seq_len=200)),
]


@pytest.mark.parametrize("G", [1, 5, 37])
@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_decode_generic_small(idx, G):
    import mla_latent_kv_decode_amd as M
    _, _, cfg = SMALL[idx]
    case = DecodeCase(cfg)
    u, lse = case.run(flags=M.FLAG_GENERIC_DECODE, G=G)
    # fp8 caches are held to relative L2 only (the stated fp8 tolerance)
    fp8 = cfg.cache_dtype == "fp8"
    compare_sampled(case, u, lse, list(range(cfg.batch)), rel_bar=5e-2 if fp8 else 1e-2,
                    abs_bar=None if fp8 else 2e-2)


def test_decode_fp32_tight_and_partition_invariance():
    """fp32 queries and outputs over a bf16 cache: every partition count gives
    the oracle's result to fp32 accuracy (the LSE merge is exact up to rounding)."""
    import mla_latent_kv_decode_amd as M
    cfg = W.scaled(W.CONFIGS["ragged"], batch=4, len_lo=1, len_hi=700)
    case = DecodeCase(cfg, act="fp32")
    outs = []
    for G in [1, 3, 16, 200]:
        u, lse = case.run(flags=M.FLAG_GENERIC_DECODE, G=G)
        compare_sampled(case, u, lse, list(range(cfg.batch)), rel_bar=1e-5, abs_bar=1e-4,
                        lse_tol=1e-4)
        outs.append(u.cpu().numpy())
    for o in outs[1:]:
        assert rel_l2(o, outs[0]) <= 1e-6


def test_decode_page_table_permutation_is_bitwise_invariant():
    import mla_latent_kv_decode_amd as M
    cfg = W.scaled(W.CONFIGS["v3"], batch=2, seq_len=500)
    a = DecodeCase(cfg, shuffle=False, guard=0)
    # same logical rows, physical blocks permuted
    perm = np.random.default_rng(3).permutation(a.nblk)
    b_table = perm[a.table].astype(np.int32)
    b = DecodeCase(cfg, table=(b_table, a.nblk), guard=0)
    inv = torch.from_numpy(np.argsort(perm)).cuda()
    b.pool = a.pool.clone()
    b.pool[torch.from_numpy(perm).cuda()] = a.pool
    ua, la = a.run(G=7)
    ub, lb = b.run(G=7)
    assert torch.isfinite(ua.float()).all() and torch.isfinite(la).all()
    assert torch.equal(ua.view(torch.int16), ub.view(torch.int16))
    assert torch.equal(la, lb)
    compare_sampled(a, ua, la, [0, 1])


def test_out_proj_v3_bf16():
    import mla_latent_kv_decode_amd as M
    d = W.V3
    rows = 70
    u = W.normal((rows, d.num_heads, d.d_latent), 21).to(torch.bfloat16)
    w = W.normal((d.num_heads, d.d_v, d.d_latent), 22, std=1 / math.sqrt(d.d_latent)).to(torch.bfloat16)
    out = torch.empty(rows, d.num_heads, d.d_v, dtype=torch.bfloat16, device="cuda")
    M.mla_out_proj(dims_of(W.CONFIGS["v3"]), u.cuda(), w.cuda(), out)
    torch.cuda.synchronize()
    ref = O.out_proj(to_f64(u), to_f64(w))
    assert rel_l2(to_f64(out), ref) <= 4e-3
    assert max_abs(to_f64(out), ref) <= 2e-2


# --------------------------------------------------------------------------
# full-size workloads, default launch configuration
# --------------------------------------------------------------------------
TWO_GIB = 1 << 31


def _ragged_sample(case, n=16):
    """n sequences spread over the length range (every len-rank n-th), plus
    the sequence that owns the highest physical block, so that some compared
    sequence reads cache blocks at byte offsets past 2^31."""
    order = np.argsort(case.lens, kind="stable")
    pick = set(int(order[i]) for i in np.linspace(0, len(order) - 1, n).round().astype(int))
    owner = int(np.argwhere(case.table == case.table.max())[0, 0])
    pick.add(owner)
    return sorted(pick)


FULL = {"v3": lambda c: list(range(64)), "long": lambda c: [0, 1, 2, 3],
        "fp8": lambda c: list(range(0, 128, 4)), "fp8p2": lambda c: list(range(1, 128, 4)),
        "ragged": _ragged_sample}


@pytest.mark.parametrize("name", sorted(FULL))
def test_full_size(name):
    """Every config at its full size in the default launch configuration:
    all sequences of v3 and long, 32 of fp8 (either scale format), and 17 of
    ragged (lengths from the shortest to the longest, the 2.29 GB pool's last
    block included)."""
    cfg = W.CONFIGS[name]
    case = DecodeCase(cfg)
    ids = FULL[name](case)
    if name == "ragged":
        row_bytes = case.d.block_size * case.d.row * 2
        assert case.nblk * row_bytes > TWO_GIB
        hi = [b for b in ids if int(case.table[b].max()) * row_bytes >= TWO_GIB]
        assert hi, "no compared sequence reads past 2 GiB"
    u, lse = case.run()
    if cfg.cache_dtype in FP8:
        compare_sampled(case, u, lse, ids, rel_bar=5e-2, abs_bar=None)
    else:
        compare_sampled(case, u, lse, ids)
    assert torch.isfinite(u.float()).all() and torch.isfinite(lse).all()


def test_full_v3_benchmark_step():
    """The benchmark's step exactly as bench.py runs it at the full v3 shape
    (B = 64, L = 4096, default partitions): the one-call append + query
    absorption, the decode, the fused merge + W^UV.  The appended rows, the
    absorbed queries, u and o are each checked against the oracle, for all
    64 sequences."""
    import mla_latent_kv_decode_amd as M
    cfg = W.CONFIGS["v3"]
    case = DecodeCase(cfg)
    d = case.d
    dev = "cuda"
    B, n_q, H = cfg.batch, cfg.n_q, d.num_heads
    dims = dims_of(cfg)
    T = B * n_q
    h = W.normal((T, d.d_model), 61, device=dev, dtype=torch.bfloat16)
    w_dkv = W.weight(d.d_latent, d.d_model, 62, dtype=torch.bfloat16, device=dev)
    w_kr = W.weight(d.d_rope, d.d_model, 63, dtype=torch.bfloat16, device=dev)
    q_in = W.normal((B, n_q, H, d.d_nope + d.d_rope), 64, device=dev, dtype=torch.bfloat16)
    w_uk = W.normal((H, d.d_nope, d.d_latent), 65, std=1 / math.sqrt(d.d_latent), device=dev,
                    dtype=torch.bfloat16)
    w_uv = W.normal((H, d.d_v, d.d_latent), 66, std=1 / math.sqrt(d.d_latent), device=dev,
                    dtype=torch.bfloat16)
    seq_ids = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(n_q)
    positions = (case.lens_t.repeat_interleave(n_q) - n_q
                 + torch.arange(n_q, dtype=torch.int32, device=dev).repeat(B)).to(torch.int32)
    aws = append_workspace(dims, T, d.d_model)
    q = torch.empty(B, n_q, H, d.row, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(M.mla_decode_workspace_size(dims, B, n_q, 0), dtype=torch.uint8, device=dev)
    o = torch.full((T, H, d.d_v), float("nan"), dtype=torch.bfloat16, device=dev)
    u = torch.full((B, n_q, H, d.d_latent), float("nan"), dtype=torch.bfloat16, device=dev)
    pool0 = case.pool.clone()
    M.mla_cache_append_query_absorb(dims, h, w_dkv, w_kr, seq_ids, positions, case.table_t, case.pool,
                                    None, aws, q_in, positions, w_uk, q)
    M.mla_decode(dims, q, case.pool, None, case.table_t, case.lens_t, ws, 0)
    M.mla_decode_combine_out_proj(dims, ws, case.lens_t, w_uv, o, B, n_q, u, None, 0)
    torch.cuda.synchronize()
    # appended rows: only the new tokens' slots changed, each within bf16 rounding
    pos = positions.cpu().numpy()
    rows_ref = O.kv_rows(to_f64(h), to_f64(w_dkv), to_f64(w_kr), pos)
    changed = (case.pool.view(torch.int16) != pool0.view(torch.int16)).any(dim=-1).cpu().numpy()
    want = np.zeros_like(changed)
    got_rows = []
    for t in range(T):
        blk, off = O.slot_of(case.table, t // n_q, int(pos[t]), d.block_size)
        want[blk, off] = True
        got_rows.append(to_f64(case.pool[blk, off]))
    assert not np.any(changed & ~want), "a slot other than the new tokens' was written"
    got_rows = np.stack(got_rows)
    assert rel_l2(got_rows, rows_ref) <= 1e-2 and max_abs(got_rows, rows_ref) <= 2e-2
    # absorbed queries
    qi = to_f64(q_in)
    q_ref = O.absorb_query(qi[..., :d.d_nope], qi[..., d.d_nope:], to_f64(w_uk),
                           pos.reshape(B, n_q))
    assert rel_l2(to_f64(q), q_ref) <= 1e-2 and max_abs(to_f64(q), q_ref) <= 2e-2
    # u and o, from the stored q and the cache as the append left it
    case.q = q
    u_ref = np.stack([case.oracle(b)[0] for b in range(B)])
    assert rel_l2(to_f64(u), u_ref) <= 1e-2 and max_abs(to_f64(u), u_ref) <= 2e-2
    o_ref = O.out_proj(u_ref.reshape(T, H, d.d_latent), to_f64(w_uv))
    got = to_f64(o)
    assert np.all(np.isfinite(got))
    assert rel_l2(got, o_ref) <= 1e-2 and max_abs(got, o_ref) <= 2e-2


# --------------------------------------------------------------------------
# more sequences than one plan chunk (a workgroup scans 256 sequences at a time)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("generic", [False, True])
@pytest.mark.parametrize("G", [1, 300, 700])
def test_decode_many_sequences(generic, G):
    import mla_latent_kv_decode_amd as M
    cfg = W.scaled(W.CONFIGS["ragged"], batch=300, len_lo=1, len_hi=160)
    case = DecodeCase(cfg)
    u, lse = case.run(flags=M.FLAG_GENERIC_DECODE if generic else 0, G=G)
    compare_sampled(case, u, lse, [0, 1, 128, 255, 256, 257, 299])
    assert torch.isfinite(u.float()).all()


# --------------------------------------------------------------------------
# the MFMA decode kernel (default path for H=128, d_c=512, d_R=64, bf16)
# --------------------------------------------------------------------------
MFMA_SMALL = [
    W.scaled(W.CONFIGS["v3"], batch=3, seq_len=333),
    W.scaled(W.CONFIGS["ragged"], batch=6, len_lo=2, len_hi=700),
    W.scaled(W.CONFIGS["v3"], batch=2, seq_len=64),
    W.scaled(W.CONFIGS["v3"], batch=5, seq_len=1),
    # four causal query tokens per sequence (lengths >= 4)
    dataclasses.replace(W.scaled(W.CONFIGS["ragged"], batch=3, len_lo=4, len_hi=500), n_q=4),
]


@pytest.mark.parametrize("G", [1, 3, 8, 64])
@pytest.mark.parametrize("idx", range(len(MFMA_SMALL)))
def test_decode_mfma_small(idx, G):
    cfg = MFMA_SMALL[idx]
    case = DecodeCase(cfg)
    u, lse = case.run(G=G)
    compare_sampled(case, u, lse, list(range(cfg.batch)))


# fp8-e4m3 cache: the MFMA kernel dequantises each step into bf16 in LDS
MFMA_FP8 = [
    W.scaled(W.CONFIGS["fp8"], batch=3, seq_len=333),
    W.scaled(W.CONFIGS["fp8"], batch=2, seq_len=64),
    W.scaled(W.CONFIGS["fp8"], batch=4, seq_len=1),
    W.scaled(W.CONFIGS["fp8"], batch=3, seq_len=97),
]


@pytest.mark.parametrize("G", [1, 3, 64])
@pytest.mark.parametrize("idx", range(len(MFMA_FP8)))
def test_decode_mfma_fp8_small(idx, G):
    cfg = MFMA_FP8[idx]
    case = DecodeCase(cfg)
    u, lse = case.run(G=G)
    compare_sampled(case, u, lse, list(range(cfg.batch)), rel_bar=5e-2, abs_bar=None)
    assert torch.isfinite(u.float()).all()


def test_decode_mfma_fp8_agrees_with_generic():
    """Both fp8 paths decode the same codes and scales; they differ only in
    where the values are rounded (bf16 operands vs fp32 products)."""
    import mla_latent_kv_decode_amd as M
    cfg = W.scaled(W.CONFIGS["fp8"], batch=5, seq_len=900)
    case = DecodeCase(cfg)
    u1, l1 = case.run(G=16)
    u2, l2 = case.run(flags=M.FLAG_GENERIC_DECODE, G=16)
    assert rel_l2(to_f64(u1), to_f64(u2)) <= 5e-3
    # the generic path's products are exact in fp32: the two differ by at most
    # the bf16 rounding bound of the MFMA path (plus fp32 noise)
    tol = np.stack([1e-3 + fp8_score_bound(case, b) for b in range(cfg.batch)])
    assert np.all(np.abs(l1.cpu().numpy() - l2.cpu().numpy()) <= tol)


def test_decode_mfma_agrees_with_generic():
    import mla_latent_kv_decode_amd as M
    cfg = W.scaled(W.CONFIGS["ragged"], batch=8, len_lo=40, len_hi=900)
    case = DecodeCase(cfg)
    u1, l1 = case.run(G=16)
    u2, l2 = case.run(flags=M.FLAG_GENERIC_DECODE, G=16)
    assert rel_l2(to_f64(u1), to_f64(u2)) <= 5e-3
    assert max_abs(l1.cpu().numpy(), l2.cpu().numpy()) <= 1e-3


def test_validation_mode_reports_bad_device_data():
    """MLA_FLAG_VALIDATE: valid data runs as without the flag (bitwise); a
    length, page-table entry, position or sequence id that breaks a call's
    preconditions is reported with its index, and the call runs nothing."""
    import mla_latent_kv_decode_amd as M
    from mla_latent_kv_decode_amd import _lib as L
    case = DecodeCase(W.scaled(W.CONFIGS["v3"], batch=3, seq_len=200))
    dims = dims_of(case.cfg, M.FLAG_VALIDATE)
    B, n_q, H = 3, 1, case.d.num_heads
    ws = torch.empty(M.mla_decode_workspace_size(dims, B, n_q, 8), dtype=torch.uint8, device="cuda")
    u = torch.empty(B, n_q, H, case.d.d_latent, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B, n_q, H, device="cuda")
    M.mla_decode(dims, case.q, case.pool, None, case.table_t, case.lens_t, ws, 8)
    M.mla_decode_combine(dims, ws, case.lens_t, u, lse, 8)
    ur, lr = case.run(G=8)
    assert torch.equal(u, ur) and torch.equal(lse, lr)

    def rejected(fn, text):
        with pytest.raises(M.MlaError) as ei:
            fn()
        assert ei.value.code == L.ERR_INVALID_ARGUMENT and text in str(ei.value), str(ei.value)

    cap = case.table.shape[1] * case.d.block_size
    for b, bad in [(1, 0), (2, cap + 1)]:
        lens = case.lens_t.clone()
        lens[b] = bad
        rejected(lambda: M.mla_decode(dims, case.q, case.pool, None, case.table_t, lens, ws, 8), f"seq_lens[{b}]")
        if bad == 0:  # the combine knows no upper bound
            rejected(lambda: M.mla_decode_combine(dims, ws, lens, u, lse, 8), f"seq_lens[{b}]")
    table = case.table_t.clone()
    table[1, 2] = -1  # read by sequence 1 (length 200: blocks 0..3)
    rejected(lambda: M.mla_decode(dims, case.q, case.pool, None, table, case.lens_t, ws, 8), "sequence 1")
    # token-side calls
    d = case.d
    h = W.normal((2, d.d_model), 3, device="cuda", dtype=torch.bfloat16)
    w_dkv = W.weight(d.d_latent, d.d_model, 4, dtype=torch.bfloat16, device="cuda")
    w_kr = W.weight(d.d_rope, d.d_model, 5, dtype=torch.bfloat16, device="cuda")
    aws = append_workspace(dims, 2, d.d_model)
    for pos, sid, text in [([5, -1], [0, 1], "positions[1]"), ([5, cap], [0, 1], "positions[1]"),
                           ([5, 6], [-2, 1], "seq_ids[0]")]:
        rejected(lambda: M.mla_cache_append(dims, h, w_dkv, w_kr, torch.tensor(sid, dtype=torch.int32, device="cuda"),
                                            torch.tensor(pos, dtype=torch.int32, device="cuda"), case.table_t,
                                            case.pool, None, aws), text)
    q_in = W.normal((2, H, d.d_nope + d.d_rope), 6, device="cuda", dtype=torch.bfloat16)
    w_uk = W.normal((H, d.d_nope, d.d_latent), 7, std=1 / math.sqrt(d.d_latent), device="cuda", dtype=torch.bfloat16)
    q_out = torch.empty(2, H, d.row, dtype=torch.bfloat16, device="cuda")
    rejected(lambda: M.mla_query_absorb(dims, q_in, torch.tensor([3, -5], dtype=torch.int32, device="cuda"), w_uk,
                                        q_out), "positions[1]")
    # the one-call form checks both halves
    good_pos = torch.tensor([5, 6], dtype=torch.int32, device="cuda")
    sids = torch.tensor([0, 1], dtype=torch.int32, device="cuda")
    pool0 = case.pool.clone()
    rejected(lambda: M.mla_cache_append_query_absorb(dims, h, w_dkv, w_kr, sids, good_pos, case.table_t, case.pool,
                                                     None, aws, q_in, torch.tensor([3, -5], dtype=torch.int32,
                                                                                   device="cuda"), w_uk, q_out),
             "positions[1]")
    assert torch.equal(case.pool.view(torch.int16), pool0.view(torch.int16))  # rejected before the append ran


def test_host_threads_on_separate_streams_match_one_thread():
    """The library keeps no per-call state: two host threads, each launching
    decode + combine (bf16 and fp8 cache, first use of both kernels included)
    on its own stream at the same time, get the one-thread results bit for bit."""
    import threading
    import mla_latent_kv_decode_amd as M
    cases = [DecodeCase(W.scaled(W.CONFIGS["v3"], batch=6, seq_len=700)),
             DecodeCase(W.scaled(W.CONFIGS["fp8"], batch=5, seq_len=400))]
    outs = [None, None]

    def work(i):
        c = cases[i]
        dims = dims_of(c.cfg)
        B, n_q = c.q.shape[0], c.q.shape[1]
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            ws = torch.empty(M.mla_decode_workspace_size(dims, B, n_q, 16), dtype=torch.uint8, device="cuda")
            u = torch.empty(B, n_q, c.d.num_heads, c.d.d_latent, dtype=torch.bfloat16, device="cuda")
            lse = torch.empty(B, n_q, c.d.num_heads, dtype=torch.float32, device="cuda")
            for _ in range(3):
                M.mla_decode(dims, c.q, c.pool, c.scales, c.table_t, c.lens_t, ws, 16, stream=st)
                M.mla_decode_combine(dims, ws, c.lens_t, u, lse, 16, stream=st)
        st.synchronize()
        outs[i] = (u, lse)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    refs = [c.run(G=16) for c in cases]
    for (u, lse), (ur, lr) in zip(outs, refs):
        assert torch.equal(u, ur) and torch.equal(lse, lr)


def test_decode_mfma_deterministic():
    cfg = W.scaled(W.CONFIGS["ragged"], batch=5, len_lo=100, len_hi=2000)
    case = DecodeCase(cfg)
    u1, l1 = case.run(G=11)
    u2, l2 = case.run(G=11)
    assert torch.equal(u1.view(torch.int16), u2.view(torch.int16)) and torch.equal(l1, l2)


def test_decode_mfma_score_spike_in_late_tile():
    """A token far above the first tile's maximum (more than the kernel's
    headroom) forces the workgroup to recompute the piece with a raised
    reference; the result must still match the oracle."""
    cfg = W.scaled(W.CONFIGS["v3"], batch=2, seq_len=700)
    case = DecodeCase(cfg)
    d = cfg.dims
    for b, t in [(0, 650), (1, 200)]:
        blk, off = O.slot_of(case.table, b, t, d.block_size)
        q0 = case.q[b, 0, 0].float()
        case.pool[blk, off] = (3.0 * q0).to(torch.bfloat16)   # score ~ +40 nats for head 0
    u, lse = case.run(G=1)
    compare_sampled(case, u, lse, [0, 1])
    assert float(lse[0, 0, 0]) > 30.0


# --------------------------------------------------------------------------
# combine + out_proj fused (the merged u stays on chip)
# --------------------------------------------------------------------------
FUSED = [
    (W.scaled(W.CONFIGS["ragged"], batch=6, len_lo=40, len_hi=900), 16),   # 12 rows: row mode
    (W.scaled(W.CONFIGS["v3"], batch=40, seq_len=333), 0),                  # 40 rows: 32 + 8
    (W.scaled(W.CONFIGS["ragged"], batch=5, len_lo=2, len_hi=3000), 64),    # up to ~30 pieces a row
    (W.scaled(W.CONFIGS["ragged"], batch=20, len_lo=2, len_hi=3000), 64),   # 40 rows, many pieces
    (W.scaled(W.CONFIGS["long"], batch=4, seq_len=16384), 256),             # 4 rows x 64 pieces
    (W.scaled(W.CONFIGS["long"], batch=3, seq_len=5000), 96),               # 3 rows: two per workgroup, odd tail
    (W.scaled(W.CONFIGS["long"], batch=1, seq_len=7000), 64),               # 1 row: one per workgroup
    # several 32-row groups per workgroup (the default above 96 rows): W^UV_i
    # loaded once and reused, per-group reads of the slot table
    (W.scaled(W.CONFIGS["v3"], batch=128, seq_len=200), 0),                 # 128 rows: 2 groups each
    (W.scaled(W.CONFIGS["ragged"], batch=256, len_lo=2, len_hi=600), 0),   # 512 rows, n_q = 2: 8 groups
    (W.scaled(W.CONFIGS["v3"], batch=200, seq_len=130), 0),                 # 7 groups, 3 per workgroup: last has 1
    # several groups per workgroup and several 4-piece chunks per row
    (W.scaled(W.CONFIGS["v3"], batch=128, seq_len=1500), 1024),             # about 8 pieces a row
    (W.scaled(W.CONFIGS["ragged"], batch=256, len_lo=2, len_hi=700), 1024),  # 512 rows, 1 to ~10 pieces
]
ROW_MODE_MAX_ROWS = 32  # the fused kernel gives each (head, row) its own workgroup up to here


@pytest.mark.parametrize("idx", range(len(FUSED)))
def test_combine_out_proj_matches_separate_calls_and_oracle(idx):
    import mla_latent_kv_decode_amd as M
    cfg, G = FUSED[idx]
    case = DecodeCase(cfg)
    d = case.d
    B, n_q, H = case.q.shape[0], case.q.shape[1], d.num_heads
    dims = dims_of(cfg)
    ws = torch.empty(M.mla_decode_workspace_size(dims, B, n_q, G), dtype=torch.uint8, device="cuda")
    M.mla_decode(dims, case.q, case.pool, None, case.table_t, case.lens_t, ws, G)
    w_uv = W.normal((H, d.d_v, d.d_latent), 51, std=1 / math.sqrt(d.d_latent), device="cuda",
                    dtype=torch.bfloat16)
    # separate calls
    u_s = torch.empty(B, n_q, H, d.d_latent, dtype=torch.bfloat16, device="cuda")
    l_s = torch.empty(B, n_q, H, dtype=torch.float32, device="cuda")
    o_s = torch.empty(B * n_q, H, d.d_v, dtype=torch.bfloat16, device="cuda")
    M.mla_decode_combine(dims, ws, case.lens_t, u_s, l_s, G)
    M.mla_out_proj(dims, u_s.view(B * n_q, H, d.d_latent), w_uv, o_s)
    # fused, with and without storing u
    u_f = torch.full_like(u_s, float("nan"))
    l_f = torch.full_like(l_s, float("nan"))
    o_f = torch.full_like(o_s, float("nan"))
    o_f2 = torch.full_like(o_s, float("nan"))
    M.mla_decode_combine_out_proj(dims, ws, case.lens_t, w_uv, o_f, B, n_q, u_f, l_f, G)
    M.mla_decode_combine_out_proj(dims, ws, case.lens_t, w_uv, o_f2, B, n_q, None, None, G)
    torch.cuda.synchronize()
    assert torch.equal(o_f.view(torch.int16), o_f2.view(torch.int16))
    if B * n_q > ROW_MODE_MAX_ROWS:
        # row groups: the merge is the same arithmetic in the same order, bit for bit
        assert torch.equal(u_f.view(torch.int16), u_s.view(torch.int16))
        assert torch.equal(l_f, l_s)
    else:
        # row mode: four waves merge interleaved pieces, then each other --
        # another fp32 summation order (a bf16 rounding may land one ulp apart)
        assert rel_l2(to_f64(u_f), to_f64(u_s)) <= 1e-3
        assert max_abs(l_f.cpu().numpy(), l_s.cpu().numpy()) <= 1e-5
    # the projection sums the 512 products in another order
    assert rel_l2(to_f64(o_f), to_f64(o_s)) <= 2e-3
    # and against the oracle
    rows = list(range(B))
    u_ref = np.stack([case.oracle(b)[0] for b in rows])
    o_ref = O.out_proj(u_ref.reshape(B * n_q, H, d.d_latent), to_f64(w_uv))
    got = to_f64(o_f)
    assert np.all(np.isfinite(got))
    assert rel_l2(got, o_ref) <= 1e-2 and max_abs(got, o_ref) <= 2e-2


# --------------------------------------------------------------------------
# the step captured into HIP graphs (how bench.py and a serving loop run it)
# --------------------------------------------------------------------------
def test_graph_replay_matches_eager():
    """append + query absorption (one call) + decode + combine + out_proj
    captured as HIP graphs and replayed three times, with eager work on the stream between replays: every replay
    reproduces the eager outputs bit for bit (the calls allocate nothing and
    record no memsets, so they are safe to capture)."""
    import mla_latent_kv_decode_amd as M
    cfg = W.scaled(W.CONFIGS["ragged"], batch=6, len_lo=40, len_hi=900)
    case = DecodeCase(cfg)
    d = case.d
    B, n_q, H = case.q.shape[0], case.q.shape[1], d.num_heads
    dims = dims_of(cfg)
    G = 16
    dev = "cuda"
    ws = torch.empty(M.mla_decode_workspace_size(dims, B, n_q, G), dtype=torch.uint8, device=dev)
    u = torch.empty(B, n_q, H, d.d_latent, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(B, n_q, H, dtype=torch.float32, device=dev)
    o = torch.empty(B * n_q, H, d.d_v, dtype=torch.bfloat16, device=dev)
    w_uv = W.normal((H, d.d_v, d.d_latent), 41, std=1 / math.sqrt(d.d_latent), device=dev,
                    dtype=torch.bfloat16)
    T = B * n_q  # the n_q newest tokens of every sequence are rewritten by append
    h = W.normal((T, d.d_model), 42, device=dev, dtype=torch.bfloat16)
    w_dkv = W.weight(d.d_latent, d.d_model, 43, dtype=torch.bfloat16, device=dev)
    w_kr = W.weight(d.d_rope, d.d_model, 44, dtype=torch.bfloat16, device=dev)
    seq_ids = torch.arange(B, dtype=torch.int32, device=dev).repeat_interleave(n_q)
    positions = (case.lens_t.repeat_interleave(n_q) - n_q
                 + torch.arange(n_q, dtype=torch.int32, device=dev).repeat(B)).to(torch.int32)
    aws = append_workspace(dims, T, d.d_model)
    q_in = W.normal((T, H, d.d_nope + d.d_rope), 45, device=dev, dtype=torch.bfloat16)
    w_uk = W.normal((H, d.d_nope, d.d_latent), 46, std=1 / math.sqrt(d.d_latent), device=dev,
                    dtype=torch.bfloat16)
    qa = torch.empty(T, H, d.row, dtype=torch.bfloat16, device=dev)  # absorbed queries of the new tokens
    calls = [
        lambda: M.mla_cache_append_query_absorb(dims, h, w_dkv, w_kr, seq_ids, positions, case.table_t,
                                                case.pool, None, aws, q_in, positions, w_uk, qa),
        lambda: M.mla_decode(dims, case.q, case.pool, None, case.table_t, case.lens_t, ws, G),
        lambda: M.mla_decode_combine(dims, ws, case.lens_t, u, lse, G),
        lambda: M.mla_out_proj(dims, u.view(B * n_q, H, d.d_latent), w_uv, o),
    ]
    for c in calls:
        c()
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    ref = [bits(x).clone() for x in (u, lse, o, case.pool, qa)]
    assert torch.isfinite(o.float()).all()
    cap = torch.cuda.Stream()
    graphs = []
    for c in calls:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            c()
        graphs.append(g)
    for rep in range(3):
        for x in (u, lse, o, ws, qa):
            x.zero_()  # eager work between replays
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        for got, want in zip((u, lse, o, case.pool, qa), ref):
            assert torch.equal(bits(got), want), f"replay {rep} differs from the eager run"

"""Pins for the CPU oracle: checks against facts fixed outside the oracle itself.

Each test names what it pins: the pages' printed figures, textbook or library
routines (2-D rotation, torch's scaled-dot-product attention and casts,
scipy's logsumexp), closed-form special cases, invariants, or brute force.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_pages_numbers():
    vals = {}
    with open(os.path.join(GOLDEN, "pages_numbers.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split("=", 1)
            vals[key.strip()] = float(rest.split("|")[0])
    return vals


# --------------------------------------------------------------------------
# footprint: the pages' printed numbers
# --------------------------------------------------------------------------
def test_footprint_matches_pages_numbers():
    g = load_pages_numbers()
    n = O.cached_scalars_per_token(int(g["d_latent"]), int(g["d_rope"]))
    assert n == g["cached_scalars"]
    assert round(100 * (g["mha32_scalars"] - n) / g["mha32_scalars"], 2) == g["reduction_vs_mha32_pct"]
    mha128 = O.mha_cache_bytes(1, g["mha128_heads"], g["mha128_dh"], 1, 1, 1)
    assert mha128 == g["mha128_scalars"]
    frac = 100 * g["d_latent"] / mha128
    assert round(frac, 2) == g["content_fraction_pct"]
    assert round(100 - frac, 2) == g["content_reduction_pct"]
    step_gb = g["streams"] * g["kv_gb_per_stream"]
    assert round(step_gb, 2) == g["kv_gb_per_step"]
    ms = 1000 * step_gb / g["h100_hbm_gb_per_s"]
    assert round(ms, 1) == g["ms_per_token"]
    assert round(1000 / ms, 1) == g["tokens_per_s"]


def test_pool_bytes_closed_form():
    # 576 scalars per token: 1152 B in bf16, 576 B + five fp32 tile scales in fp8
    assert O.pool_bytes(1, 1, 512, 64, 2) == 1152
    assert O.pool_bytes(1, 1, 512, 64, 1, scale_tiles=5) == 596
    assert O.pool_bytes(4096, 64, 512, 64, 2) == 4096 * 64 * 1152
    assert len(O.fp8_tiles(576)) == 5 and O.fp8_tiles(576)[-1] == (512, 576)
    assert O.pool_bytes(2, 64, 32, 8, 4) == 2 * 64 * 160


# --------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------
def test_rope_two_dims_is_textbook_rotation():
    # n = 2: a single pair rotated by theta_0 = pos radians (base^0 = 1)
    rng = np.random.default_rng(0)
    for pos in [0.0, 1.0, 3.0, 17.0, 131071.0]:
        x = rng.standard_normal(2)
        R = np.array([[math.cos(pos), -math.sin(pos)], [math.sin(pos), math.cos(pos)]])
        np.testing.assert_allclose(O.rope(x, pos), R @ x, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [8, 64])
def test_rope_pairs_channel_j_with_j_plus_half(n):
    h = n // 2
    pos = 5.0
    for j in range(h):
        e = np.zeros(n)
        e[j] = 1.0
        y = O.rope(e, pos)
        mask = np.ones(n, bool)
        mask[[j, j + h]] = False
        assert np.all(y[mask] == 0), "rotation leaks outside the (j, j+n/2) plane"
        ang = math.atan2(y[j + h], y[j])
        want = math.remainder(pos * 10000.0 ** (-j / h), 2 * math.pi)
        assert abs(math.remainder(ang - want, 2 * math.pi)) < 1e-9


def test_rope_norm_identity_and_relative_position():
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    assert np.array_equal(O.rope(q, 0), q)
    for p in [1, 77, 4095, 131071]:
        assert abs(np.linalg.norm(O.rope(q, p)) - np.linalg.norm(q)) < 1e-12 * np.linalg.norm(q) * 10
    for m, n in [(10, 3), (4096, 4000), (131071, 5)]:
        lhs = O.rope(q, m) @ O.rope(k, n)
        rhs = O.rope(q, m - n) @ k
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(lhs))


# --------------------------------------------------------------------------
# bf16 and e4m3 formats
# --------------------------------------------------------------------------
def test_bf16_rounding_known_values():
    one = 1.0
    assert O.round_bf16(np.float32(one))[()] == 1.0
    # 1 + 2^-8 sits halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert O.round_bf16(np.float32(1 + 2 ** -8))[()] == 1.0
    # 1 + 3*2^-8 sits halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even)
    assert O.round_bf16(np.float32(1 + 3 * 2 ** -8))[()] == 1 + 2 ** -6
    assert O.round_bf16(np.float32(1 + 2 ** -8 + 2 ** -20))[()] == 1 + 2 ** -7
    ints = np.arange(-256, 257, dtype=np.float32)
    assert np.array_equal(O.round_bf16(ints), ints.astype(np.float64))
    x = np.array([3.140625, -0.0078125], dtype=np.float32)  # exactly representable
    assert np.array_equal(O.round_bf16(x), x.astype(np.float64))


def test_e4m3_decode_known_codes():
    d = O.e4m3_decode
    assert d(0x7E) == 448.0            # largest finite
    assert d(0x08) == 2.0 ** -6        # smallest normal
    assert d(0x01) == 2.0 ** -9        # smallest subnormal
    assert d(0x38) == 1.0
    assert d(0x39) == 1.125
    assert d(0xB8) == -1.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x80) == 0.0 and math.copysign(1, d(0x80)) == -1
    pos = d(np.arange(0, 0x7F))
    assert np.all(np.diff(pos) > 0), "positive finite codes must increase"
    assert len(np.unique(pos)) == 127


def _nearest_even_e4m3(x):
    """Brute force over the decode table: nearest finite code, ties to even."""
    table = O.e4m3_decode(np.arange(0, 0x7F))
    out = []
    for v in np.asarray(x, dtype=np.float64):
        a = min(abs(v), 448.0)
        dist = np.abs(table - a)
        best = np.flatnonzero(dist == dist.min())
        c = int(best[0]) if len(best) == 1 else int([b for b in best if b % 2 == 0][0])
        out.append(c | (0x80 if v < 0 or (v == 0 and math.copysign(1, v) < 0) else 0))
    return np.array(out, dtype=np.uint8)


def test_e4m3_encode_round_trip_ties_and_saturation():
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = O.e4m3_decode(finite).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(vals), finite)
    # ties to even
    assert O.e4m3_encode(np.float32(1.0625))[()] == 0x38
    assert O.e4m3_encode(np.float32(1.1875))[()] == 0x3A
    # saturation instead of NaN
    assert O.e4m3_encode(np.float32(500.0))[()] == 0x7E
    assert O.e4m3_encode(np.float32(-1e9))[()] == 0xFE
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(3000) * 50, rng.standard_normal(1000) * 0.01,
                        rng.uniform(-460, 460, 1000)]).astype(np.float32)
    assert np.array_equal(O.e4m3_encode(x), _nearest_even_e4m3(x))


def test_fp8_row_quantizer_properties():
    rng = np.random.default_rng(3)
    row = rng.standard_normal(576).astype(np.float32)
    row[[5, 300]] *= 20
    row[512:576] = 0.0
    row[520] = -2.5
    codes, scales = O.quantize_fp8_row(row)
    assert codes.shape == (576,) and scales.shape == (5,)
    for k, (lo, hi) in enumerate(O.fp8_tiles(576)):
        t = row[lo:hi]
        amax = np.max(np.abs(t))
        i = int(np.argmax(np.abs(t)))
        assert codes[lo + i] & 0x7F == 0x7E, "the tile maximum encodes to +-448"
        assert scales[k] == np.float32(amax / np.float32(448))
        dec = O.e4m3_decode(codes[lo:hi]) * scales[k]
        # e4m3 has 3 mantissa bits: relative error <= 2^-4 for normals,
        # absolute error <= 2^-10 * scale in the subnormal range
        err = np.abs(dec - t)
        assert np.all(err <= np.maximum(np.abs(t) * 2.0 ** -4, 2.0 ** -10 * scales[k]) * 1.0001)
    zc, zs = O.quantize_fp8_row(np.zeros(576, np.float32))
    assert np.all(zc == 0) and np.all(zs == 1.0)
    # the vectorised version is the same function
    rows = rng.standard_normal((7, 576)).astype(np.float32)
    rows[3] = 0
    vc, vs = O.quantize_fp8_rows(rows)
    for r in range(7):
        c1, s1 = O.quantize_fp8_row(rows[r])
        assert np.array_equal(vc[r], c1) and np.array_equal(vs[r], s1)


def _smallest_pow2_exponent(a):
    """Brute force over exponents: the smallest E with a <= 448 * 2^E."""
    return min(e for e in range(-160, 160) if a <= 448.0 * 2.0 ** e)


def test_pow2_scale_exponent_brute_force_and_boundaries():
    rng = np.random.default_rng(11)
    vals = np.concatenate([np.abs(rng.standard_normal(200)) * 10.0 ** rng.integers(-12, 12, 200),
                           [448.0, 224.0, 56.0, 1.0, 2.0 ** -20, 3.5]])
    for a in vals:
        assert O.pow2_scale_exponent(a) == _smallest_pow2_exponent(a), a
    # the tile maximum lands in the top binade (224, 448]
    assert O.pow2_scale_exponent(448.0) == 0
    assert O.pow2_scale_exponent(np.nextafter(448.0, 1e9)) == 1
    assert O.pow2_scale_exponent(224.0) == -1
    assert O.pow2_scale_exponent(np.nextafter(224.0, 1e9)) == 0


def test_fp8_pow2_quantizer_properties():
    """Power-of-two tile scales: each scale is 2^E with the tile maximum in
    (224, 448] after scaling, and each code is the nearest e4m3 value (ties to
    even) of r / scale, found by brute force over the code table."""
    rng = np.random.default_rng(12)
    rows = rng.standard_normal((6, 576)).astype(np.float32)
    rows[:, [5, 300, 530]] *= 20
    rows[1, 128:256] = 0.0                      # a zero tile
    rows[2, 0:128] = rows[2, 0:128] / np.max(np.abs(rows[2, 0:128])) * 56.0   # amax = 448 * 2^-3
    rows[3, 256:384] *= np.float32(1e-3)
    codes, scales = O.quantize_fp8_rows(rows, pow2_scales=True)
    assert codes.shape == rows.shape and scales.shape == (6, 5)
    for r in range(6):
        for k, (lo, hi) in enumerate(O.fp8_tiles(576)):
            t = rows[r, lo:hi].astype(np.float64)
            amax = np.max(np.abs(t))
            if amax == 0:
                assert scales[r, k] == 1.0 and np.all(codes[r, lo:hi] == 0)
                continue
            sc = float(scales[r, k])
            assert np.frexp(sc)[0] == 0.5, "the scale is a power of two"
            assert sc == 2.0 ** _smallest_pow2_exponent(amax)
            assert 224.0 < amax / sc <= 448.0
            assert np.array_equal(codes[r, lo:hi], _nearest_even_e4m3(t / sc))
    assert scales[2, 0] == 2.0 ** -3
    # the dequantised rows are the codes times their tile's power of two
    deq = O.dequantize_fp8_rows(codes, scales)
    err = np.abs(deq - rows)
    assert np.all(err <= np.maximum(np.abs(rows) * 2.0 ** -4,
                                    2.0 ** -10 * np.repeat(scales, [128] * 4 + [64], axis=1)) * 1.0001)


def test_query_rows_e4m3_pow2():
    """One power-of-two scale per row: rows of very different magnitude each
    keep e4m3's relative precision."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((3, 2, 40)).astype(np.float32)
    x[0, 1] *= 1e4
    x[1, 0] *= 1e-5
    x[2, 1] = 0.0
    out = O.quantize_rows_e4m3_pow2(x)
    assert out.shape == x.shape
    for i in range(3):
        for j in range(2):
            row = x[i, j].astype(np.float64)
            a = np.max(np.abs(row))
            if a == 0:
                assert np.all(out[i, j] == 0)
                continue
            e = _smallest_pow2_exponent(a)
            want = O.e4m3_decode(_nearest_even_e4m3(row * 2.0 ** -e)) * 2.0 ** e
            assert np.array_equal(out[i, j], want)
            assert 224.0 < np.max(np.abs(out[i, j])) / 2.0 ** e <= 448.0


# --------------------------------------------------------------------------
# attention: brute force, un-absorbed form, library attention, special cases
# --------------------------------------------------------------------------
def _rand_case(rng, n_heads=3, d_c=8, d_r=4, d_nope=5, d_v=6, L=9, n_q=1):
    rows = rng.standard_normal((L, d_c + d_r))
    q_c = rng.standard_normal((n_q, n_heads, d_nope))
    q_r = rng.standard_normal((n_q, n_heads, d_r))
    w_uk = rng.standard_normal((n_heads, d_nope, d_c)) / math.sqrt(d_c)
    w_uv = rng.standard_normal((n_heads, d_v, d_c)) / math.sqrt(d_c)
    q = np.concatenate([np.einsum("jin,inc->jic", q_c, w_uk), q_r], axis=-1)
    return rows, q_c, q_r, w_uk, w_uv, q


@pytest.mark.parametrize("n_q", [1, 2, 3])
def test_absorbed_equals_bruteforce(n_q):
    rng = np.random.default_rng(10 + n_q)
    for L in [n_q, 5, 13]:
        rows, q_c, q_r, w_uk, w_uv, q = _rand_case(rng, L=L, n_q=n_q)
        scale = O.softmax_scale(5, 4)
        u, lse = O.attend_absorbed(q, rows, n_q, 8, scale)
        ub, lseb = O.attend_bruteforce(q, rows, n_q, 8, scale)
        np.testing.assert_allclose(u, ub, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse, lseb, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n_q", [1, 2])
def test_absorbed_equals_unabsorbed(n_q):
    rng = np.random.default_rng(20 + n_q)
    rows, q_c, q_r, w_uk, w_uv, q = _rand_case(rng, n_heads=4, d_c=32, d_r=8, d_nope=16,
                                              d_v=16, L=70, n_q=n_q)
    scale = O.softmax_scale(16, 8)
    u, _ = O.attend_absorbed(q, rows, n_q, 32, scale)
    o = O.out_proj(u, w_uv)
    o2 = O.attend_unabsorbed(q_c, q_r, rows, w_uk, w_uv, n_q, 32, scale)
    np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("n_q", [1, 2])
def test_unabsorbed_matches_library_attention(n_q):
    """Per-head keys [W^UK c ; k^R], values W^UV c, scale 1/sqrt(d_nope + d_R),
    causal visibility -- built here from the pages' definitions and fed to
    torch's scaled_dot_product_attention (math backend, float64)."""
    rng = np.random.default_rng(30 + n_q)
    H, d_c, d_r, d_nope, d_v, L = 4, 32, 8, 16, 12, 40
    rows, q_c, q_r, w_uk, w_uv, q = _rand_case(rng, H, d_c, d_r, d_nope, d_v, L, n_q)
    c, kr = rows[:, :d_c], rows[:, d_c:]
    K = np.stack([np.concatenate([c @ w_uk[i].T, kr], 1) for i in range(H)])  # [H, L, 24]
    V = np.stack([c @ w_uv[i].T for i in range(H)])                            # [H, L, d_v]
    Q = np.concatenate([q_c, q_r], -1).transpose(1, 0, 2)                      # [H, n_q, 24]
    mask = np.zeros((n_q, L), bool)
    for j in range(n_q):
        mask[j, : L - n_q + j + 1] = True
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(Q)[None], torch.tensor(K)[None], torch.tensor(V)[None],
        attn_mask=torch.tensor(mask), scale=1.0 / math.sqrt(d_nope + d_r)).numpy()[0]
    u, _ = O.attend_absorbed(q, rows, n_q, d_c, O.softmax_scale(d_nope, d_r))
    np.testing.assert_allclose(O.out_proj(u, w_uv).transpose(1, 0, 2), ref, rtol=1e-10, atol=1e-12)


def test_decode_special_cases():
    rng = np.random.default_rng(40)
    H, D, d_c = 3, 12, 8
    scale = 0.3
    q = rng.standard_normal((1, H, D))
    rows = rng.standard_normal((1, D))
    u, lse = O.attend_absorbed(q, rows, 1, d_c, scale)
    assert np.array_equal(u[0], np.broadcast_to(rows[0, :d_c], (H, d_c))), "seq_len 1 -> u = c_0"
    np.testing.assert_allclose(lse[0], scale * (q[0] @ rows[0]), rtol=1e-14)
    same = np.tile(rng.standard_normal((1, D)), (33, 1))
    u, lse = O.attend_absorbed(q, same, 1, d_c, scale)
    np.testing.assert_allclose(u[0], np.broadcast_to(same[0, :d_c], (H, d_c)), rtol=1e-13)
    np.testing.assert_allclose(lse[0], scale * (q[0] @ same[0]) + math.log(33), rtol=1e-13)
    rows = rng.standard_normal((20, D))
    u, lse = O.attend_absorbed(np.zeros((1, H, D)), rows, 1, d_c, scale)
    np.testing.assert_allclose(u[0], np.broadcast_to(rows[:, :d_c].mean(0), (H, d_c)), rtol=1e-13)
    np.testing.assert_allclose(lse[0], math.log(20), rtol=1e-14)
    big = rows.copy()
    big[7, d_c:] = 0
    big[7, d_c] = 1e4
    qb = np.zeros((1, H, D))
    qb[0, :, d_c] = 1.0
    u, _ = O.attend_absorbed(qb, big, 1, d_c, 1.0)
    np.testing.assert_allclose(u[0], np.broadcast_to(big[7, :d_c], (H, d_c)), rtol=0, atol=0)


def test_causal_query0_equals_shorter_single_query():
    rng = np.random.default_rng(41)
    rows = rng.standard_normal((30, 12))
    q = rng.standard_normal((2, 3, 12))
    u2, l2 = O.attend_absorbed(q, rows, 2, 8, 0.4)
    u1, l1 = O.attend_absorbed(q[:1], rows[:29], 1, 8, 0.4)
    np.testing.assert_allclose(u2[0], u1[0], rtol=1e-14)
    np.testing.assert_allclose(l2[0], l1[0], rtol=1e-14)
    u1b, _ = O.attend_absorbed(q[1:], rows, 1, 8, 0.4)
    np.testing.assert_allclose(u2[1], u1b[0], rtol=1e-14)


# --------------------------------------------------------------------------
# split-KV partials and the log-sum-exp merge
# --------------------------------------------------------------------------
def test_combine_of_any_partition_equals_unsplit():
    from scipy.special import logsumexp
    rng = np.random.default_rng(50)
    rows = rng.standard_normal((100, 12))
    q = rng.standard_normal((1, 5, 12))
    u, lse = O.attend_absorbed(q, rows, 1, 8, 0.5)
    s = 0.5 * (q[0] @ rows.T)
    np.testing.assert_allclose(lse[0], logsumexp(s, axis=1), rtol=1e-14)
    for cuts in [[0, 100], [0, 1, 100], [0, 37, 64, 65, 100], [0, 0, 50, 50, 100, 100]]:
        parts = [O.attend_partial(q[0], rows, a, b, 8, 0.5) for a, b in zip(cuts[:-1], cuts[1:])]
        uc, lc = O.combine([p[0] for p in parts], [p[1] for p in parts])
        np.testing.assert_allclose(uc, u[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(lc, lse[0], rtol=1e-13)


# --------------------------------------------------------------------------
# up-projection, paging, append, query path
# --------------------------------------------------------------------------
def test_out_proj_explicit_loops():
    rng = np.random.default_rng(60)
    u = rng.standard_normal((3, 4, 7))
    w = rng.standard_normal((4, 5, 7))   # [H, d_v, d_c], d_v != d_c
    o = O.out_proj(u, w)
    for r in range(3):
        for i in range(4):
            for v in range(5):
                assert abs(o[r, i, v] - sum(w[i, v, d] * u[r, i, d] for d in range(7))) < 1e-12


def test_paging_gather_and_permutation_invariance():
    rng = np.random.default_rng(70)
    bs, D, L = 4, 6, 10
    contig = rng.standard_normal((L, D)).astype(np.float32)
    nblk = 3
    # hand-built table: logical block k of sequence 0 lives in physical block perm[k]
    perm = [5, 1, 3]
    pool = {"dtype": "fp32", "data": np.full((7, bs, D), np.nan, np.float32)}
    for t in range(L):
        pool["data"][perm[t // bs], t % bs] = contig[t]
    table = np.array([perm + [-1]], dtype=np.int32)
    assert O.slot_of(table, 0, 9, bs) == (3, 1)
    got = O.gather_sequence(pool, table, 0, L, bs)
    assert np.array_equal(got, contig.astype(np.float64)), "NaN tail slots must not be read"
    q = rng.standard_normal((1, 1, 2, D))
    a = O.decode(q, pool, table, [L], bs, 4, 0.5)[0]
    pool2 = {"dtype": "fp32", "data": np.zeros((nblk, bs, D), np.float32)}
    pool2["data"].reshape(-1, D)[:L] = contig
    b = O.decode(q, pool2, np.array([[0, 1, 2]], np.int32), [L], bs, 4, 0.5)[0]
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("dtype", ["fp32", "bf16", "fp8"])
def test_append_identity_projection_is_a_copy(dtype):
    rng = np.random.default_rng(80)
    d_c, d_r, bs = 16, 8, 4
    D = d_c + d_r
    w_dkv = np.concatenate([np.eye(d_c), np.zeros((d_c, d_r))], 1)
    w_kr = np.concatenate([np.zeros((d_r, d_c)), np.eye(d_r)], 1)
    h = rng.standard_normal((5, D)).astype(np.float32)
    if dtype == "bf16":
        h = O.round_bf16(h).astype(np.float32)
    table = np.array([[2, 0], [1, 3]], np.int32)
    seq_ids = np.array([0, 0, 1, 1, 1])
    positions = np.array([0, 0, 0, 0, 0]) * 0
    positions = np.array([0, 5, 0, 3, 6])
    data = {"fp32": np.zeros((4, bs, D), np.float32), "bf16": np.zeros((4, bs, D), np.uint16),
            "fp8": np.zeros((4, bs, D), np.uint8)}[dtype]
    pool = {"dtype": dtype, "data": data, "scales": np.zeros((4, bs, 1), np.float32)}
    if dtype == "fp8":
        pool["scales"] = np.zeros((4, bs, 1), np.float32)
    O.append(pool, h, w_dkv, w_kr, seq_ids, positions, table, bs)
    vals = O.pool_values(pool)
    written = {(2, 0): 0, (0, 1): 1, (1, 0): 2, (1, 3): 3, (3, 2): 4}
    for (blk, off), i in written.items():
        want = np.concatenate([h[i, :d_c], O.rope(h[i, d_c:], positions[i])]).astype(np.float32)
        if dtype == "fp8":
            codes, sc = O.quantize_fp8_row(want)
            assert np.array_equal(pool["data"][blk, off], codes)
        elif dtype == "bf16":
            assert np.array_equal(pool["data"][blk, off], O.to_bf16_bits(want))
        else:
            assert np.array_equal(vals[blk, off], want.astype(np.float64))
        if positions[i] == 0 and dtype != "fp8":
            assert np.array_equal(vals[blk, off], h[i].astype(np.float64)), "RoPE at 0 is the identity"
    untouched = np.ones((4, bs), bool)
    for k in written:
        untouched[k] = False
    assert np.all(pool["data"][untouched] == 0)


def test_query_path_absorption_is_associativity():
    rng = np.random.default_rng(90)
    H, d_nope, d_r, d_c, d_model = 4, 16, 8, 32, 64
    w_q = rng.standard_normal((H * (d_nope + d_r), d_model)) / 8
    w_uk = rng.standard_normal((H, d_nope, d_c)) / math.sqrt(d_c)
    h = rng.standard_normal(d_model)
    packed, q_c, q_r = O.query_from_hidden(h, w_q, w_uk, 64, H, d_nope, d_r)
    full = w_q @ h
    for i in range(H):
        seg = full[i * (d_nope + d_r):(i + 1) * (d_nope + d_r)]
        assert np.array_equal(q_c[i], seg[:d_nope])
        np.testing.assert_allclose(q_r[i], O.rope(seg[d_nope:], 64), rtol=1e-14)
    c = rng.standard_normal(d_c)
    for i in range(H):
        lhs = packed[i, :d_c] @ c
        rhs = q_c[i] @ (w_uk[i] @ c)
        assert abs(lhs - rhs) < 1e-12 * (1 + abs(rhs))


# --------------------------------------------------------------------------
# dense layers of the decoding section: low-rank query path, W^O
# --------------------------------------------------------------------------
def test_linear_explicit_loops():
    rng = np.random.default_rng(100)
    x = rng.standard_normal((3, 7))
    w = rng.standard_normal((5, 7))     # [n, k]
    y = O.linear(x, w)
    assert y.shape == (3, 5)
    for r in range(3):
        for n in range(5):
            assert abs(y[r, n] - sum(x[r, k] * w[n, k] for k in range(7))) < 1e-12
    # a permutation weight picks input columns
    perm = [4, 0, 6, 2]
    np.testing.assert_array_equal(O.linear(x, np.eye(7)[perm]), x[:, perm])


def test_lowrank_query_equals_composed_single_projection():
    """W^UQ (W^DQ h) = (W^UQ W^DQ) h: with the two up-projections' rows put
    head by head ([W^UQ_i ; W^QR_i]) the product is the single-matrix W^Q of
    the small workload, split by split_query."""
    rng = np.random.default_rng(101)
    H, d_nope, d_r, d_q, d_model = 3, 4, 2, 5, 9
    w_dq = rng.standard_normal((d_q, d_model))
    w_uq = rng.standard_normal((H * d_nope, d_q))
    w_qr = rng.standard_normal((H * d_r, d_q))
    h = rng.standard_normal((2, d_model))
    q_c, q_r = O.query_lowrank(h, w_dq, w_uq, w_qr, H, d_nope, d_r)
    w_q = np.concatenate([np.concatenate([w_uq[i * d_nope:(i + 1) * d_nope],
                                          w_qr[i * d_r:(i + 1) * d_r]]) for i in range(H)]) @ w_dq
    c2, r2 = O.split_query(h @ w_q.T, H, d_nope, d_r)
    np.testing.assert_allclose(q_c, c2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(q_r, r2, rtol=1e-12, atol=1e-12)
    # head i's content query uses rows i*d_nope .. of W^UQ only
    c_q = w_dq @ h[1]
    assert abs(q_c[1, 2, 3] - w_uq[2 * d_nope + 3] @ c_q) < 1e-12
    assert abs(q_r[1, 1, 0] - w_qr[1 * d_r + 0] @ c_q) < 1e-12


def test_output_projection_equals_fused_w_ov():
    """The offline fusion of [MLA-93] Core Mechanics 3: with W^O_i the
    columns of W^O that meet head i, sum_i (W^O_i W^UV_i) u_i equals
    W^O applied to the concatenated W^UV_i u_i."""
    rng = np.random.default_rng(102)
    rows, H, d_v, d_c, d = 2, 3, 4, 6, 5
    u = rng.standard_normal((rows, H, d_c))
    w_uv = rng.standard_normal((H, d_v, d_c))
    w_o = rng.standard_normal((d, H * d_v))
    out = O.output_projection(O.out_proj(u, w_uv), w_o)
    fused = sum(u[:, i] @ (w_o[:, i * d_v:(i + 1) * d_v] @ w_uv[i]).T for i in range(H))
    np.testing.assert_allclose(out, fused, rtol=1e-12, atol=1e-12)



# --------------------------------------------------------------------------
# fp8 dequantisation and the rotated half of the packed query
# --------------------------------------------------------------------------
# (code, value) pairs of the OCP E4M3 encoding, read off its bit layout by
# hand: sign, 4 exponent bits (bias 7), 3 mantissa bits, subnormals m * 2^-9.
E4M3_KNOWN = [(0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
              (0x30, 0.5), (0x38, 1.0), (0x3C, 1.5), (0x40, 2.0), (0x4B, 5.5),
              (0x7E, 448.0), (0xB8, -1.0), (0xC4, -3.0), (0xFE, -448.0)]


def test_dequantize_fp8_rows_per_tile_scales():
    """Each channel decodes to its code's value times the scale of its own
    128-channel tile; the row's last tile (channels 512..575) is half width.
    The expected values are the listed code values times a scale chosen
    distinct for every (row, tile) -- powers of two and non-dyadic ones -- so
    a tile boundary off by any amount, or one tile's scale reused for another,
    changes some element."""
    rng = np.random.default_rng(110)
    n_rows, D = 3, 576
    pick = rng.integers(0, len(E4M3_KNOWN), size=(n_rows, D))
    codes = np.array([[E4M3_KNOWN[k][0] for k in r] for r in pick], dtype=np.uint8)
    vals = np.array([[E4M3_KNOWN[k][1] for k in r] for r in pick], dtype=np.float64)
    # tile k of row r: 2^(k - 2) * (1 + r / 3), written out per tile
    scales = np.array([[np.float32(2.0 ** (k - 2) * (1 + r / 3)) for k in range(5)]
                       for r in range(n_rows)], dtype=np.float32)
    got = O.dequantize_fp8_rows(codes, scales)
    assert got.shape == (n_rows, D)
    for r in range(n_rows):
        for c in range(D):
            tile = 0 if c < 128 else 1 if c < 256 else 2 if c < 384 else 3 if c < 512 else 4
            want = vals[r, c] * float(scales[r, tile])
            assert got[r, c] == want, (r, c, got[r, c], want)
    # leading axes (blocks x tokens) broadcast the same way
    got3 = O.dequantize_fp8_rows(codes.reshape(1, n_rows, D), scales.reshape(1, n_rows, 5))
    assert np.array_equal(got3[0], got)


def test_absorbed_query_rope_half_is_rotated_at_each_rows_position():
    """packed[..., d_c:] of absorb_query is q^R rotated at the row's own
    position.  With d_R = 2 the rotation is the textbook 2-D rotation by
    pos radians (the only frequency is base^0 = 1); the positions differ per
    row, so a broadcast of one row's position, an unrotated q^R or a rotation
    at position 0 all fail.  The content half is checked against explicit
    sums of q^C_i[n] W^UK_i[n, c]."""
    rng = np.random.default_rng(111)
    rows, H, d_nope, d_c = 4, 3, 5, 6
    pos = np.array([[0], [1], [7], [131071]], dtype=np.int64)[:, 0]
    for d_r in (2, 8):
        q_c = rng.standard_normal((rows, H, d_nope))
        q_r = rng.standard_normal((rows, H, d_r))
        w_uk = rng.standard_normal((H, d_nope, d_c))
        packed = O.absorb_query(q_c, q_r, w_uk, pos)
        assert packed.shape == (rows, H, d_c + d_r)
        for r in range(rows):
            for i in range(H):
                for c in range(d_c):
                    want = sum(q_c[r, i, n] * w_uk[i, n, c] for n in range(d_nope))
                    assert abs(packed[r, i, c] - want) <= 1e-12 * (1 + abs(want))
                if d_r == 2:
                    th = float(pos[r])
                    R = np.array([[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]])
                    np.testing.assert_allclose(packed[r, i, d_c:], R @ q_r[r, i], rtol=0, atol=1e-12)
                else:
                    # each pair (j, j + 4) is turned by pos * 10000^(-j/4)
                    for j in range(d_r // 2):
                        th = float(pos[r]) * 10000.0 ** (-j / (d_r // 2))
                        x, y = q_r[r, i, j], q_r[r, i, j + d_r // 2]
                        assert abs(packed[r, i, d_c + j] - (x * math.cos(th) - y * math.sin(th))) <= 1e-9
                        assert abs(packed[r, i, d_c + j + d_r // 2]
                                   - (y * math.cos(th) + x * math.sin(th))) <= 1e-9
    # a [B, n_q] position grid (the decode's query layout) rotates each query at its own position
    q_c = rng.standard_normal((2, 2, H, d_nope))
    q_r = rng.standard_normal((2, 2, H, 2))
    w_uk = rng.standard_normal((H, d_nope, d_c))
    grid = np.array([[10, 11], [500, 501]])
    packed = O.absorb_query(q_c, q_r, w_uk, grid)
    for b in range(2):
        for j in range(2):
            th = float(grid[b, j])
            R = np.array([[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]])
            for i in range(H):
                np.testing.assert_allclose(packed[b, j, i, d_c:], R @ q_r[b, j, i], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# chunked prefill (un-absorbed form over the latent cache)
# --------------------------------------------------------------------------
def test_prefill_chunk_equals_absorbed_decode_of_every_token():
    """The un-absorbed chunk equals, token by token, the absorbed decode of
    that token at its own position followed by W^UV (associativity, [MLA-93]
    Core Mechanics 3), with the causal rule of the decode (each token sees the
    cache up to and including itself)."""
    rng = np.random.default_rng(120)
    H, d_c, d_r, d_nope, d_v, T, C = 3, 8, 4, 5, 6, 11, 4
    rows = rng.standard_normal((T, d_c + d_r))
    q_in = rng.standard_normal((C, H, d_nope + d_r))
    w_uk = rng.standard_normal((H, d_nope, d_c)) / math.sqrt(d_c)
    w_uv = rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c)
    scale = O.softmax_scale(d_nope, d_r)
    o = O.prefill_chunk(q_in, rows, w_uk, w_uv, d_c, d_nope, scale)
    assert o.shape == (C, H, d_v)
    for i in range(C):
        p = T - C + i
        q = O.absorb_query(q_in[i:i + 1, :, :d_nope], q_in[i:i + 1, :, d_nope:], w_uk, np.array([p]))
        u, _ = O.attend_absorbed(q, rows[:p + 1], 1, d_c, scale)
        np.testing.assert_allclose(o[i], O.out_proj(u, w_uv)[0], rtol=1e-11, atol=1e-12)


def test_prefill_chunk_split_in_two_gives_the_same_outputs():
    """A prompt processed as one chunk or as two consecutive chunks (the
    second seeing the first through the cache) gives every token the same
    output: chunking changes the schedule, not the attention."""
    rng = np.random.default_rng(121)
    H, d_c, d_r, d_nope, d_v, T0, C = 2, 8, 4, 5, 6, 7, 6
    rows = rng.standard_normal((T0 + C, d_c + d_r))
    q_in = rng.standard_normal((C, H, d_nope + d_r))
    w_uk = rng.standard_normal((H, d_nope, d_c)) / math.sqrt(d_c)
    w_uv = rng.standard_normal((H, d_v, d_c)) / math.sqrt(d_c)
    scale = O.softmax_scale(d_nope, d_r)
    whole = O.prefill_chunk(q_in, rows, w_uk, w_uv, d_c, d_nope, scale)
    first = O.prefill_chunk(q_in[:2], rows[:T0 + 2], w_uk, w_uv, d_c, d_nope, scale)
    second = O.prefill_chunk(q_in[2:], rows, w_uk, w_uv, d_c, d_nope, scale)
    np.testing.assert_allclose(np.concatenate([first, second]), whole, rtol=1e-12, atol=1e-13)

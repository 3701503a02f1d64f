"""CPU oracle for MLA decode over a paged latent cache.  TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its Python binding)
never imports, links or calls anything here, and this module never imports
the product path.

Everything is computed in float64 from inputs that are upcast exactly from
the stored values (fp32, bf16 bit patterns, or e4m3 codes times fp32 scales).
The arithmetic is the plain definition, step by step, with no blocking,
fusion or reordering.  The functions the benchmark's CPU baseline runs
(``kv_rows``, ``absorb_query``, ``decode`` / ``attend_absorbed``,
``out_proj``) take a ``dtype`` argument so that the same steps can be timed
in float32; every parity test uses the float64 default.

Sources (page titles; sections named on each page):

* [MLA-93]  "DeepSeek MLA Architecture: How Multi-Head Latent Attention Cuts
            KV Cache by 93%" -- "Core Mechanics" 1 (low-rank KV compression),
            2 (RoPE non-commutativity), 3 (decoupled RoPE and matrix
            absorption); "Total Cached Scalars per Token"; the section
            "Production PyTorch Implementation: Single-Token MLA Decoding"
            (the rotation it applies and its decoding procedure).
* [V3-ARCH] "DeepSeek-V3 Architecture: Multi-Head Latent Attention (MLA) &
            FP8 Mixed-Precision Training" -- 1 "The Memory Wall",
            2 "MLA Mathematics", A "Decoupled RoPE", 3 "Matrix Absorption".
* [DUALPIPE] "DeepSeek Unveils DualPipe & Multi-Head Latent Attention ..."
            -- FP8 training with tile-level quantisation and per-tile scales.
* OCP 8-bit floating point specification, E4M3 encoding (no infinities,
  max finite 448): the fp8 cache format.

Readings where the pages leave a step open are listed in the design notes;
the ones this file depends on are restated where they are used.

Parity status: every function here is pinned by tests under ``tests/``
(brute force, library routines, closed forms, invariants, the pages' printed
numbers).  None is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Callable, Iterable, List, Sequence, Tuple

import numpy as np
import torch

# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits).astype(np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_bf16_bits(x) -> np.ndarray:
    """Round to bf16 (round-to-nearest-even, via fp32) and return bit patterns."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def round_bf16(x) -> np.ndarray:
    """Values rounded to bf16 the way a device with fp32 results stores them."""
    return bf16_bits_to_f64(to_bf16_bits(x))


E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """OCP E4M3 code -> float64.

    Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
    field 0 encodes subnormals m * 2^-9; S.1111.111 is NaN; there are no
    infinities, so S.1111.110 = 448 is the largest finite magnitude.
    """
    c = np.asarray(codes).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return s * val


def e4m3_encode(x) -> np.ndarray:
    """fp32 -> OCP E4M3 code, round-to-nearest-even with saturation to +-448.

    The rounding is the library's float8_e4m3fn cast; magnitudes are first
    clamped to 448 so that out-of-range values saturate instead of becoming
    NaN.  (Any |x| in [448, 464) rounds to 448 under RNE anyway, so the clamp
    only changes values that would otherwise overflow.)
    """
    t = torch.as_tensor(np.asarray(x, dtype=np.float32))
    t = torch.clamp(t, -E4M3_MAX, E4M3_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def fp8_tiles(d: int, tile: int = 128) -> List[Tuple[int, int]]:
    """Channel ranges [lo, hi) of the per-token quantisation tiles of a row."""
    return [(lo, min(lo + tile, d)) for lo in range(0, d, tile)]


def quantize_fp8_row(row) -> Tuple[np.ndarray, np.ndarray]:
    """Tile-scaled e4m3 encoding of one cached row ([DUALPIPE] FP8 paragraph).

    For each 128-channel tile (the last may be shorter): a = max |r| over the
    tile; a = 0 gives scale 1 and zero codes; otherwise scale = a / 448 and
    code = e4m3(r * (448 / a)).  The decisions are taken in fp32: 448/a is
    one correctly rounded fp32 division and r * (448/a) one fp32 product.
    Returns (codes uint8 [D], scales fp32 [n_tiles]).
    """
    r = np.asarray(row, dtype=np.float32)
    tiles = fp8_tiles(r.shape[-1])
    codes = np.zeros(r.shape, dtype=np.uint8)
    scales = np.ones(len(tiles), dtype=np.float32)
    for k, (lo, hi) in enumerate(tiles):
        a = np.float32(np.max(np.abs(r[lo:hi])))
        if a == 0:
            continue
        inv = np.float32(np.float32(E4M3_MAX) / a)
        scales[k] = np.float32(a / np.float32(E4M3_MAX))
        codes[lo:hi] = e4m3_encode((r[lo:hi] * inv).astype(np.float32))
    return codes, scales


def pow2_scale_exponent(a: float) -> int:
    """The smallest integer E with a <= 448 * 2^E, for a > 0.

    A power-of-two tile scale 2^E maps the tile's largest magnitude a into
    (224, 448]: the top binade of e4m3.  The pages ask for a scaling factor
    per tile ([DUALPIPE] FP8 paragraph) without fixing its number format; a
    power of two is the reading under which the scale can be applied by
    exponent arithmetic alone.  The comparisons below are exact in float64.
    """
    a = float(a)
    e = math.ceil(math.log2(a / E4M3_MAX))
    while a > E4M3_MAX * 2.0 ** e:
        e += 1
    while a <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return e


def quantize_fp8_rows(rows, pow2_scales: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """``quantize_fp8_row`` applied to every row of [N, D] (vectorised over N).

    With ``pow2_scales`` each nonzero tile's scale is 2^E with
    E = ``pow2_scale_exponent(a)`` (a = the tile's max |r|) and code =
    e4m3(r * 2^-E), an exact fp32 scaling; zero tiles keep scale 1 and zero
    codes.  The stored scale is still one fp32 value per (token, tile).
    """
    r = np.asarray(rows, dtype=np.float32)
    tiles = fp8_tiles(r.shape[-1])
    codes = np.zeros(r.shape, dtype=np.uint8)
    scales = np.ones(r.shape[:-1] + (len(tiles),), dtype=np.float32)
    for k, (lo, hi) in enumerate(tiles):
        a = np.max(np.abs(r[..., lo:hi]), axis=-1).astype(np.float32)
        nz = a != 0
        safe = np.where(nz, a, np.float32(1)).astype(np.float32)
        if pow2_scales:
            ex = np.array([pow2_scale_exponent(v) for v in safe.reshape(-1)], dtype=np.float64)
            sc = np.exp2(ex).reshape(safe.shape).astype(np.float32)
            inv = (np.float32(1) / sc).astype(np.float32)  # exact: a power of two
            scales[..., k] = np.where(nz, sc, np.float32(1))
        else:
            inv = (np.float32(E4M3_MAX) / safe).astype(np.float32)
            scales[..., k] = np.where(nz, (safe / np.float32(E4M3_MAX)).astype(np.float32),
                                      np.float32(1))
        x = (r[..., lo:hi] * inv[..., None]).astype(np.float32)
        codes[..., lo:hi] = np.where(nz[..., None], e4m3_encode(x), np.uint8(0))
    return codes, scales


def quantize_rows_e4m3_pow2(x) -> np.ndarray:
    """Each row of x (last axis) rounded to e4m3 under one power-of-two scale.

    The value an fp8 product sees for a query quantised with one scale per
    head: scale 2^E with E = ``pow2_scale_exponent(max |row|)``, value =
    e4m3(row * 2^-E) * 2^E (all-zero rows stay zero).  Returns float64 values.
    """
    r = np.asarray(x, dtype=np.float32)
    flat = r.reshape(-1, r.shape[-1])
    out = np.zeros(flat.shape, dtype=np.float64)
    for i, row in enumerate(flat):
        a = float(np.max(np.abs(row)))
        if a == 0:
            continue
        e = pow2_scale_exponent(a)
        codes = e4m3_encode((row * np.float32(2.0 ** -e)).astype(np.float32))
        out[i] = e4m3_decode(codes) * 2.0 ** e
    return out.reshape(r.shape)


def dequantize_fp8_rows(codes, scales) -> np.ndarray:
    """Decoded value = float(code) * scale of its tile, in float64."""
    c = np.asarray(codes)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    out = e4m3_decode(c)
    for k, (lo, hi) in enumerate(fp8_tiles(c.shape[-1])):
        out[..., lo:hi] *= s[..., k:k + 1]
    return out


# --------------------------------------------------------------------------
# RoPE ([MLA-93] Core Mechanics 2 and 3, and the rotation used in its decoding section)
# --------------------------------------------------------------------------

def rope_angles(n: int, pos: float, base: float = 10000.0) -> np.ndarray:
    """theta_j = pos * base^(-j / (n/2)) for j < n/2, in float64."""
    half = n // 2
    j = np.arange(half, dtype=np.float64)
    return float(pos) * np.power(float(base), -j / half)


def rope(x, pos, base: float = 10000.0) -> np.ndarray:
    """Rotate-half RoPE of the last axis (length n, even).

    Channel j is paired with channel j + n/2 and the pair is rotated by
    theta_j:  y_j = x_j cos - x_{j+h} sin,  y_{j+h} = x_{j+h} cos + x_j sin.
    ``pos`` may be a scalar or an array broadcasting against x[..., 0].
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    assert n % 2 == 0
    h = n // 2
    pos = np.asarray(pos, dtype=np.float64)[..., None]
    j = np.arange(h, dtype=np.float64)
    theta = pos * np.power(float(base), -j / h)
    c, s = np.cos(theta), np.sin(theta)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# --------------------------------------------------------------------------
# cache append ([MLA-93] Core Mechanics 1 and 3; decoding section)
# --------------------------------------------------------------------------

def kv_rows(h, w_dkv, w_kr, positions, base: float = 10000.0, dtype=np.float64) -> np.ndarray:
    """Cached rows [c ; k^R] for hidden states h [T, d_model].

    c = W^DKV h (W^DKV: [d_c, d_model]); k^R = RoPE(W^KR h, pos)
    (W^KR: [d_R, d_model]).  Returns [T, d_c + d_R] (float64 by default).
    """
    h = np.asarray(h, dtype=dtype)
    c = h @ np.asarray(w_dkv, dtype=dtype).T
    kr = rope(h @ np.asarray(w_kr, dtype=dtype).T, np.asarray(positions), base).astype(dtype)
    return np.concatenate([c, kr], axis=-1)


def slot_of(page_table, b: int, pos: int, block_size: int) -> Tuple[int, int]:
    """(physical block, offset) of logical position ``pos`` of sequence b."""
    return int(page_table[b][pos // block_size]), pos % block_size


def append(pool: dict, h, w_dkv, w_kr, seq_ids, positions, page_table,
           block_size: int, base: float = 10000.0) -> None:
    """Write the projected rows of tokens into a paged pool (in place).

    ``pool`` is {"dtype": "fp32"|"bf16"|"fp8", "data": array [nblk, bs, D]
    (float32 / uint16 bf16 bits / uint8 codes), "scales": float32
    [nblk, bs, n_tiles] (fp8 only)}.  Rows are computed in float64, rounded
    to fp32 (the device keeps fp32 results), then stored in the cache format.
    """
    rows = kv_rows(h, w_dkv, w_kr, positions, base).astype(np.float32)
    for i in range(rows.shape[0]):
        blk, off = slot_of(page_table, int(seq_ids[i]), int(positions[i]), block_size)
        if pool["dtype"] == "fp32":
            pool["data"][blk, off] = rows[i]
        elif pool["dtype"] == "bf16":
            pool["data"][blk, off] = to_bf16_bits(rows[i])
        elif pool["dtype"] == "fp8":
            codes, scales = quantize_fp8_row(rows[i])
            pool["data"][blk, off] = codes
            pool["scales"][blk, off] = scales
        else:
            raise ValueError(pool["dtype"])


def pool_values(pool: dict, blocks=None) -> np.ndarray:
    """Decoded float64 values of (a subset of) the pool's blocks."""
    sel = slice(None) if blocks is None else np.asarray(blocks)
    data = pool["data"][sel]
    if pool["dtype"] == "fp32":
        return data.astype(np.float64)
    if pool["dtype"] == "bf16":
        return bf16_bits_to_f64(data)
    if pool["dtype"] == "fp8":
        return dequantize_fp8_rows(data, pool["scales"][sel])
    raise ValueError(pool["dtype"])


def gather_sequence(pool: dict, page_table, b: int, length: int, block_size: int) -> np.ndarray:
    """Rows 0..length-1 of sequence b, read through its page table, float64 [L, D]."""
    nblk = (length + block_size - 1) // block_size
    blocks = np.asarray(page_table[b][:nblk], dtype=np.int64)
    vals = pool_values(pool, blocks).reshape(nblk * block_size, -1)
    return vals[:length]


# --------------------------------------------------------------------------
# attention over the latent cache
# --------------------------------------------------------------------------

def softmax_scale(d_nope: int, d_rope: int) -> float:
    """1 / sqrt(d_nope + d_R): the per-head key is 192-wide for DeepSeek dims
    ([MLA-93] Core Mechanics 3 and the scale its decoding section uses)."""
    return 1.0 / math.sqrt(d_nope + d_rope)


def visible(seq_len: int, n_q: int, j: int) -> int:
    """Number of positions query j of a sequence attends to.

    The new tokens join the cache before attention, so query j (at position
    seq_len - n_q + j) sees positions 0 .. seq_len - n_q + j, itself included.
    """
    return seq_len - n_q + j + 1


def attend_absorbed(q_b, rows, n_q: int, d_latent: int, scale: float, dtype=np.float64):
    """Absorbed-form attention for one sequence.

    q_b: [n_q, H, d_c + d_R] packed [q~ ; q^R]; rows: [L, d_c + d_R] cached
    [c ; k^R].  Score s_t = scale * (q~ . c_t + q^R . k^R_t); p = softmax over
    the visible positions; u = sum_t p_t c_t ([MLA-93] Core Mechanics 3, the
    absorbed query and latent value aggregation).
    Returns u [n_q, H, d_c] and lse [n_q, H] (natural log), float64 by default.
    """
    q_b = np.asarray(q_b, dtype=dtype)
    rows = np.asarray(rows, dtype=dtype)
    L = rows.shape[0]
    n_heads = q_b.shape[1]
    u = np.zeros((n_q, n_heads, d_latent), dtype=dtype)
    lse = np.zeros((n_q, n_heads), dtype=dtype)
    for j in range(n_q):
        n = visible(L, n_q, j)
        s = dtype(scale) * (q_b[j] @ rows[:n].T)           # [H, n]
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        z = e.sum(axis=1, keepdims=True)
        u[j] = (e / z) @ rows[:n, :d_latent]
        lse[j] = (m + np.log(z))[:, 0]
    return u, lse


def decode(q, pool: dict, page_table, seq_lens, block_size: int, d_latent: int,
           scale: float, batch_ids: Iterable[int] = None, dtype=np.float64):
    """Absorbed decode of a batch (or of the listed sequences).

    q: [B, n_q, H, D].  Returns dict b -> (u [n_q, H, d_c], lse [n_q, H]).
    """
    q = np.asarray(q)
    n_q = q.shape[1]
    out = {}
    ids = range(q.shape[0]) if batch_ids is None else batch_ids
    for b in ids:
        rows = gather_sequence(pool, page_table, b, int(seq_lens[b]), block_size)
        out[b] = attend_absorbed(q[b], rows, n_q, d_latent, scale, dtype)
    return out


def attend_unabsorbed(q_c, q_r, rows, w_uk, w_uv, n_q: int, d_latent: int, scale: float):
    """Un-absorbed (explicit K, V) attention for one sequence.

    Per head i: k_{t,i} = [W^UK_i c_t ; k^R_t] (192-wide for DeepSeek dims),
    v_{t,i} = W^UV_i c_t; s = scale * [q^C_i ; q^R_i] . k_{t,i};
    o_i = sum_t p_t v_{t,i} ([MLA-93] Core Mechanics 3; [V3-ARCH] A).
    q_c: [n_q, H, d_nope]; q_r: [n_q, H, d_R] (already rotated);
    w_uk: [H, d_nope, d_c]; w_uv: [H, d_v, d_c].  Returns o [n_q, H, d_v].
    """
    rows = np.asarray(rows, dtype=np.float64)
    c, kr = rows[:, :d_latent], rows[:, d_latent:]
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    L = rows.shape[0]
    n_heads = w_uk.shape[0]
    o = np.zeros((n_q, n_heads, w_uv.shape[1]))
    for i in range(n_heads):
        k_c = c @ w_uk[i].T                                 # [L, d_nope]
        v = c @ w_uv[i].T                                   # [L, d_v]
        k = np.concatenate([k_c, kr], axis=1)               # [L, d_nope + d_R]
        for j in range(n_q):
            n = visible(L, n_q, j)
            qv = np.concatenate([np.asarray(q_c[j, i], np.float64),
                                 np.asarray(q_r[j, i], np.float64)])
            s = scale * (k[:n] @ qv)
            p = np.exp(s - s.max())
            p /= p.sum()
            o[j, i] = p @ v[:n]
    return o


def prefill_chunk(q_in, rows, w_uk, w_uv, d_latent: int, d_nope: int, scale: float,
                  base: float = 10000.0):
    """A prefill chunk over the latent cache in the un-absorbed form.

    The prefill phase processes many prompt tokens at once ([MLA-93], the
    prefill/decode contrast at its start); for a long chunk the per-head keys
    and values are expanded from the cached latents once (k = [W^UK_i c ; k^R],
    v = W^UV_i c) and attention runs in the usual form.  q_in: [C, H, d_nope +
    d_R] per head q^C and the not yet rotated q^R of the chunk's C tokens;
    rows: [T, D] the cached rows of the sequence, the chunk's own C rows last
    (chunk token i sits at position T - C + i and sees positions 0 .. T - C + i).
    q^R is rotated at each token's position.  Returns o [C, H, d_v].
    """
    q_in = np.asarray(q_in, dtype=np.float64)
    C = q_in.shape[0]
    T = np.asarray(rows).shape[0]
    pos = np.arange(T - C, T, dtype=np.float64)
    q_r = rope(q_in[..., d_nope:], pos[:, None], base)
    return attend_unabsorbed(q_in[..., :d_nope], q_r, rows, w_uk, w_uv, C, d_latent, scale)


def attend_bruteforce(q_b, rows, n_q: int, d_latent: int, scale: float):
    """Explicit loops, softmax as exp(s) / sum exp(s) with no max shift.

    Tiny inputs only.  Returns u [n_q, H, d_c] and lse [n_q, H].
    """
    q_b = np.asarray(q_b, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    L, D = rows.shape
    n_heads = q_b.shape[1]
    u = np.zeros((n_q, n_heads, d_latent))
    lse = np.zeros((n_q, n_heads))
    for j in range(n_q):
        n = visible(L, n_q, j)
        for i in range(n_heads):
            ex = []
            for t in range(n):
                dot = 0.0
                for k in range(D):
                    dot += q_b[j, i, k] * rows[t, k]
                ex.append(math.exp(scale * dot))
            z = sum(ex)
            for k in range(d_latent):
                acc = 0.0
                for t in range(n):
                    acc += ex[t] * rows[t, k]
                u[j, i, k] = acc / z
            lse[j, i] = math.log(z)
    return u, lse


# --------------------------------------------------------------------------
# split-KV partials and log-sum-exp merge
# --------------------------------------------------------------------------

def attend_partial(q_row, rows, lo: int, hi: int, d_latent: int, scale: float):
    """Softmax restricted to positions [lo, hi) for query rows q_row [R, D].

    Returns (o [R, d_c], lse [R]); an empty range gives o = 0, lse = -inf.
    """
    q_row = np.asarray(q_row, dtype=np.float64)
    if hi <= lo:
        return np.zeros((q_row.shape[0], d_latent)), np.full(q_row.shape[0], -np.inf)
    r = np.asarray(rows[lo:hi], dtype=np.float64)
    s = scale * (q_row @ r.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ r[:, :d_latent], (m + np.log(z))[:, 0]


def combine(o_parts, lse_parts):
    """Merge split results: M = max_s lse_s, w_s = exp(lse_s - M),
    u = sum_s w_s o_s / sum_s w_s, lse = M + ln sum_s w_s.

    o_parts: [S, ..., d_c], lse_parts: [S, ...].  Splits with lse = -inf get
    weight 0.  Returns (u, lse).
    """
    o = np.asarray(o_parts, dtype=np.float64)
    l = np.asarray(lse_parts, dtype=np.float64)
    M = l.max(axis=0)
    w = np.exp(l - M)
    z = w.sum(axis=0)
    u = (w[..., None] * o).sum(axis=0) / z[..., None]
    return u, M + np.log(z)


# --------------------------------------------------------------------------
# per-head value up-projection ([MLA-93] decoding section)
# --------------------------------------------------------------------------

def out_proj(u, w_uv, dtype=np.float64) -> np.ndarray:
    """o[r, i, :] = W^UV_i u[r, i, :] with W^UV: [H, d_v, d_c]."""
    u = np.asarray(u, dtype=dtype)
    w = np.asarray(w_uv, dtype=dtype)
    return np.einsum("rid,ivd->riv", u, w)


# --------------------------------------------------------------------------
# query side ([MLA-93] decoding section and Core Mechanics 3)
# --------------------------------------------------------------------------

def split_query(qfull, n_heads: int, d_nope: int, d_rope: int):
    """[.., H*(d_nope+d_R)] -> (q^C [.., H, d_nope], q^R [.., H, d_R]), head-major."""
    q = np.asarray(qfull, dtype=np.float64)
    q = q.reshape(q.shape[:-1] + (n_heads, d_nope + d_rope))
    return q[..., :d_nope], q[..., d_nope:]


def absorb_query(q_c, q_r, w_uk, pos, base: float = 10000.0, dtype=np.float64):
    """Packed absorbed query [q~ ; RoPE(q^R, pos)].

    q~_i = (W^UK_i)^T q^C_i in R^{d_c}: the associativity regrouping of
    Core Mechanics 3.  q_c: [.., H, d_nope]; q_r: [.., H, d_R];
    w_uk: [H, d_nope, d_c]; pos broadcasts against the leading axes.
    """
    q_c = np.asarray(q_c, dtype=dtype)
    w = np.asarray(w_uk, dtype=dtype)
    q_t = np.einsum("...in,inc->...ic", q_c, w)
    pos = np.asarray(pos, dtype=np.float64)
    q_rr = rope(q_r, pos[..., None] if pos.ndim else pos, base).astype(dtype)
    return np.concatenate([q_t, q_rr], axis=-1)


def query_from_hidden(h_q, w_q, w_uk, pos, n_heads: int, d_nope: int, d_rope: int,
                      base: float = 10000.0):
    """Single-projection query path of the tiny workload.

    W^Q h -> [H, d_nope + d_R] head-major; the first d_nope entries are q^C,
    the rest q^R; q^R is rotated at the query's position; then absorbed.
    Returns (packed [.., H, d_c + d_R], q^C, rotated q^R).
    """
    qfull = np.asarray(h_q, dtype=np.float64) @ np.asarray(w_q, dtype=np.float64).T
    q_c, q_r = split_query(qfull, n_heads, d_nope, d_rope)
    packed = absorb_query(q_c, q_r, w_uk, pos, base)
    pos_a = np.asarray(pos, dtype=np.float64)
    q_rr = rope(q_r, pos_a[..., None] if pos_a.ndim else pos_a, base)
    return packed, q_c, q_rr


# --------------------------------------------------------------------------
# the decoding section's dense layers: the low-rank query path and W^O
# ([MLA-93] decoding section: its W_DQ, W_UQ, W_QR and W_O Linears)
# --------------------------------------------------------------------------

def linear(x, w) -> np.ndarray:
    """A bias-free linear layer y = x W^T, with W stored [n, k] as a torch
    Linear keeps it (the module's every projection is bias-free)."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def query_lowrank(h, w_dq, w_uq, w_qr, n_heads: int, d_nope: int, d_rope: int):
    """Step 2 of the decoding procedure: the compressed query c^Q = W^DQ h,
    then q^C = W^UQ c^Q and q^R = W^QR c^Q, each viewed head-major as
    [.., H, d_nope] and [.., H, d_R] (q^R not yet rotated)."""
    c_q = linear(h, w_dq)
    q_c = linear(c_q, w_uq)
    q_r = linear(c_q, w_qr)
    return (q_c.reshape(q_c.shape[:-1] + (n_heads, d_nope)),
            q_r.reshape(q_r.shape[:-1] + (n_heads, d_rope)))


def output_projection(v, w_o) -> np.ndarray:
    """The module's last step: the per-head outputs v [.., H, d_v] are laid
    end to end (head-major, [.., H * d_v]) and projected by W^O [d, H d_v]."""
    v = np.asarray(v, dtype=np.float64)
    return linear(v.reshape(v.shape[:-2] + (v.shape[-2] * v.shape[-1],)), w_o)


# --------------------------------------------------------------------------
# footprint arithmetic ([MLA-93] bottleneck and cached-scalar sections;
# [V3-ARCH] 1)
# --------------------------------------------------------------------------

def cached_scalars_per_token(d_latent: int, d_rope: int) -> int:
    """Scalars cached per token per layer: the latent plus the shared RoPE key."""
    return d_latent + d_rope


def mha_cache_bytes(n_layers, n_kv, d_h, bytes_per_el, batch, length) -> float:
    """Standard K+V cache: two tensors of n_kv * d_h per token per layer."""
    return 2 * n_layers * n_kv * d_h * bytes_per_el * batch * length


def pool_bytes(num_blocks: int, block_size: int, d_latent: int, d_rope: int,
               elem_bytes: int, scale_tiles: int = 0) -> int:
    """Device bytes of a paged pool (plus per-token fp32 scales for fp8)."""
    per_tok = (d_latent + d_rope) * elem_bytes + 4 * scale_tiles
    return num_blocks * block_size * per_tok

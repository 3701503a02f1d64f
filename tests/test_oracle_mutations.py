"""Plant plausible mistakes in the oracle (CPU only) and check a pin catches each.

Every case monkeypatches one oracle function with a subtly wrong variant and
runs the pins that should reject it; the test passes only if one of them fails.
"""
import math

import numpy as np
import pytest

from oracle import mla_oracle as O
from tests import test_oracle_pins as P


def _rope_interleaved(x, pos, base=10000.0):
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    h = n // 2
    pos = np.asarray(pos, dtype=np.float64)[..., None]
    th = pos * np.power(base, -np.arange(h) / h)
    c, s = np.cos(th), np.sin(th)
    y = x.copy()
    y[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    y[..., 1::2] = x[..., 1::2] * c + x[..., 0::2] * s
    return y


def _rope_sign(x, pos, base=10000.0):
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    pos = np.asarray(pos, dtype=np.float64)[..., None]
    th = pos * np.power(base, -np.arange(h) / h)
    c, s = np.cos(th), np.sin(th)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c + hi * s, hi * c - lo * s], -1)


def _rope_freq(x, pos, base=10000.0):
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    h = n // 2
    pos = np.asarray(pos, dtype=np.float64)[..., None]
    th = pos * np.power(base, -np.arange(h) / n)
    c, s = np.cos(th), np.sin(th)
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], -1)


_orig_pow2_exp = O.pow2_scale_exponent
_orig_qrows = O.quantize_fp8_rows


def _query_quant_shared_scale(x):
    r = np.asarray(x, dtype=np.float32)
    e = _orig_pow2_exp(float(np.max(np.abs(r))))
    return O.e4m3_decode(O.e4m3_encode((r * np.float32(2.0 ** -e)).astype(np.float32))) * 2.0 ** e


_orig_absorbed = O.attend_absorbed


def _absorbed_no_rope_term(q_b, rows, n_q, d_latent, scale):
    q = np.array(q_b, dtype=np.float64)
    q[..., d_latent:] = 0
    return _orig_absorbed(q, rows, n_q, d_latent, scale)


def _combine_unweighted(o_parts, lse_parts):
    o = np.asarray(o_parts, dtype=np.float64)
    l = np.asarray(lse_parts, dtype=np.float64)
    return o.mean(0), l.max(0)


def _encode_no_saturation(x):
    import torch
    t = __import__("torch").as_tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def _lowrank_views_swapped(h, w_dq, w_uq, w_qr, n_heads, d_nope, d_rope):
    # q^C viewed dimension-major ([d_nope, H] then transposed) instead of head-major
    c_q = O.linear(h, w_dq)
    q_c = O.linear(c_q, w_uq)
    q_r = O.linear(c_q, w_qr)
    q_c = np.swapaxes(q_c.reshape(q_c.shape[:-1] + (d_nope, n_heads)), -1, -2)
    return q_c, q_r.reshape(q_r.shape[:-1] + (n_heads, d_rope))


def _output_projection_dv_major(v, w_o):
    v = np.asarray(v, dtype=np.float64)
    return O.linear(np.swapaxes(v, -1, -2).reshape(v.shape[:-2] + (-1,)), w_o)


def _dequant_tile0_scale(codes, scales):
    # every tile decoded with tile 0's scale
    c = np.asarray(codes)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    return O.e4m3_decode(c) * s[..., 0:1]


def _dequant_tiles_of_64(codes, scales):
    # tile boundaries every 64 channels instead of 128
    c = np.asarray(codes)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    out = O.e4m3_decode(c)
    for k in range(c.shape[-1] // 64):
        out[..., 64 * k:64 * k + 64] *= s[..., min(k, s.shape[-1] - 1):min(k, s.shape[-1] - 1) + 1]
    return out


_orig_absorb_query = O.absorb_query


def _absorb_unrotated(q_c, q_r, w_uk, pos, base=10000.0):
    return _orig_absorb_query(q_c, q_r, w_uk, np.zeros_like(np.asarray(pos)), base)


def _absorb_first_row_position(q_c, q_r, w_uk, pos, base=10000.0):
    p = np.asarray(pos)
    return _orig_absorb_query(q_c, q_r, w_uk, np.full_like(p, p.flat[0]) if p.ndim else p, base)


def _prefill_positions_from_zero(q_in, rows, w_uk, w_uv, d_latent, d_nope, scale, base=10000.0):
    # q^R rotated at 0 .. C-1 instead of the tokens' own positions
    q_in = np.asarray(q_in, dtype=np.float64)
    C = q_in.shape[0]
    q_r = O.rope(q_in[..., d_nope:], np.arange(C, dtype=np.float64)[:, None], base)
    return O.attend_unabsorbed(q_in[..., :d_nope], q_r, rows, w_uk, w_uv, C, d_latent, scale)


def _prefill_not_causal(q_in, rows, w_uk, w_uv, d_latent, d_nope, scale, base=10000.0):
    # every chunk token sees the whole chunk
    q_in = np.asarray(q_in, dtype=np.float64)
    C, T = q_in.shape[0], np.asarray(rows).shape[0]
    pos = np.arange(T - C, T, dtype=np.float64)
    q_r = O.rope(q_in[..., d_nope:], pos[:, None], base)
    return np.concatenate([O.attend_unabsorbed(q_in[i:i + 1, :, :d_nope], q_r[i:i + 1], rows, w_uk, w_uv, 1,
                                               d_latent, scale) for i in range(C)])


MUTANTS = {
    "prefill_rope_positions_from_zero": ("prefill_chunk", _prefill_positions_from_zero,
                                         [P.test_prefill_chunk_equals_absorbed_decode_of_every_token]),
    "prefill_not_causal": ("prefill_chunk", _prefill_not_causal,
                           [P.test_prefill_chunk_equals_absorbed_decode_of_every_token,
                            P.test_prefill_chunk_split_in_two_gives_the_same_outputs]),
    "fp8_dequant_tile0_scale": ("dequantize_fp8_rows", _dequant_tile0_scale,
                                [P.test_dequantize_fp8_rows_per_tile_scales]),
    "fp8_dequant_tiles_of_64": ("dequantize_fp8_rows", _dequant_tiles_of_64,
                                [P.test_dequantize_fp8_rows_per_tile_scales]),
    "absorb_query_rope_unrotated": ("absorb_query", _absorb_unrotated,
                                    [P.test_absorbed_query_rope_half_is_rotated_at_each_rows_position]),
    "absorb_query_rope_first_row_position": (
        "absorb_query", _absorb_first_row_position,
        [P.test_absorbed_query_rope_half_is_rotated_at_each_rows_position]),
    "linear_dropped_last_k": ("linear", lambda x, w: np.asarray(x, np.float64)[..., :-1]
                              @ np.asarray(w, np.float64)[:, :-1].T,
                              [P.test_linear_explicit_loops]),
    "lowrank_query_dim_major_view": ("query_lowrank", _lowrank_views_swapped,
                                     [P.test_lowrank_query_equals_composed_single_projection]),
    "output_projection_dv_major": ("output_projection", _output_projection_dv_major,
                                   [P.test_output_projection_equals_fused_w_ov]),
    "rope_interleaved_pairs": ("rope", _rope_interleaved,
                               [P.test_rope_pairs_channel_j_with_j_plus_half]),
    "rope_sign_flip": ("rope", _rope_sign, [P.test_rope_two_dims_is_textbook_rotation]),
    "rope_freq_over_n": ("rope", _rope_freq, [P.test_rope_pairs_channel_j_with_j_plus_half]),
    "scale_over_full_row": ("softmax_scale", lambda dn, dr: 1.0 / math.sqrt(dn + 2 * dr + 8),
                            [P.test_unabsorbed_matches_library_attention]),
    "query_excludes_itself": ("visible", lambda L, n_q, j: L - n_q + j,
                              [P.test_decode_special_cases,
                               P.test_unabsorbed_matches_library_attention]),
    "dropped_rope_score_term": ("attend_absorbed", _absorbed_no_rope_term,
                                [P.test_unabsorbed_matches_library_attention]),
    "out_proj_transposed": ("out_proj", lambda u, w: np.einsum("rid,idv->riv", np.asarray(u),
                                                               np.asarray(w).transpose(0, 1, 2)),
                            [P.test_out_proj_explicit_loops]),
    "combine_unweighted": ("combine", _combine_unweighted,
                           [P.test_combine_of_any_partition_equals_unsplit]),
    "fp8_no_saturation": ("e4m3_encode", _encode_no_saturation,
                          [P.test_e4m3_encode_round_trip_ties_and_saturation]),
    "fp8_scale_off": ("E4M3_MAX", 447.0, [P.test_fp8_row_quantizer_properties]),
    "pow2_exponent_floor": ("pow2_scale_exponent", lambda a: math.floor(math.log2(float(a) / 448.0)),
                            [P.test_pow2_scale_exponent_brute_force_and_boundaries,
                             P.test_fp8_pow2_quantizer_properties]),
    "pow2_exponent_one_high": ("pow2_scale_exponent", lambda a: _orig_pow2_exp(a) + 1,
                               [P.test_fp8_pow2_quantizer_properties, P.test_query_rows_e4m3_pow2]),
    "pow2_scales_ignored": ("quantize_fp8_rows", lambda rows, pow2_scales=False: _orig_qrows(rows),
                            [P.test_fp8_pow2_quantizer_properties]),
    "query_quant_one_scale_for_all_rows": ("quantize_rows_e4m3_pow2", _query_quant_shared_scale,
                                           [P.test_query_rows_e4m3_pow2]),
    "bf16_truncation": ("to_bf16_bits",
                        lambda x: (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16),
                        [P.test_bf16_rounding_known_values]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, repl, pins = MUTANTS[name]
    monkeypatch.setattr(O, attr, repl)
    caught = False
    for pin in pins:
        try:
            if "n" in pin.__code__.co_varnames[:pin.__code__.co_argcount]:
                pin(8)
            elif "n_q" in pin.__code__.co_varnames[:pin.__code__.co_argcount]:
                pin(2)
            elif "dtype" in pin.__code__.co_varnames[:pin.__code__.co_argcount]:
                pin("fp32")
            else:
                pin()
        except Exception:
            caught = True
    assert caught, f"no pin rejected the planted mistake {name}"

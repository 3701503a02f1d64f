"""GPU parity of the chunked prefill (mla_prefill) against the oracle.

A chunk of C prompt tokens attends causally to its sequence's T cached rows
(its own C rows last) in the un-absorbed form.  Bars as for the bf16 decode:
relative L2 <= 1e-2 and max-abs <= 2e-2 against the float64 oracle; the
expanded keys and values and the probabilities are rounded to bf16 on the GPU.
Heads are independent, so the larger cases check a sample of heads against
the oracle run on those heads alone and every output for finiteness.
"""
import dataclasses
import math

import numpy as np
import pytest
import torch

import mla_workloads as W
from oracle import mla_oracle as O
from tests.cases import dims_of, max_abs, rel_l2, to_f64

pytestmark = pytest.mark.gpu

V3 = W.CONFIGS["v3"]


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_decode_amd as M
    M.lib()  # raises if the HIP library is missing: no fallback exists
    return M


class PrefillCase:
    """One sequence of T cached bf16 rows in a shuffled paged pool (unused
    slots and guard blocks hold NaN) and a chunk of C queries and the
    expansion weights, all resident on the GPU."""

    def __init__(self, T: int, C: int, seed: int, cache: str = "bf16"):
        d = self.d = V3.dims
        self.T, self.C = T, C
        lens = np.array([T], np.int32)
        table, nblk = W.page_table(lens, d.block_size, seed, shuffle=True, guard_blocks=2)
        self.table = table
        rows = W.cache_rows(nblk * d.block_size, V3, seed=seed + 10, device="cuda")
        used = torch.zeros(nblk, d.block_size, dtype=torch.bool)
        nb = (T + d.block_size - 1) // d.block_size
        flat = torch.zeros(nb * d.block_size, dtype=torch.bool)
        flat[:T] = True
        used[torch.from_numpy(table[0, :nb].astype(np.int64))] = flat.view(nb, d.block_size)
        self.scales = None
        if cache == "bf16":
            pool = rows.to(torch.bfloat16).view(nblk, d.block_size, d.row)
            pool[(~used).cuda()] = float("nan")
        else:  # e4m3 codes and tile scales from the oracle's encoder; unused slots NaN codes and scales
            codes, sc = O.quantize_fp8_rows(rows.cpu().numpy(), pow2_scales=cache == "fp8p2")
            pool = torch.from_numpy(codes).cuda().view(nblk, d.block_size, d.row)
            scales = torch.from_numpy(sc).cuda().view(nblk, d.block_size, 5)
            pool[(~used).cuda()] = 0x7F
            scales[(~used).cuda()] = float("nan")
            self.scales = scales
        del rows
        self.pool = pool
        self.table_t = torch.from_numpy(table[0]).cuda()
        self.q = W.normal((C, d.num_heads, d.d_nope + d.d_rope), seed + 20, device="cuda").to(torch.bfloat16)
        std = 1 / math.sqrt(d.d_latent)
        self.w_uk = W.normal((d.num_heads, d.d_nope, d.d_latent), seed + 30, std=std, device="cuda").to(torch.bfloat16)
        self.w_uv = W.normal((d.num_heads, d.d_v, d.d_latent), seed + 40, std=std, device="cuda").to(torch.bfloat16)
        self.scale = O.softmax_scale(d.d_nope, d.d_rope)
        self.dims = dims_of(V3 if cache == "bf16" else dataclasses.replace(V3, cache_dtype=cache))

    def run(self):
        import mla_latent_kv_decode_amd as M
        d = self.d
        ws = torch.empty(M.mla_prefill_workspace_size(self.dims, self.C, self.T), dtype=torch.uint8, device="cuda")
        out = torch.empty(self.C, d.num_heads, d.d_v, dtype=torch.bfloat16, device="cuda")
        M.mla_prefill(self.dims, self.q, self.pool, self.table_t, self.T, self.w_uk, self.w_uv, out, ws,
                      cache_scales=self.scales)
        torch.cuda.synchronize()
        return out

    def oracle_rows(self) -> np.ndarray:
        d = self.d
        nb = (self.T + d.block_size - 1) // d.block_size
        idx = torch.from_numpy(self.table[0, :nb].astype(np.int64)).cuda()
        if self.scales is None:
            return to_f64(self.pool.index_select(0, idx)).reshape(nb * d.block_size, d.row)[:self.T]
        codes = self.pool.index_select(0, idx).cpu().numpy().reshape(nb * d.block_size, d.row)[:self.T]
        sc = self.scales.index_select(0, idx).cpu().numpy().reshape(nb * d.block_size, 5)[:self.T]
        return O.dequantize_fp8_rows(codes, sc)

    def oracle(self, heads) -> np.ndarray:
        d = self.d
        hs = torch.as_tensor(heads, device="cuda")
        return O.prefill_chunk(to_f64(self.q.index_select(1, hs)), self.oracle_rows(),
                               to_f64(self.w_uk.index_select(0, hs)), to_f64(self.w_uv.index_select(0, hs)),
                               d.d_latent, d.d_nope, self.scale)


SAMPLE_HEADS = [0, 1, 37, 64, 101, 127]

# (T, C): a whole prompt as one chunk and chunks after a cached prefix, with
# ragged tails against the 32-token key steps and the 128-token query blocks
PREFILL = [
    (1, 1, "all"),           # degenerate: one token attending to itself
    (33, 1, "all"),          # one query, two key steps
    (200, 200, "all"),       # whole prompt, two query blocks, ragged key tail
    (300, 77, "all"),        # chunk after a 223-token prefix
    (129, 128, "sample"),    # prefix of one token, one full query block
    (1000, 130, "sample"),   # 32 key steps, a 2-token second query block
    (2100, 257, "sample"),   # three query blocks
]


@pytest.mark.parametrize("T,C,heads", PREFILL)
def test_prefill_matches_oracle(T, C, heads):
    case = PrefillCase(T, C, seed=500 + T + C)
    out = case.run()
    assert torch.isfinite(out).all()
    hs = list(range(case.d.num_heads)) if heads == "all" else SAMPLE_HEADS
    ref = case.oracle(hs)
    got = to_f64(out)[:, hs]
    assert rel_l2(got, ref) <= 1e-2, (T, C)
    assert max_abs(got, ref) <= 2e-2, (T, C)


@pytest.mark.parametrize("T,C,seed", [(8192, 1024, 77), (16384, 2048, 78), (3000, 3000, 79)])
def test_prefill_full_size_chunk(T, C, seed):
    """The benchmark's chunk shapes (the last C of T tokens) and a whole
    3000-token prompt as one chunk: sampled heads against the oracle, every
    output finite."""
    case = PrefillCase(T, C, seed=seed)
    out = case.run()
    assert torch.isfinite(out).all()
    heads = [0, 77, 127]
    ref = case.oracle(heads)
    got = to_f64(out)[:, heads]
    assert rel_l2(got, ref) <= 1e-2 and max_abs(got, ref) <= 2e-2, (T, C)


@pytest.mark.parametrize("cache", ["fp8", "fp8p2"])
@pytest.mark.parametrize("T,C", [(300, 77), (1000, 257)])
def test_prefill_over_fp8_cache(cache, T, C):
    """An e4m3 cache (tile scales of any value, or powers of two): the gather
    dequantises each value (code x scale, one bf16 rounding, exact for
    powers of two) and the rest is the bf16 path; against the oracle on the
    dequantised rows, with the bf16 bars."""
    case = PrefillCase(T, C, seed=600 + T + C, cache=cache)
    out = case.run()
    assert torch.isfinite(out).all()
    ref = case.oracle(SAMPLE_HEADS)
    got = to_f64(out)[:, SAMPLE_HEADS]
    assert rel_l2(got, ref) <= 1e-2 and max_abs(got, ref) <= 2e-2, (cache, T, C)


def test_prefill_matches_absorbed_decode_on_gpu():
    """The same chunk through the absorbed decode path (q absorbed and rotated
    at positions T - C + j, decode with n_q = C, combine, W^UV projection)
    gives the prefill's outputs: two independent kernels, one result."""
    import mla_latent_kv_decode_amd as M
    case = PrefillCase(700, 90, seed=9)
    d, C, T = case.d, case.C, case.T
    out = case.run()
    pos = torch.arange(T - C, T, dtype=torch.int32, device="cuda")
    q_abs = torch.empty(C, d.num_heads, d.row, dtype=torch.bfloat16, device="cuda")
    M.mla_query_absorb(case.dims, case.q, pos, case.w_uk, q_abs)
    lens = torch.tensor([T], dtype=torch.int32, device="cuda")
    table = case.table_t.view(1, -1)
    ws = torch.empty(M.mla_decode_workspace_size(case.dims, 1, C, 0), dtype=torch.uint8, device="cuda")
    M.mla_decode(case.dims, q_abs.view(1, C, d.num_heads, d.row), case.pool, None, table, lens, ws)
    u = torch.empty(1, C, d.num_heads, d.d_latent, dtype=torch.bfloat16, device="cuda")
    M.mla_decode_combine(case.dims, ws, lens, u)
    o_dec = torch.empty(C, d.num_heads, d.d_v, dtype=torch.bfloat16, device="cuda")
    M.mla_out_proj(case.dims, u.view(C, d.num_heads, d.d_latent), case.w_uv, o_dec)
    torch.cuda.synchronize()
    a, b = to_f64(out), to_f64(o_dec)
    assert rel_l2(a, b) <= 1.5e-2 and max_abs(a, b) <= 3e-2


def test_prefill_rejects_bad_arguments():
    import mla_latent_kv_decode_amd as M
    case = PrefillCase(64, 8, seed=3)
    d = case.d
    out = torch.empty(case.C, d.num_heads, d.d_v, dtype=torch.bfloat16, device="cuda")
    need = M.mla_prefill_workspace_size(case.dims, case.C, case.T)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="workspace"):
        M.mla_prefill(case.dims, case.q, case.pool, case.table_t, case.T, case.w_uk, case.w_uv, out, small)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError):
        M.mla_prefill(case.dims, case.q, case.pool, case.table_t, case.C - 1, case.w_uk, case.w_uv, out, ws)
    assert M.mla_prefill_workspace_size(case.dims, 9, 8) == 0
    # scales exactly for an e4m3 cache
    with pytest.raises(RuntimeError, match="cache_scales"):
        M.mla_prefill(case.dims, case.q, case.pool, case.table_t, case.T, case.w_uk, case.w_uv, out, ws,
                      cache_scales=torch.ones(4, dtype=torch.float32, device="cuda"))
    f8 = PrefillCase(64, 8, seed=4, cache="fp8")
    with pytest.raises(RuntimeError, match="cache_scales"):
        M.mla_prefill(f8.dims, f8.q, f8.pool, f8.table_t, f8.T, f8.w_uk, f8.w_uv, out, ws)

"""Shared builders for GPU parity tests: seeded inputs on the device plus the
oracle's view of the same bytes.  Expected values come only from ``oracle/``."""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np
import torch

import mla_workloads as W
from oracle import mla_oracle as O

DT = {"fp32": 0, "bf16": 1, "fp8": 2, "fp8p2": 3}
FP8 = ("fp8", "fp8p2")  # the e4m3 cache formats (tile scales of any value / powers of two)
TORCH_ACT = {"fp32": torch.float32, "bf16": torch.bfloat16}


def dims_of(cfg: W.Config, flags: int = 0, act: Optional[str] = None):
    import mla_latent_kv_decode_amd as M
    d = cfg.dims
    return M.make_dims(d.num_heads, d.d_latent, d.d_rope, d.d_nope, d.d_v, d.block_size,
                       DT[cfg.cache_dtype], DT[act or cfg.act_dtype], flags=flags)


def append_workspace(dims, n_tokens: int, d_model: int, device="cuda"):
    """Device scratch for mla_cache_append (None when the path needs none)."""
    import mla_latent_kv_decode_amd as M
    n = M.mla_cache_append_workspace_size(dims, n_tokens, d_model)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def rel_l2(x, y) -> float:
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    return float(np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300))


def max_abs(x, y) -> float:
    return float(np.max(np.abs(np.asarray(x, np.float64) - np.asarray(y, np.float64))))


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 view of a device tensor (fp32 / bf16)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return O.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    return t.to(torch.float64).numpy()


class DecodeCase:
    """A paged-cache decode problem resident on the GPU.

    Tail slots past each sequence's length and the guard blocks (never
    referenced) hold NaN, so an out-of-range read shows up in the outputs.
    """

    def __init__(self, cfg: W.Config, device="cuda", guard: int = 2, nan_tail: bool = True,
                 act: Optional[str] = None, shuffle: bool = True, table=None, lens=None):
        self.cfg = cfg
        d = self.d = cfg.dims
        self.act = act or cfg.act_dtype
        self.lens = W.seq_lens(cfg) if lens is None else np.asarray(lens, np.int32)
        if table is None:
            self.table, self.nblk = W.page_table(self.lens, d.block_size, cfg.seed, shuffle, guard)
        else:
            self.table, self.nblk = table
        bs, D = d.block_size, d.row
        rows = W.cache_rows(self.nblk * bs, cfg, seed=cfg.seed + 10, device=device)
        self.scales = None
        if cfg.cache_dtype == "fp32":
            pool = rows.view(self.nblk, bs, D).clone()
        elif cfg.cache_dtype == "bf16":
            pool = rows.to(torch.bfloat16).view(self.nblk, bs, D)
        else:
            codes, scales = O.quantize_fp8_rows(rows.cpu().numpy(), pow2_scales=cfg.cache_dtype == "fp8p2")
            pool = torch.from_numpy(codes).to(device).view(self.nblk, bs, D)
            self.scales = torch.from_numpy(scales).to(device).view(self.nblk, bs, -1)
        del rows
        used = np.zeros((self.nblk, bs), bool)
        for b, L in enumerate(self.lens):
            nb = (int(L) + bs - 1) // bs
            blk = self.table[b, :nb]
            flat = np.zeros(nb * bs, bool)
            flat[:L] = True
            used[blk] = flat.reshape(nb, bs)
        if nan_tail:
            mask = torch.from_numpy(~used).to(device)
            if cfg.cache_dtype in FP8:
                pool[mask] = 0x7F
                self.scales[mask] = float("nan")
            else:
                pool[mask] = float("nan")
        self.pool = pool
        self.q = W.absorbed_queries(cfg, seed=cfg.seed + 20, device=device).to(TORCH_ACT[self.act])
        self.table_t = torch.from_numpy(self.table).to(device)
        self.lens_t = torch.from_numpy(self.lens).to(device)
        self.scale = O.softmax_scale(d.d_nope, d.d_rope)

    # -- oracle side -----------------------------------------------------
    def oracle_rows(self, b: int) -> np.ndarray:
        d = self.d
        L = int(self.lens[b])
        nb = (L + d.block_size - 1) // d.block_size
        idx = torch.from_numpy(self.table[b, :nb].astype(np.int64)).to(self.pool.device)
        blocks = self.pool.index_select(0, idx).cpu()
        if self.cfg.cache_dtype in FP8:
            sc = self.scales.index_select(0, idx).cpu().numpy()
            vals = O.dequantize_fp8_rows(blocks.numpy(), sc)
        else:
            vals = to_f64(blocks)
        return vals.reshape(nb * d.block_size, d.row)[:L]

    def oracle(self, b: int):
        qb = to_f64(self.q[b])
        return O.attend_absorbed(qb, self.oracle_rows(b), self.cfg.n_q, self.d.d_latent, self.scale)

    # -- GPU side ----------------------------------------------------------
    def run(self, flags: int = 0, G: int = 0):
        import mla_latent_kv_decode_amd as M
        dims = dims_of(self.cfg, flags, self.act)
        B, n_q = self.q.shape[0], self.q.shape[1]
        ws = torch.empty(M.mla_decode_workspace_size(dims, B, n_q, G), dtype=torch.uint8,
                         device=self.q.device)
        M.mla_decode(dims, self.q, self.pool, self.scales, self.table_t, self.lens_t, ws, G)
        u = torch.empty(B, n_q, self.d.num_heads, self.d.d_latent, dtype=TORCH_ACT[self.act],
                        device=self.q.device)
        lse = torch.empty(B, n_q, self.d.num_heads, dtype=torch.float32, device=self.q.device)
        M.mla_decode_combine(dims, ws, self.lens_t, u, lse, G)
        torch.cuda.synchronize()
        return u, lse


def fp8_score_bound(case: DecodeCase, b: int) -> np.ndarray:
    """Bound on |score error| per (query, head) of sequence b when the
    dequantised fp8 rows are rounded to bf16 before the dot products: each
    operand moves by at most 2^-8 of itself (bf16 round-to-nearest), so
    |ds_t| <= 2^-8 * scale * sum_i |q_i| |c_t,i|, and the log-sum-exp moves by
    at most max_t |ds_t|.  A 5% margin covers the fp32 product and sums."""
    rows = np.abs(case.oracle_rows(b))
    q = np.abs(to_f64(case.q[b]))                     # [n_q, H, D]
    dots = q.reshape(-1, q.shape[-1]) @ rows.T       # [n_q * H, L]
    return (1.05 * 2.0 ** -8 * case.scale * dots.max(axis=1)).reshape(q.shape[:2])


FP8_MFMA_ACC = 2.0 ** -10   # fp8 MFMA dot products: |error| <= this x the block's largest |product|


def fp8_mfma_accumulation_bound(q_abs, rows_abs, scale: float, block: int = 64,
                                exact: bool = True) -> np.ndarray:
    """Bound on the score error of fp8 matrix-core products beyond the exact
    products: the MFMA sums each 64-term block of products below fp32
    precision (measured on the device: at most 2^-11.5 of the block's largest
    |product|); with a 2^-10 allowance per block, |ds_t| <= scale * 2^-10 *
    sum_blocks max_k |q_k c_t,k|.  q_abs [..., D], rows_abs [L, D]; returns
    the max over t, shape q_abs.shape[:-1].  With ``exact=False`` each block's
    max |q_k c_t,k| is replaced by max |q_k| * max |c_t,k| (never smaller;
    one small matrix product instead of a pass over every product)."""
    q = np.asarray(q_abs, dtype=np.float32)
    r = np.asarray(rows_abs, dtype=np.float32)
    qf = q.reshape(-1, q.shape[-1])
    if not exact:
        edges = list(range(0, q.shape[-1], block))
        qm = np.stack([qf[:, lo:lo + block].max(axis=1) for lo in edges], 1).astype(np.float64)
        rm = np.stack([r[:, lo:lo + block].max(axis=1) for lo in edges], 1).astype(np.float64)
        return (1.01 * scale * FP8_MFMA_ACC * (qm @ rm.T).max(axis=1)).reshape(q.shape[:-1])
    best = np.zeros(qf.shape[0])
    for t0 in range(0, r.shape[0], 512):   # tokens in chunks: [rows, 512, 64] at a time
        rc = r[t0:t0 + 512]
        tot = np.zeros((qf.shape[0], rc.shape[0]))
        for lo in range(0, q.shape[-1], block):
            tot += (qf[:, None, lo:lo + block] * rc[None, :, lo:lo + block]).max(axis=-1)
        best = np.maximum(best, tot.max(axis=1))
    return (1.01 * scale * FP8_MFMA_ACC * best).reshape(q.shape[:-1])


def fp8_pow2_score_bound(case: DecodeCase, b: int) -> np.ndarray:
    """Bound on |score error| per (query, head) of sequence b for the
    power-of-two e4m3 cache on the matrix cores: the cached values enter the
    products exactly (code x power of two), and each head's query is rounded
    to e4m3 under one power-of-two scale 2^E (the smallest with max |q| <=
    448 * 2^E), which moves an element by at most max(2^-4 |q_i|, 2^-10 * 2^E)
    (half a unit in the last place of a normal, or of the subnormal grid).  So
    |ds_t| <= scale * sum_i dq_i |c_t,i| plus the matrix cores' accumulation
    term (``fp8_mfma_accumulation_bound``), and the log-sum-exp moves by at
    most max_t |ds_t|; a 5% margin covers the rest."""
    rows = np.abs(case.oracle_rows(b))
    q = np.abs(to_f64(case.q[b]))                                  # [n_q, H, D]
    amax = q.max(axis=-1, keepdims=True)
    ex = np.vectorize(lambda a: O.pow2_scale_exponent(a) if a > 0 else 0)(amax)
    dq = np.maximum(2.0 ** -4 * q, 2.0 ** -10 * np.exp2(ex))
    dots = dq.reshape(-1, q.shape[-1]) @ rows.T
    acc = fp8_mfma_accumulation_bound(q + dq, rows, case.scale, exact=False)
    return (1.05 * case.scale * dots.max(axis=1)).reshape(q.shape[:2]) + acc


def compare_sampled(case: DecodeCase, u, lse, batch_ids: List[int], rel_bar=1e-2, abs_bar=2e-2,
                    lse_tol=1e-3) -> Dict[str, float]:
    """Compare GPU outputs with the oracle on the listed sequences; returns metrics.

    For an fp8 cache the LSE tolerance is ``lse_tol`` plus the per-(query,
    head) bound of ``fp8_score_bound`` (the MFMA kernel feeds bf16-rounded
    dequantised rows to the matrix cores); for the power-of-two fp8 cache the
    larger of that and ``fp8_pow2_score_bound`` (its matrix-core path rounds
    the queries to e4m3 instead; the generic path stays within the former)."""
    got, want, gl, wl, tl = [], [], [], [], []
    for b in batch_ids:
        ou, ol = case.oracle(b)
        got.append(to_f64(u[b]))
        want.append(ou)
        gl.append(lse[b].cpu().numpy().astype(np.float64))
        wl.append(ol)
        if case.cfg.cache_dtype == "fp8":
            tl.append(lse_tol + fp8_score_bound(case, b))
        elif case.cfg.cache_dtype == "fp8p2":
            tl.append(lse_tol + np.maximum(fp8_score_bound(case, b), fp8_pow2_score_bound(case, b)))
        else:
            tl.append(lse_tol + np.zeros(ol.shape))
    got, want = np.stack(got), np.stack(want)
    lse_err = np.abs(np.stack(gl) - np.stack(wl))
    tol = np.stack(tl)
    m = {"rel_l2": rel_l2(got, want), "max_abs": max_abs(got, want),
         "lse_max_abs": float(lse_err.max()), "lse_worst_vs_tol": float((lse_err / tol).max()),
         "worst_seq_rel_l2": max(rel_l2(g, w) for g, w in zip(got, want))}
    assert np.all(np.isfinite(got)), "non-finite output (a masked or guard row leaked?)"
    assert m["rel_l2"] <= rel_bar, m
    if abs_bar is not None:
        assert m["max_abs"] <= abs_bar, m
    assert np.all(lse_err <= tol), m
    return m

"""Seeded synthetic inputs for the MLA latent-cache decode path.

This module only draws random numbers and lays them out (shapes, page tables,
length mixes).  It contains none of the attention arithmetic: no projection,
no RoPE, no softmax, no quantisation.  Both the CPU oracle (through the tests)
and the HIP path consume what it returns, so the two sides always see the same
bytes.

Workloads (sizes follow the decode shapes of the DeepSeek-V3 attention block
described on the pages; the recipe is restated in the design notes):

* ``tiny``      H=4, d_c=32, d_R=8, d_nope=d_v=16, d_model=64, fp32, one
                sequence whose 64 prior tokens (positions 0..63) are appended
                from hidden states, one query token at position 64.
* ``v3``        B=64, L=4096, n_q=1, bf16, H=128, d_c=512, d_R=64.
* ``long``      B=4, L=131072, n_q=1, bf16.
* ``ragged``    B=256, L_b log-uniform in [512, 32768], n_q=2 (causal), bf16.
* ``fp8``       B=128, L=16384, n_q=1, e4m3 cache with per-(token, 128-wide
                tile) fp32 scales; 1% of the 576 channels are scaled x20.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

BLOCK = 64


@dataclasses.dataclass(frozen=True)
class Dims:
    num_heads: int
    d_latent: int
    d_rope: int
    d_nope: int
    d_v: int
    d_model: int
    d_q: int = 0                # query compression width (W^DQ rows); 0: a single W^Q
    block_size: int = BLOCK
    rope_base: float = 10000.0

    @property
    def row(self) -> int:
        """Elements cached per token: latent plus shared RoPE key."""
        return self.d_latent + self.d_rope


TINY = Dims(num_heads=4, d_latent=32, d_rope=8, d_nope=16, d_v=16, d_model=64)
V3 = Dims(num_heads=128, d_latent=512, d_rope=64, d_nope=128, d_v=128, d_model=7168, d_q=1536)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    dims: Dims
    batch: int
    n_q: int
    seed: int
    cache_dtype: str          # "fp32" | "bf16" | "fp8" | "fp8p2" (e4m3, power-of-two tile scales)
    act_dtype: str            # "fp32" | "bf16"
    seq_len: Optional[int]    # uniform length, or None for the ragged mix
    len_lo: int = 0
    len_hi: int = 0
    outlier_frac: float = 0.0
    outlier_gain: float = 1.0


CONFIGS = {
    "tiny": Config("tiny", TINY, 1, 1, 0, "fp32", "fp32", 65),
    "v3": Config("v3", V3, 64, 1, 1, "bf16", "bf16", 4096),
    "long": Config("long", V3, 4, 1, 2, "bf16", "bf16", 131072),
    "ragged": Config("ragged", V3, 256, 2, 3, "bf16", "bf16", None, 512, 32768),
    "fp8": Config("fp8", V3, 128, 1, 4, "fp8", "bf16", 16384, outlier_frac=0.01,
                  outlier_gain=20.0),
    # the fp8 workload's rows (same seed) with power-of-two tile scales
    "fp8p2": Config("fp8p2", V3, 128, 1, 4, "fp8p2", "bf16", 16384, outlier_frac=0.01,
                    outlier_gain=20.0),
}


def scaled(cfg: Config, batch: Optional[int] = None, seq_len: Optional[int] = None,
           len_hi: Optional[int] = None, len_lo: Optional[int] = None) -> Config:
    """A smaller copy of a workload (same dims, dtypes and structure)."""
    return dataclasses.replace(
        cfg,
        batch=cfg.batch if batch is None else batch,
        seq_len=cfg.seq_len if seq_len is None or cfg.seq_len is None else seq_len,
        len_hi=cfg.len_hi if len_hi is None else len_hi,
        len_lo=cfg.len_lo if len_lo is None else len_lo,
    )


# --------------------------------------------------------------------------
# lengths and page tables
# --------------------------------------------------------------------------
def seq_lens(cfg: Config) -> np.ndarray:
    """Cached tokens per sequence, counting the n_q new tokens."""
    if cfg.seq_len is not None:
        return np.full(cfg.batch, cfg.seq_len, dtype=np.int32)
    rng = np.random.default_rng(cfg.seed)
    lo, hi = math.log(cfg.len_lo), math.log(cfg.len_hi)
    lens = np.floor(np.exp(rng.uniform(lo, hi, size=cfg.batch))).astype(np.int64)
    return np.clip(lens, max(cfg.len_lo, cfg.n_q), cfg.len_hi).astype(np.int32)


def page_table(lens: np.ndarray, block_size: int, seed: int, shuffle: bool = True,
               guard_blocks: int = 0):
    """Random paged layout.

    Returns (table int32 [B, max_blocks], num_blocks).  Physical block ids are
    a seeded permutation of range(guard_blocks, guard_blocks + needed); the
    first ``guard_blocks`` ids are never referenced (they stay as sentinels).
    Unused table entries are -1.
    """
    nblk = (lens.astype(np.int64) + block_size - 1) // block_size
    need = int(nblk.sum())
    maxb = int(nblk.max()) if len(nblk) else 0
    ids = np.arange(guard_blocks, guard_blocks + need, dtype=np.int64)
    if shuffle:
        np.random.default_rng(seed + 1000).shuffle(ids)
    table = np.full((len(lens), max(maxb, 1)), -1, dtype=np.int32)
    k = 0
    for b, n in enumerate(nblk):
        table[b, :n] = ids[k:k + n]
        k += n
    return table, need + 2 * guard_blocks


def identity_table(lens: np.ndarray, block_size: int):
    """Contiguous layout: sequence b owns blocks [b*maxb, (b+1)*maxb)."""
    nblk = (lens.astype(np.int64) + block_size - 1) // block_size
    maxb = int(nblk.max())
    table = np.full((len(lens), maxb), -1, dtype=np.int32)
    for b, n in enumerate(nblk):
        table[b, :n] = b * maxb + np.arange(n)
    return table, len(lens) * maxb


# --------------------------------------------------------------------------
# random values
# --------------------------------------------------------------------------
def _gen(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(shape, seed: int, std: float = 1.0, device="cpu", dtype=torch.float32):
    """N(0, std^2) draws from a seeded torch generator, cast to ``dtype``."""
    g = _gen(seed, device)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def weight(rows: int, cols: int, seed: int, dtype=torch.float32, device="cpu"):
    """Weight matrix [rows, cols] ~ N(0, 1/cols): fan-in is the input width."""
    return normal((rows, cols), seed, std=1.0 / math.sqrt(cols), device=device, dtype=dtype)


def outlier_channels(cfg: Config) -> np.ndarray:
    """Channel indices that are scaled by ``outlier_gain`` (fp8 workload)."""
    n = int(round(cfg.outlier_frac * cfg.dims.row))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.default_rng(cfg.seed + 2000)
    return np.sort(rng.choice(cfg.dims.row, size=n, replace=False))


def cache_rows(n_rows: int, cfg: Config, seed: int, device="cpu"):
    """Synthetic cached rows [n_rows, d_c + d_R] in fp32.

    Latent and RoPE-key channels are both N(0, 1) (a rotation of an isotropic
    Gaussian is isotropic, so these stand in for already-rotated keys).  For the
    fp8 workload the outlier channels are multiplied by the gain.
    """
    x = normal((n_rows, cfg.dims.row), seed, device=device)
    ch = outlier_channels(cfg)
    if len(ch):
        x[:, torch.as_tensor(ch, device=device)] *= cfg.outlier_gain
    return x


def absorbed_queries(cfg: Config, seed: int, device="cpu"):
    """Packed absorbed queries [B, n_q, H, d_c + d_R] in fp32.

    The latent part is drawn N(0, d_nope / d_c): the variance a content query
    q^C ~ N(0, 1) has after multiplication by W^UK_i^T with W^UK ~ N(0, 1/d_c).
    The RoPE part is N(0, 1).  With scale 1/sqrt(d_nope + d_R) the logits then
    have unit variance.
    """
    d = cfg.dims
    q = normal((cfg.batch, cfg.n_q, d.num_heads, d.row), seed, device=device)
    q[..., :d.d_latent] *= math.sqrt(d.d_nope / d.d_latent)
    return q

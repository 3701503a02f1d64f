"""GPU parity of the e4m3 cache with power-of-two tile scales (MLA_FP8_E4M3_PO2).

The matrix-core decode of this format runs its scores on fp8 MFMAs: the
cached codes and their power-of-two tile scales enter exactly, and each head's
query is rounded to e4m3 under one power-of-two scale.  Two bars apply:

* against the oracle on the stored cache and the bf16 queries: the fp8
  tolerance (relative L2 <= 5e-2) and, for the log-sum-exp, 1e-3 plus the
  derived bound of the queries' e4m3 rounding (``fp8_pow2_score_bound``);
* against the oracle whose queries are rounded the same way
  (``quantize_rows_e4m3_pow2``): then both sides compute the same scores, and
  the bf16 bars hold: relative L2 <= 1e-2, LSE <= 1e-3, and elementwise the
  derived bound of what is still rounded -- the probabilities to bf16 before
  the output product (each by at most 2^-8 of itself, bf16's unit roundoff,
  so u moves by at most 2^-8 sum_t p_t |c_t| / sum_t p_t) and u itself to
  bf16 (2^-8 |u|) -- with a 10% margin and 1e-4 for the fp32 sums.  The fp8
  matrix cores sum each 64-term block of exact products below fp32 precision
  (``fp8_mfma_accumulation_bound``): that moves a score by at most ds, the
  log-sum-exp by ds and u by about ds * sum_t p_t |c_t - u|, which both bars
  add.  (The workload's x20 outlier
  channels make sum_t p_t |c_t| far larger than |u| where they cancel.)
"""
import dataclasses

import numpy as np
import pytest
import torch

import mla_workloads as W
from oracle import mla_oracle as O
from tests.cases import (DecodeCase, compare_sampled, fp8_mfma_accumulation_bound, fp8_pow2_score_bound,
                         max_abs, rel_l2, to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_decode_amd as M
    M.lib()  # raises if the HIP library is missing: no fallback exists
    return M


P2 = W.CONFIGS["fp8p2"]
RAGGED_P2 = dataclasses.replace(W.CONFIGS["ragged"], cache_dtype="fp8p2")

SMALL = [
    W.scaled(P2, batch=3, seq_len=333),                       # ragged last step
    W.scaled(P2, batch=2, seq_len=64),                        # exactly one block
    W.scaled(P2, batch=4, seq_len=1),                         # one token
    W.scaled(P2, batch=3, seq_len=97),
    W.scaled(RAGGED_P2, batch=6, len_lo=2, len_hi=700),       # n_q = 2, causal pair
]


def _oracle_e4m3_queries(case, b):
    """The oracle with the queries rounded to e4m3 per head (one power-of-two
    scale over the head's d_c + d_R channels), and the elementwise bound of
    the remaining bf16 roundings (see the module docstring)."""
    q8 = O.quantize_rows_e4m3_pow2(to_f64(case.q[b]))
    rows = case.oracle_rows(b)
    u, lse = O.attend_absorbed(q8, rows, case.cfg.n_q, case.d.d_latent, case.scale)
    L, n_q, d_c = rows.shape[0], case.cfg.n_q, case.d.d_latent
    absw = np.zeros_like(u)
    ds = np.zeros(lse.shape)
    for j in range(n_q):
        n = O.visible(L, n_q, j)
        s = case.scale * (q8[j] @ rows[:n].T)                   # [H, n]
        p = np.exp(s - lse[j][:, None])                         # softmax weights (sum 1)
        absw[j] = p @ np.abs(rows[:n, :d_c])
        ds[j] = fp8_mfma_accumulation_bound(np.abs(q8[j]), np.abs(rows[:n]), case.scale)
    bound = 1.1 * (2.0 ** -8 + 2 * ds[..., None]) * (absw + np.abs(u)) + 1e-4
    return u, lse, bound, ds


@pytest.mark.parametrize("G", [1, 3, 64])
@pytest.mark.parametrize("idx", range(len(SMALL)))
def test_decode_fp8_pow2_small(idx, G):
    cfg = SMALL[idx]
    case = DecodeCase(cfg)
    u, lse = case.run(G=G)
    compare_sampled(case, u, lse, list(range(cfg.batch)), rel_bar=5e-2, abs_bar=None)
    assert torch.isfinite(u.float()).all()


@pytest.mark.parametrize("idx", [0, 3, 4])
def test_decode_fp8_pow2_matches_oracle_on_e4m3_queries(idx):
    cfg = SMALL[idx]
    case = DecodeCase(cfg)
    u, lse = case.run(G=5)
    got, want, gl, wl, bd, lt = [], [], [], [], [], []
    for b in range(cfg.batch):
        ou, ol, ob, ods = _oracle_e4m3_queries(case, b)
        got.append(to_f64(u[b]))
        want.append(ou)
        bd.append(ob)
        lt.append(1e-3 + ods)
        gl.append(lse[b].cpu().numpy().astype(np.float64))
        wl.append(ol)
    got, want, bd = np.stack(got), np.stack(want), np.stack(bd)
    gl, wl = np.stack(gl), np.stack(wl)
    err = np.abs(got - want)
    w = np.unravel_index(np.argmax(err / bd), err.shape)
    head = w[:3]
    info = {"worst": tuple(int(i) for i in w), "got": float(got[w]), "want": float(want[w]), "bound": float(bd[w]),
            "head_rel_l2": rel_l2(got[head], want[head]), "head_lse_diff": float(gl[head] - wl[head]),
            "heads_over_1e-2": int(sum(rel_l2(got[i], want[i]) > 1e-2 for i in np.ndindex(got.shape[:3])))}
    assert rel_l2(got, want) <= 1e-2, info
    assert np.all(err <= bd), info
    assert np.all(np.abs(gl - wl) <= np.stack(lt)), info


def test_decode_fp8_pow2_agrees_with_generic():
    """The generic kernel decodes the same codes and scales with the bf16
    queries: the two differ by the queries' e4m3 rounding only."""
    import mla_latent_kv_decode_amd as M
    cfg = W.scaled(P2, batch=5, seq_len=900)
    case = DecodeCase(cfg)
    u1, l1 = case.run(G=16)
    u2, l2 = case.run(flags=M.FLAG_GENERIC_DECODE, G=16)
    assert rel_l2(to_f64(u1), to_f64(u2)) <= 5e-2
    tol = np.stack([2e-3 + fp8_pow2_score_bound(case, b) for b in range(cfg.batch)])
    assert np.all(np.abs(l1.cpu().numpy() - l2.cpu().numpy()) <= tol)


def test_decode_fp8_pow2_deterministic():
    case = DecodeCase(W.scaled(RAGGED_P2, batch=5, len_lo=100, len_hi=2000))
    u1, l1 = case.run(G=11)
    u2, l2 = case.run(G=11)
    assert torch.equal(u1.view(torch.int16), u2.view(torch.int16)) and torch.equal(l1, l2)


def test_decode_fp8_pow2_score_spike_in_late_tile():
    """A token far above the first step's maximum forces the exact softmax
    path (reference raised, output rescaled) with the query's power-of-two
    scale folded into the log2 factor."""
    cfg = W.scaled(P2, batch=2, seq_len=700)
    case = DecodeCase(cfg)
    d = cfg.dims
    for b, t in [(0, 650), (1, 200)]:
        blk, off = O.slot_of(case.table, b, t, d.block_size)
        row = (3.0 * case.q[b, 0, 0].float()).cpu().numpy()[None]
        codes, sc = O.quantize_fp8_rows(row, pow2_scales=True)
        case.pool[blk, off] = torch.from_numpy(codes[0]).cuda()
        case.scales[blk, off] = torch.from_numpy(sc[0]).cuda()
    u, lse = case.run(G=1)
    compare_sampled(case, u, lse, [0, 1], rel_bar=5e-2, abs_bar=None)
    assert float(lse[0, 0, 0]) > 30.0


def test_decode_fp8_pow2_page_table_permutation_is_bitwise_invariant():
    cfg = W.scaled(P2, batch=2, seq_len=500)
    a = DecodeCase(cfg, shuffle=False, guard=0)
    # same logical rows (codes and scales), physical blocks permuted
    perm = np.random.default_rng(3).permutation(a.nblk)
    b = DecodeCase(cfg, table=(perm[a.table].astype(np.int32), a.nblk), guard=0)
    pt = torch.from_numpy(perm).cuda()
    b.pool = a.pool.clone()
    b.pool[pt] = a.pool
    b.scales = a.scales.clone()
    b.scales[pt] = a.scales
    ua, la = a.run(G=7)
    ub, lb = b.run(G=7)
    assert torch.isfinite(ua.float()).all() and torch.isfinite(la).all()
    assert torch.equal(ua.view(torch.int16), ub.view(torch.int16)) and torch.equal(la, lb)

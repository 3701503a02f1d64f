"""mla_decode_noalloc: the decode + combine with the library's static scratch
as the workspace, against mla_decode + mla_decode_combine with a caller
workspace on the same inputs.  Two calls in a row, the second on a smaller
batch, so the scratch holds the first call's contents when the second runs."""
import numpy as np
import pytest
import torch

import mla_workloads as W
from tests.cases import DecodeCase, compare_sampled, dims_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_decode_amd as M
    M.lib()
    return M


def _noalloc(case, G):
    import mla_latent_kv_decode_amd as M
    dims = dims_of(case.cfg)
    B, n_q, H = case.q.shape[0], case.q.shape[1], case.d.num_heads
    u = torch.full((B, n_q, H, case.d.d_latent), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, n_q, H), float("nan"), dtype=torch.float32, device="cuda")
    M.mla_decode_noalloc(dims, case.q, case.pool, case.scales, case.table_t, case.lens_t, u, lse, G)
    torch.cuda.synchronize()
    return u, lse


@pytest.mark.parametrize("G", [0, 37])
def test_noalloc_matches_workspace_decode_two_calls(G):
    big = DecodeCase(W.scaled(W.CONFIGS["ragged"], batch=40, len_lo=2, len_hi=3000))
    small = DecodeCase(W.scaled(W.CONFIGS["v3"], batch=5, seq_len=700))
    for case in (big, small):
        u, lse = _noalloc(case, G)
        ur, lr = case.run(G=G)
        assert torch.equal(u.view(torch.int16), ur.view(torch.int16)) and torch.equal(lse, lr)
        compare_sampled(case, u, lse, list(range(case.cfg.batch)))


@pytest.mark.parametrize("name", ["fp8", "fp8p2"])
def test_noalloc_fp8_cache(name):
    case = DecodeCase(W.scaled(W.CONFIGS[name], batch=6, seq_len=900))
    u, lse = _noalloc(case, 16)
    ur, lr = case.run(G=16)
    assert torch.equal(u.view(torch.int16), ur.view(torch.int16)) and torch.equal(lse, lr)


def test_noalloc_rejects_calls_beyond_the_scratch():
    import mla_latent_kv_decode_amd as M
    from mla_latent_kv_decode_amd import _lib as L
    case = DecodeCase(W.scaled(W.CONFIGS["v3"], batch=2, seq_len=100))
    dims = dims_of(case.cfg)
    G = 4000  # (2 + 4000) slots x 128 heads x ~1 KB > 64 MiB
    assert M.mla_decode_workspace_size(dims, 2, 1, G) > M.NOALLOC_SCRATCH_BYTES
    u = torch.zeros(2, 1, 128, 512, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MlaError) as ei:
        M.mla_decode_noalloc(dims, case.q, case.pool, None, case.table_t, case.lens_t, u, None, G)
    assert ei.value.code == L.ERR_WORKSPACE_TOO_SMALL and "static scratch" in str(ei.value)
    assert torch.count_nonzero(u) == 0
    # the scratch still serves a call that fits
    u2, l2 = _noalloc(case, 4)
    ur, lr = case.run(G=4)
    assert torch.equal(u2.view(torch.int16), ur.view(torch.int16)) and torch.equal(l2, lr)

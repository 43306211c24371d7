"""HIP LSE merge against the oracle's fp64 merge, plus its exact special cases."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import context_causal_attention_amd as cp
import oracle
from helpers import max_abs

pytestmark = pytest.mark.gpu
DEV = "cuda"


EPS32 = 2.0 ** -23


def _fp32_bound(o1, l1, o2, l2):
    """Error bound of the fp32 merge against exact arithmetic.  The weights are
    exp(lse - merged): rounding of merged (absolute <= |merged| * 2^-23 after log1p/exp)
    and of the exponential (a few ulp) give each weight a relative error of about
    (|merged| + 4) * 2^-23; the two products and the sum add three roundings of |out|."""
    fin = lambda x: np.where(np.isfinite(x), np.abs(x), 0.0)
    m = np.maximum(fin(l1.numpy()), fin(l2.numpy())).max() + 1.0
    omax = max(np.abs(o1.numpy()).max(), np.abs(o2.numpy()).max())
    return (2.0 * (m + 4.0) + 3.0) * EPS32 * omax, 4.0 * m * EPS32


def _partial(g, B, S, H, D, empty_frac=0.0):
    o = torch.randn((B, S, H, D), generator=g)
    lse = torch.randn((B, H, S), generator=g) * 4.0 + 6.0
    if empty_frac:
        empty = torch.rand((B, H, S), generator=g) < empty_frac
        lse[empty] = -float("inf")
        o.permute(0, 2, 1, 3)[empty] = 0.0
    return o, lse


@pytest.mark.parametrize("B,S,H,D", [(1, 300, 3, 128), (2, 65, 4, 64), (1, 1, 1, 4), (2, 129, 16, 128)])
def test_merge_matches_oracle(B, S, H, D):
    g = torch.Generator().manual_seed(B * 1000 + S)
    o1, l1 = _partial(g, B, S, H, D, 0.2)
    o2, l2 = _partial(g, B, S, H, D, 0.2)
    ref_o, ref_l = oracle.merge(o1.numpy(), l1.numpy(), o2.numpy(), l2.numpy())
    do, dl = o1.to(DEV), l1.to(DEV)
    cp.lse_merge(do, dl, o2.to(DEV), l2.to(DEV))
    tol_o, tol_l = _fp32_bound(o1, l1, o2, l2)
    assert max_abs(do.cpu().numpy(), ref_o) <= tol_o
    assert max_abs(dl.cpu().numpy(), ref_l) <= tol_l
    assert not torch.isnan(do).any() and not torch.isnan(dl).any()


def test_merge_special_cases_exact():
    g = torch.Generator().manual_seed(7)
    B, S, H, D = 1, 130, 2, 128
    o1, l1 = _partial(g, B, S, H, D)
    o2, l2 = _partial(g, B, S, H, D)
    empty_o, empty_l = torch.zeros_like(o1), torch.full_like(l1, -float("inf"))
    # empty tile: identity, bit for bit
    do, dl = o1.to(DEV), l1.to(DEV)
    cp.lse_merge(do, dl, empty_o.to(DEV), empty_l.to(DEV))
    assert torch.equal(do.cpu(), o1) and torch.equal(dl.cpu(), l1)
    # empty accumulator: takes the tile, bit for bit
    do, dl = empty_o.to(DEV), empty_l.to(DEV)
    cp.lse_merge(do, dl, o1.to(DEV), l1.to(DEV))
    assert torch.equal(do.cpu(), o1) and torch.equal(dl.cpu(), l1)
    # both empty: stays (0, -inf), no NaN
    do, dl = empty_o.to(DEV), empty_l.to(DEV)
    cp.lse_merge(do, dl, empty_o.to(DEV), empty_l.to(DEV))
    assert torch.equal(do.cpu(), empty_o) and torch.equal(dl.cpu(), empty_l)
    # commutative, bit for bit
    a_o, a_l = o1.to(DEV), l1.to(DEV)
    cp.lse_merge(a_o, a_l, o2.to(DEV), l2.to(DEV))
    b_o, b_l = o2.to(DEV), l2.to(DEV)
    cp.lse_merge(b_o, b_l, o1.to(DEV), l1.to(DEV))
    assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l)
    # identical tiles: same output, lse + ln 2
    do, dl = o1.to(DEV), l1.to(DEV)
    cp.lse_merge(do, dl, o1.to(DEV), l1.to(DEV))
    tol_o, tol_l = _fp32_bound(o1, l1, o1, l1)
    assert max_abs(do.cpu().numpy(), o1.numpy()) <= tol_o
    assert max_abs(dl.cpu().numpy(), l1.numpy().astype(np.float64) + np.log(2.0)) <= tol_l


def test_merge_long_context_tile_sampled():
    """The merge at the long-context share's tile size (32768 rows x 32 heads x 128, 512 MiB
    per operand, as each ring step of the per-step form merges), sampled rows against the
    oracle's fp64 merge: every (row, head) of 512 seeded rows, a fifth of them empty on one
    side."""
    B, S, H, D = 1, 32768, 32, 128
    g = torch.Generator().manual_seed(32768)
    o1, l1 = _partial(g, B, S, H, D, 0.2)
    o2, l2 = _partial(g, B, S, H, D, 0.2)
    rows = np.sort(np.random.default_rng(5).choice(S, 512, replace=False)).astype(np.int64)
    rows = np.unique(np.concatenate([rows, [0, 1, S - 2, S - 1]]))
    ref_o, ref_l = oracle.merge(o1[:, rows].numpy(), l1[:, :, rows].numpy(), o2[:, rows].numpy(),
                                l2[:, :, rows].numpy())
    do, dl = o1.to(DEV), l1.to(DEV)
    cp.lse_merge(do, dl, o2.to(DEV), l2.to(DEV))
    torch.cuda.synchronize()
    tol_o, tol_l = _fp32_bound(o1[:, rows], l1[:, :, rows], o2[:, rows], l2[:, :, rows])
    ridx = torch.from_numpy(rows).to(DEV)
    assert max_abs(do[:, ridx].cpu().numpy(), ref_o) <= tol_o
    assert max_abs(dl[:, :, ridx].cpu().numpy(), ref_l) <= tol_l
    assert not torch.isnan(do).any() and not torch.isnan(dl).any()

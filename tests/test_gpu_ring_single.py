"""The one-launch ring share (cpattn_ring_share_fwd) against the oracle: every rank and row at
small sizes for both dtypes and GQA ratios, bit-identity with cpattn_block_fwd for a single
block, skipped empty blocks, fully hidden blocks and the all-empty case."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import context_causal_attention_amd as cp
import oracle
from helpers import TOL, max_abs

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _rand(seed, shape, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(TDT[dtype])


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("C,t,Hq,Hkv", [(4, 96, 4, 2), (3, 70, 6, 3), (8, 32, 8, 1)])
def test_single_launch_share_every_rank(dtype, C, t, Hq, Hkv):
    B, D = 1, 128
    S = 2 * C * t
    scale = 1 / math.sqrt(D)
    q_full = _rand(1, (B, S, Hq, D), dtype)
    k_full = _rand(2, (B, S, Hkv, D), dtype)
    v_full = _rand(3, (B, S, Hkv, D), dtype)
    pos = [oracle.zigzag_positions(S, C, o) for o in range(C)]
    ks = [k_full[:, p].contiguous().to(DEV) for p in pos]
    vs = [v_full[:, p].contiguous().to(DEV) for p in pos]
    tpos = [torch.from_numpy(p).to(DEV) for p in pos]
    gpos = np.arange(S, dtype=np.int64)
    ref_o, ref_l = oracle.attention_rows(q_full.float().numpy(), k_full.float().numpy(), v_full.float().numpy(),
                                         gpos, gpos, scale)
    tol_o, tol_l = TOL[dtype]
    for r in range(C):
        q = q_full[:, pos[r]].contiguous().to(DEV)
        out, lse = cp.ring_share_fwd(q, ks, vs, tpos, r, scale)
        torch.cuda.synchronize()
        eo = max_abs(out.cpu().numpy(), ref_o[:, pos[r]])
        el = max_abs(lse.cpu().numpy(), ref_l[:, :, pos[r]])
        assert eo <= tol_o and el <= tol_l, f"rank {r}: O {eo:.3g} lse {el:.3g}"
        # the step-by-step share is the same attention rounded differently: both are within
        # the tolerance of the oracle (checked above and in the fused-merge tests)
        fo, fl = cp.ring_share_fwd(q, ks, vs, tpos, r, scale, mode="fused")
        torch.cuda.synchronize()
        assert max_abs(out.cpu().numpy(), fo.cpu().numpy()) <= 2 * tol_o


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_one_block_is_block_fwd(dtype):
    q = _rand(4, (2, 150, 4, 128), dtype).to(DEV)
    k = _rand(5, (2, 230, 2, 128), dtype).to(DEV)
    v = _rand(6, (2, 230, 2, 128), dtype).to(DEV)
    qpos = torch.arange(80, 230, device=DEV)
    kpos = torch.arange(230, device=DEV)
    a_o, a_l = cp.ring_blocks_fwd(q, [k], [v], [kpos], qpos, 0.09)
    b_o, b_l = cp.block_fwd(q, k, v, qpos, kpos, 0.09)
    torch.cuda.synchronize()
    assert torch.equal(a_o, b_o) and torch.equal(a_l, b_l)


def test_empty_and_hidden_blocks():
    # blocks: a visible one, an empty one (skipped), one entirely after every query (hidden)
    q = _rand(7, (1, 64, 2, 128), "bf16").to(DEV)
    k = _rand(8, (1, 100, 2, 128), "bf16")
    v = _rand(9, (1, 100, 2, 128), "bf16")
    qpos = torch.arange(100, 164, device=DEV)
    blocks_k = [k[:, :60].contiguous().to(DEV), k[:, :0].contiguous().to(DEV), k[:, 60:].contiguous().to(DEV)]
    blocks_v = [v[:, :60].contiguous().to(DEV), v[:, :0].contiguous().to(DEV), v[:, 60:].contiguous().to(DEV)]
    blocks_p = [torch.arange(0, 60, device=DEV), torch.arange(0, device=DEV), torch.arange(1000, 1040, device=DEV)]
    out, lse = cp.ring_blocks_fwd(q, blocks_k, blocks_v, blocks_p, qpos, 0.1)
    ref_o, ref_l = cp.block_fwd(q, blocks_k[0], blocks_v[0], qpos, blocks_p[0], 0.1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    # nothing visible at all: zeros and -inf
    out2, lse2 = cp.ring_blocks_fwd(q, blocks_k[1:], blocks_v[1:], blocks_p[1:], qpos, 0.1)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out2) == 0 and bool(torch.isneginf(lse2).all())

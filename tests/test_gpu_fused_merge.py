"""block_fwd_merge (attention with the lse merge in its epilogue) on the HIP path.

Bit for bit against block_fwd into a tile followed by lse_merge, since both use the same
merge arithmetic and rounding; against the oracle for the merged result of two key halves;
and the special cases: an empty accumulator (-inf) takes the block's result unchanged, an
empty key set leaves finite rows untouched."""
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


def _same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("C,t,Hq,Hkv,B", [(4, 96, 4, 2, 1), (2, 150, 8, 2, 2), (3, 64, 6, 3, 1)])
def test_fused_ring_share_equals_tile_then_merge(dtype, C, t, Hq, Hkv, B):
    S, D = 2 * C * t, 128
    pos = [cp.zigzag_index(S, C, o, device=DEV) for o in range(C)]
    ks = [_rand(100 + o, (B, 2 * t, Hkv, D), dtype).to(DEV) for o in range(C)]
    vs = [_rand(200 + o, (B, 2 * t, Hkv, D), dtype).to(DEV) for o in range(C)]
    for r in range(C):
        q = _rand(300 + r, (B, 2 * t, Hq, D), dtype).to(DEV)
        fo, fl = cp.ring_share_fwd(q, ks, vs, pos, r, 1 / math.sqrt(D), mode="fused")
        uo, ul = cp.ring_share_fwd(q, ks, vs, pos, r, 1 / math.sqrt(D), mode="unfused")
        torch.cuda.synchronize()
        assert _same_bits(fo, uo) and _same_bits(fl, ul), f"rank {r}"


def test_fused_ring_share_equals_tile_then_merge_at_launch_size():
    """The same at launch sizes (6000 local rows, 32/8 heads): the diagonal step shares the
    query positions tensor (12-wave kernel), the other steps do not (8-wave kernel)."""
    C, t, Hq, Hkv, B, D = 4, 3000, 32, 8, 1, 128
    S = 2 * C * t
    pos = [cp.zigzag_index(S, C, o, device=DEV) for o in range(C)]
    ks = [_rand(400 + o, (B, 2 * t, Hkv, D), "bf16").to(DEV) for o in range(C)]
    vs = [_rand(500 + o, (B, 2 * t, Hkv, D), "bf16").to(DEV) for o in range(C)]
    for r in (0, 2):
        q = _rand(600 + r, (B, 2 * t, Hq, D), "bf16").to(DEV)
        fo, fl = cp.ring_share_fwd(q, ks, vs, pos, r, 1 / math.sqrt(D), mode="fused")
        uo, ul = cp.ring_share_fwd(q, ks, vs, pos, r, 1 / math.sqrt(D), mode="unfused")
        torch.cuda.synchronize()
        assert _same_bits(fo, uo) and _same_bits(fl, ul), f"rank {r}"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_two_key_halves_merge_to_full_attention(dtype):
    """Keys split at an arbitrary point: block_fwd over the first part, block_fwd_merge over
    the second, against the oracle's attention over all keys (and its merge of the halves)."""
    B, Sq, Skv, Hq, Hkv, D = 2, 190, 301, 4, 2, 128
    q, k, v = (_rand(s, shp, dtype) for s, shp in ((1, (B, Sq, Hq, D)), (2, (B, Skv, Hkv, D)),
                                                    (3, (B, Skv, Hkv, D))))
    qpos = np.arange(Skv - Sq, Skv, dtype=np.int64)
    kvpos = np.arange(Skv, dtype=np.int64)
    cut = 117
    scale = 1 / math.sqrt(D)
    d = lambda x: x.to(DEV)  # noqa: E731
    tq = torch.from_numpy(qpos).to(DEV)
    out, lse = cp.block_fwd(d(q), d(k[:, :cut].contiguous()), d(v[:, :cut].contiguous()), tq,
                            torch.from_numpy(kvpos[:cut]).to(DEV), scale)
    cp.block_fwd_merge(d(q), d(k[:, cut:].contiguous()), d(v[:, cut:].contiguous()), tq,
                       torch.from_numpy(kvpos[cut:]).to(DEV), scale, out, lse)
    qf, kf, vf = q.float().numpy(), k.float().numpy(), v.float().numpy()
    ref_o, ref_l = oracle.attention_rows(qf, kf, vf, qpos, kvpos, scale)
    tol_o, tol_l = TOL[dtype]
    assert max_abs(out.cpu().numpy(), ref_o) <= tol_o
    assert max_abs(lse.cpu().numpy(), ref_l) <= tol_l
    o1, l1 = oracle.attention_rows(qf, kf[:, :cut], vf[:, :cut], qpos, kvpos[:cut], scale)
    o2, l2 = oracle.attention_rows(qf, kf[:, cut:], vf[:, cut:], qpos, kvpos[cut:], scale)
    mo, ml = oracle.merge(o1, l1, o2, l2)
    assert max_abs(out.cpu().numpy(), mo) <= tol_o
    assert max_abs(lse.cpu().numpy(), ml) <= tol_l


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_empty_accumulator_takes_block_result(dtype):
    B, Sq, Skv, Hq, Hkv, D = 1, 130, 200, 4, 1, 128
    q, k, v = (_rand(s, shp, dtype).to(DEV) for s, shp in ((4, (B, Sq, Hq, D)), (5, (B, Skv, Hkv, D)),
                                                           (6, (B, Skv, Hkv, D))))
    qpos = torch.arange(50, 50 + Sq, device=DEV)  # the first rows see only part of the keys
    kvpos = torch.arange(Skv, device=DEV)
    ref_o, ref_l = cp.block_fwd(q, k, v, qpos, kvpos, 0.09)
    out = torch.zeros_like(ref_o)
    lse = torch.full_like(ref_l, -math.inf)
    cp.block_fwd_merge(q, k, v, qpos, kvpos, 0.09, out, lse)
    torch.cuda.synchronize()
    assert _same_bits(out, ref_o) and _same_bits(lse, ref_l)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_no_keys_and_hidden_keys_leave_accumulator(dtype):
    """A block with no keys, or with every key later than every query, contributes nothing:
    finite rows keep their bits and rows at -inf become (0, -inf)."""
    B, Sq, Hq, Hkv, D = 2, 77, 4, 2, 128
    q = _rand(7, (B, Sq, Hq, D), dtype).to(DEV)
    qpos = torch.arange(Sq, device=DEV)
    g = torch.Generator().manual_seed(8)
    out0 = torch.randn((B, Sq, Hq, D), generator=g)
    lse0 = torch.randn((B, Hq, Sq), generator=g) * 3
    lse0[0, 1, 5:9] = -math.inf
    expect_o = out0.clone()
    expect_o.permute(0, 2, 1, 3)[torch.isneginf(lse0)] = 0.0
    kv = _rand(9, (B, 40, Hkv, D), dtype).to(DEV)
    for seq_kv in (0, 40):
        out, lse = out0.clone().to(DEV), lse0.clone().to(DEV)
        k = kv[:, :seq_kv].contiguous()
        kvpos = torch.arange(1000, 1000 + seq_kv, device=DEV)
        cp.block_fwd_merge(q, k, k, qpos, kvpos, 0.1, out, lse)
        torch.cuda.synchronize()
        assert _same_bits(lse.cpu(), lse0), f"seq_kv={seq_kv}"
        assert _same_bits(out.cpu(), expect_o), f"seq_kv={seq_kv}"

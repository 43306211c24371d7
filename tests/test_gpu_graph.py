"""A rank share captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library's calls only enqueue kernels on the caller's stream (no allocation, no memset, no
synchronisation), so a whole step can be captured once and replayed.  Every replay must give
the eager result bit for bit, with eager work on the same buffers between the replays."""
from __future__ import annotations

import math

import pytest
import torch

import context_causal_attention_amd as cp

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rand(seed, shape, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype).to(DEV)


def _same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.contiguous().view(torch.int32), b.contiguous().view(torch.int32))


def _capture(step):
    """Warm up on a side stream, then capture one call of ``step``."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_forward_share_replays_match_eager(dtype):
    S, C, r, B, Hq, Hkv, D = 2048, 4, 1, 1, 8, 2, 128
    t = S // (2 * C)
    scale = 1 / math.sqrt(D)
    q = _rand(1, (B, 2 * t, Hq, D), dtype)
    ks = [_rand(10 + o, (B, 2 * t, Hkv, D), dtype) for o in range(C)]
    vs = [_rand(20 + o, (B, 2 * t, Hkv, D), dtype) for o in range(C)]
    pos = [torch.empty(2 * t, dtype=torch.int64, device=DEV) for _ in range(C)]
    out = torch.empty((B, 2 * t, Hq, D), dtype=torch.float32, device=DEV)
    lse = torch.empty((B, Hq, 2 * t), dtype=torch.float32, device=DEV)
    order = [(r - s) % C for s in range(C)]

    def step():
        for o in range(C):
            cp.zigzag_index(S, C, o, out=pos[o])
        cp.ring_blocks_fwd(q, [ks[o] for o in order], [vs[o] for o in order], [pos[o] for o in order], pos[r],
                           scale, out, lse)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    g = _capture(step)
    for i in range(4):
        out.fill_(float(i))  # eager work on the graph's buffers between the replays
        lse.fill_(-1.0)
        for p in pos:
            p.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same_bits(out, ref_o) and _same_bits(lse, ref_l), f"replay {i}"


def test_backward_share_replays_match_eager():
    S, C, r, B, Hq, Hkv, D = 1024, 4, 2, 1, 4, 2, 128
    t = S // (2 * C)
    scale = 1 / math.sqrt(D)
    q = _rand(1, (B, 2 * t, Hq, D))
    dout = _rand(2, (B, 2 * t, Hq, D))
    ks = [_rand(10 + o, (B, 2 * t, Hkv, D)) for o in range(C)]
    vs = [_rand(20 + o, (B, 2 * t, Hkv, D)) for o in range(C)]
    pos = [cp.zigzag_index(S, C, o, device=DEV) for o in range(C)]
    out, lse = cp.ring_share_fwd(q, ks, vs, pos, r, scale)
    dq = torch.empty((B, 2 * t, Hq, D), dtype=torch.float32, device=DEV)
    dks = [torch.empty(k.shape, dtype=torch.float32, device=DEV) for k in ks]
    dvs = [torch.empty(v.shape, dtype=torch.float32, device=DEV) for v in vs]

    def step():
        cp.ring_share_bwd(q, ks, vs, pos, r, scale, out, lse, dout, dq=dq, dk_blocks=dks, dv_blocks=dvs)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in [dq] + dks + dvs]
    g = _capture(step)
    for i in range(3):
        for x in [dq] + dks + dvs:
            x.fill_(float(i + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for j, (x, y) in enumerate(zip([dq] + dks + dvs, ref)):
            assert _same_bits(x, y), f"replay {i}, tensor {j}"

"""Forward launches that take their query tiles from work queues at run time.

Launches of at least 1024 blocks (four rounds of the chip's CUs) let each block claim its
tile from a queue (one per XCD when the columns divide by 8, else one for all) instead of
taking the tile its block index names, so that XCDs holding higher clocks under load take
over the others' last tiles.  Each tile is still computed by exactly one block with the same
code, so results do not depend on which block takes which tile.  Checked here: sampled rows
against the oracle with 8 queues and with 1 (ragged last tiles), bit-identical repeats, two
launches in flight on two streams (each call takes its own counter slot), and replays of a
captured launch (the counters are reset by a kernel, not a memset, so every replay starts
from zero)."""
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


def _inputs(seed, B, S, Hq, Hkv, D=128):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, S, Hq, D), generator=g).to(torch.bfloat16)
    k = torch.randn((B, S, Hkv, D), generator=g).to(torch.bfloat16)
    v = torch.randn((B, S, Hkv, D), generator=g).to(torch.bfloat16)
    return q, k, v


def _blocks_12wave(S, Hq, Hkv):
    """Blocks of the 12-wave causal launch (384 / G positions per block)."""
    ratio = Hq // Hkv
    G = 4 if ratio % 4 == 0 else 2 if ratio % 2 == 0 else 1
    return -(-S // (384 // G)) * (Hq // G)


@pytest.mark.parametrize("S,Hq,Hkv", [(30001, 16, 16), (40003, 12, 12), (20011, 32, 8)])
def test_queue_launch_against_oracle(S, Hq, Hkv):
    """Causal self-attention with 8 queues (16 columns; 8 columns of GQA groups) and with one
    (12 columns), ragged last tiles; sampled rows against the oracle."""
    assert _blocks_12wave(S, Hq, Hkv) >= 1024
    D = 128
    scale = 1 / math.sqrt(D)
    q, k, v = _inputs(S % 991, 1, S, Hq, Hkv, D)
    pos = np.arange(S, dtype=np.int64)
    rng = np.random.default_rng(S)
    rows = np.unique(np.concatenate([[0, 1, 383, 384, S - 385, S - 384, S - 2, S - 1],
                                     rng.integers(0, S, 24)])).astype(np.int64)
    ref_o, ref_l = oracle.attention_rows(q.float().numpy(), k.float().numpy(), v.float().numpy(), pos, pos, scale,
                                         rows=rows)
    tp = torch.from_numpy(pos).to(DEV)
    out, lse = cp.block_fwd(q.to(DEV), k.to(DEV), v.to(DEV), tp, tp, scale)
    torch.cuda.synchronize()
    tol_o, tol_l = TOL["bf16"]
    eo = max_abs(out[:, rows].cpu().numpy(), ref_o)
    el = max_abs(lse[:, :, rows].cpu().numpy(), ref_l)
    assert eo <= tol_o and el <= tol_l, f"max abs err O {eo:.3g} lse {el:.3g}"
    # the same bits on a second call, whichever blocks take which tiles this time
    out2, lse2 = cp.block_fwd(q.to(DEV), k.to(DEV), v.to(DEV), tp, tp, scale)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_queue_launches_on_two_streams():
    """Two queue launches in flight at once on two streams give what they give one after the
    other."""
    S, Hq, Hkv, D = 16384, 32, 8, 128
    assert _blocks_12wave(S, Hq, Hkv) >= 1024
    scale = 1 / math.sqrt(D)
    tp = torch.arange(S, device=DEV)
    ins = [tuple(x.to(DEV) for x in _inputs(seed, 1, S, Hq, Hkv, D)) for seed in (5, 6)]
    outs = [(torch.empty((1, S, Hq, D), device=DEV), torch.empty((1, Hq, S), device=DEV)) for _ in range(2)]
    refs = [cp.block_fwd(*x, tp, tp, scale) for x in ins]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(3):
        for s in streams:
            s.wait_stream(torch.cuda.current_stream())
        for s, x, (o, l) in zip(streams, ins, outs):
            with torch.cuda.stream(s):
                cp.block_fwd(*x, tp, tp, scale, out=o, lse=l)
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for (o, l), (ro, rl) in zip(outs, refs):
            assert torch.equal(o, ro) and torch.equal(l, rl)


def test_queue_launch_graph_replays():
    """A captured queue launch replayed several times, with eager calls on the same buffers in
    between: every replay gives the eager bits."""
    S, Hq, Hkv, D = 16384, 32, 8, 128
    scale = 1 / math.sqrt(D)
    tp = torch.arange(S, device=DEV)
    q, k, v = (x.to(DEV) for x in _inputs(9, 1, S, Hq, Hkv, D))
    ref_o, ref_l = cp.block_fwd(q, k, v, tp, tp, scale)
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)

    def step():
        cp.block_fwd(q, k, v, tp, tp, scale, out=out, lse=lse)

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
    for i in range(4):
        out.fill_(7.0)
        lse.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i}"
        step()  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o)

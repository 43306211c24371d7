"""Seeded synthetic inputs for the rank-share attention workloads.

This module only draws random numbers and rounds them to the storage dtype; it holds none
of the attention, layout or merge arithmetic.  Both the HIP path (tests, bench) and the CPU
oracle take their inputs from here, so the two see bit-identical values.

Recipe: tensor ``name`` in {q, k, v, dout} (dout: the output gradient of the backward) is drawn one sequence chunk at a time.  Chunk ``c``
(tokens [c*chunk_len, (c+1)*chunk_len) of the global sequence) comes from
``torch.Generator().manual_seed(seed + 1_000_003 * tensor_id + c)`` as iid N(0, 1) fp32
of shape [B, chunk_len, H, D], then rounded to the storage dtype (bf16 with
round-to-nearest-even).  Any chunk can thus be rebuilt alone, without the others.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "dout": 3}
SEED_STRIDE = 1_000_003


def chunk(name: str, c: int, *, batch: int, chunk_len: int, heads: int, head_dim: int,
          dtype: torch.dtype, seed: int = 0) -> torch.Tensor:
    """One chunk of tensor ``name``: CPU tensor [batch, chunk_len, heads, head_dim]."""
    g = torch.Generator().manual_seed(seed + SEED_STRIDE * TENSOR_IDS[name] + int(c))
    x = torch.randn((batch, chunk_len, heads, head_dim), generator=g, dtype=torch.float32)
    return x.to(dtype)


def chunks(name: str, ids, *, threads: int = 8, **kw) -> torch.Tensor:
    """Chunks ``ids`` of tensor ``name`` concatenated along the sequence axis, in the
    given order.  Chunks are drawn in parallel (each has its own generator)."""
    ids = [int(c) for c in ids]
    if len(ids) == 1:
        return chunk(name, ids[0], **kw)
    with ThreadPoolExecutor(max_workers=max(1, min(threads, len(ids)))) as ex:
        parts = list(ex.map(lambda c: chunk(name, c, **kw), ids))
    return torch.cat(parts, dim=1)

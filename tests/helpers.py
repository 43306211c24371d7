"""Test-side helpers: inputs for the workloads (from the seeded generator) and row samples.

Inputs are drawn once per global chunk by ``context_causal_attention_amd.synthetic``; the
HIP path gets the bf16 (or fp32) tensors, the oracle gets the same values upcast to fp32.
"""
from __future__ import annotations

import numpy as np
import torch

from context_causal_attention_amd import synthetic
from context_causal_attention_amd.workloads import Workload

TORCH_DTYPE = {"bf16": torch.bfloat16, "fp32": torch.float32}

# tolerances stated for the method: fp32 configs 1e-5 max abs on O and lse; bf16 configs
# 1e-2 on O and 1e-3 on lse, against fp64 on the same rounded inputs
TOL = {"fp32": (1e-5, 1e-5), "bf16": (1e-2, 1e-3)}


def gen(w: Workload, name: str, chunk_ids, heads: int) -> torch.Tensor:
    """Chunks ``chunk_ids`` (each of w.chunk_len tokens) of tensor ``name``, CPU."""
    return synthetic.chunks(name, chunk_ids, batch=w.batch, chunk_len=w.chunk_len, heads=heads,
                            head_dim=w.head_dim, dtype=TORCH_DTYPE[w.dtype])


def zigzag_chunks(C: int, r: int) -> list[int]:
    """Chunk ids rank r holds under zigzag sharding, as the workloads state their inputs."""
    return [r, 2 * C - 1 - r]


def sample_rows(n: int, chunk: int, seed: int, per_chunk_random: int = 16) -> np.ndarray:
    """Local row indices to compare at full size: each chunk's first and last rows, the rows
    around the 128-row tile edges, and seeded random rows."""
    rng = np.random.default_rng(seed)
    rows = set()
    for c0 in range(0, n, chunk):
        for off in (0, 1, 63, 64, 127, 128, 129, chunk - 1):
            if 0 <= off < chunk:
                rows.add(c0 + off)
        rows.update((c0 + rng.integers(0, chunk, per_chunk_random)).tolist())
    return np.array(sorted(r for r in rows if r < n), dtype=np.int64)


def max_abs(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):  # inf - inf on the rows excluded by both_inf
        d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nan_to_num(d, nan=np.inf).max()) if d.size else 0.0


def f32np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy()

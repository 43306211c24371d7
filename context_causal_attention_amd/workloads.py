"""The synthetic workloads the library is checked and measured on.

Each is a rank's (or head group's) share of causal attention under context parallelism,
with the shapes the pages work with: zigzag sharding with C=4 ("On Context Parallelism",
section "All-gather"), the 32K-token four-GPU case ("Context parallelism -- splitting the
sequence across GPUs", "Worked example"), 32 query / 8 KV heads of D=128 ("Context
parallelism: Ring Attention and Ulysses", "Exercises"), bf16 at B=1 and D=128 ("On Context
Parallelism", "Results and Conclusion").  Inputs are iid N(0,1) from ``synthetic``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "ring_share" | "allgather" | "ulysses" | "usp"
    batch: int
    seq_len: int
    heads_q: int
    heads_kv: int
    head_dim: int
    dtype: str         # "fp32" | "bf16"
    cp_size: int
    rank: int | None = None    # ring_share, usp: the rank whose share is computed (None: every rank)
    group: int | None = None   # ulysses: the head group
    a2a: int | None = None     # usp: all-to-all group size A (ring size R = C / A)
    zigzag: bool = False       # ulysses: zigzag shards (the exchange folds in the chunk reorder)

    @property
    def chunk_len(self) -> int:
        """t = S / (2C): one zigzag chunk, also the unit the inputs are drawn in."""
        return self.seq_len // (2 * self.cp_size)

    @property
    def sharding(self) -> str:
        """How the sequence is split over the C ranks: zigzag (rank r owns chunks r and
        2C-1-r) for the ring, all-gather and mesh shares and the zigzag Ulysses workload;
        contiguous (rank r owns [r*S/C, (r+1)*S/C)) for the plain Ulysses workload."""
        if self.kind == "ulysses" and not self.zigzag:
            return "contiguous"
        return "zigzag"

    @property
    def local_len(self) -> int:
        return self.seq_len // self.cp_size

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def zigzag_pairs_per_head(self) -> int:
        """Unmasked (query, key) pairs of one zigzag rank, per batch and query head:
        chunk c's t queries see c*t^2 + t(t+1)/2 keys; chunks r and 2C-1-r add up to
        2C*t^2 + t whatever r is."""
        t, C = self.chunk_len, self.cp_size
        return 2 * C * t * t + t

    def usp_pairs_per_head(self) -> int:
        """A mesh rank's share: its A2A group's tokens form rank g's zigzag shard over R,
        so per query head of its group it sees 2R t'^2 + t' pairs with t' = S/(2R)."""
        R = self.cp_size // self.a2a
        t2 = self.seq_len // (2 * R)
        return 2 * R * t2 * t2 + t2

    def causal_pairs_per_head(self) -> int:
        S = self.seq_len
        return S * (S + 1) // 2


WORKLOADS = {
    w.name: w
    for w in (
        Workload("tiny_fp32", "ring_share", 1, 256, 2, 2, 64, "fp32", 4, rank=None),
        Workload("rank_share_8k", "ring_share", 1, 8192, 16, 16, 128, "bf16", 4, rank=3),
        Workload("allgather_32k", "allgather", 1, 32768, 32, 32, 128, "bf16", 4, rank=None),
        Workload("ulysses_gqa_128k", "ulysses", 1, 131072, 32, 8, 128, "bf16", 8, group=3),
        Workload("ring_share_256k", "ring_share", 1, 262144, 32, 8, 128, "bf16", 8, rank=3),
        # zigzag-sharded Ulysses (exchange with the chunk reorder folded in) and one rank of
        # the two-dimensional mesh ("On Context Parallelism", "Peer-to-peer + All-to-all":
        # C = 8 as A = 2 times R = 4; rank 3 is ring position 1, head group 1)
        Workload("ulysses_zz_128k", "ulysses", 1, 131072, 32, 8, 128, "bf16", 8, group=3, zigzag=True),
        Workload("usp_128k", "usp", 1, 131072, 32, 8, 128, "bf16", 8, rank=3, a2a=2),
    )
}

"""bench.py on the CPU: the one-GPU contract and the FLOP accounting of the workloads."""
from __future__ import annotations

import subprocess
import sys
from dataclasses import replace
from pathlib import Path

import numpy as np

import oracle
from context_causal_attention_amd.workloads import WORKLOADS

ROOT = Path(__file__).resolve().parent.parent


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_unmasked_pair_counts_match_oracle():
    """The closed forms the metric counts FLOPs with, against the oracle's exact count on
    shrunken copies of every workload (same C, rank and chunk structure)."""
    for w in WORKLOADS.values():
        small = replace(w, seq_len=2 * w.cp_size * 24)
        kv = np.arange(small.seq_len)
        if w.kind == "ulysses":
            assert small.causal_pairs_per_head() == oracle.visible_pairs(kv, kv)
            continue
        ranks = [w.rank] if w.rank is not None else range(w.cp_size)
        for r in ranks:
            zz = oracle.zigzag_positions(small.seq_len, w.cp_size, r)
            assert small.zigzag_pairs_per_head() == oracle.visible_pairs(zz, kv)

#!/usr/bin/env python3
"""Benchmark: causal-attention TFLOP/s of one context-parallel rank's share on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--mode single|fused|unfused] [--pass fwd|bwd]

A step is one pass of the whole hot path over one batch of synthetic input already resident
in HBM.  For the default workload (ring_share_256k: S=262144, C=8 zigzag, rank 3, 32 query /
8 KV heads, D=128, bf16) that is: the zigzag positions of every owner, then for each of the
8 ring steps one block attention of the rank's 32768 local queries against the owner's
32768-token K/V shard, all in ONE launch that walks the 8 blocks in ring order with one running
softmax per row, which folds the blocks together as the LSE merge would (``--mode fused``: one
launch per step, merging in the epilogue; ``--mode unfused``: per-step tiles and the merge
kernel).  ``--pass bwd`` times the ring-share backward instead.

The value is whole-job throughput in TFLOP/s counting unmasked FLOPs only: 4*D FLOPs per
visible (query, key) pair and query head (two matrix products; softmax not counted).
The line also carries the roofline of the dominant kernel (block attention, measured with
HIP events around each of its launches inside the timed steps), the CPU oracle timed on
a bounded sample of the same workload (``cpu_baseline``: its rate, the one-thread rate and the
full share's time extrapolated from it), the bandwidth of the layout and merge kernels of the
step (``hbm_kernels``, HIP events), the median and minimum step time, and the device
(``device``: CU count and maximum clock as the device reports them, and the graphics clock
read from the GPU metrics while the workload runs).

One GPU only: --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "causal attn TFLOP/s per rank share (unmasked FLOPs) + % of bf16 MFMA peak"
METRIC_BWD = ("causal attn backward TFLOP/s per rank share (10*D FLOPs per unmasked pair and query "
              "head) + % of bf16 MFMA peak")
PEAK_BF16_TFLOPS = 2500.0   # MI355X published dense bf16 matrix peak
PEAK_FP32_TFLOPS = 157.3    # MI355X published fp32 vector peak
PEAK_HBM_GBS = 8000.0       # MI355X published HBM3E bandwidth


def parse_args(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="ring_share_256k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="bwd: time the ring-share backward (delta + cpattn_ring_share_bwd; with "
                         "--mode unfused, one cpattn_block_bwd per ring step) instead of the forward; "
                         "ring_share workloads only")
    ap.add_argument("--mode", choices=("single", "fused", "unfused"), default="single",
                    help="ring share: one launch over all ring blocks (single), one launch per step "
                         "merging in its epilogue (fused), or per-step tiles plus the merge kernel "
                         "(unfused); Ulysses: the workload's explicit permute kernels around the "
                         "attention (default), or, with one batch and contiguous shards, the "
                         "exchanges as the attention's row addressing (fused)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-sclk", action="store_true",
                    help="skip the clock reading (2 s of extra untimed steps after the timed ones)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step in a HIP graph and time its replays (for launch-bound "
                         "small workloads); the attention launches are then timed as part of the step")
    ap.add_argument("--extras", default=None,
                    help="comma-separated workload[:mode] list measured after the main line and reported "
                         "under 'extra' (mode 'bwd': the workload's backward; default: the Ulysses group in "
                         "its explicit and its fused form, the per-step ring share and the ring share's "
                         "backward when the main line is the default one; '' for none)")
    ap.add_argument("--no-flush", action="store_true",
                    help="skip the bandwidth-bound kernels' separate timing under the MALL flush")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the steps, run one plain elementwise copy (torch.neg over fp32, "
                         "cached loads and stores) of this many MiB, as the reference dispatch for "
                         "hardware byte counters")
    return ap.parse_args(argv)


class Plan:
    """Buffers and the launch sequence of one step of a workload."""

    def __init__(self, w, dev, mode="single", backward=False):
        import torch
        import context_causal_attention_amd as cp
        from context_causal_attention_amd import synthetic

        self.w, self.dev, self.cp, self.torch = w, dev, cp, torch
        td = {"bf16": torch.bfloat16, "fp32": torch.float32}[w.dtype]
        kw = dict(batch=w.batch, chunk_len=w.chunk_len, head_dim=w.head_dim, dtype=td)
        C = w.cp_size
        self.kind = w.kind
        self.mode = mode
        self.attn_flops = []   # FLOPs of each block attention launch of a step, in order
        if w.kind == "ring_share":
            # the rank's share, or every rank's share when the workload names no rank
            self.ranks = [w.rank] if w.rank is not None else list(range(C))
            self.qs = {r: synthetic.chunks("q", [r, 2 * C - 1 - r], heads=w.heads_q, **kw).to(dev) for r in self.ranks}
            self.k = [synthetic.chunks("k", [o, 2 * C - 1 - o], heads=w.heads_kv, **kw).to(dev) for o in range(C)]
            self.v = [synthetic.chunks("v", [o, 2 * C - 1 - o], heads=w.heads_kv, **kw).to(dev) for o in range(C)]
            # every owner's positions, one row each, written by one launch per step
            self.pos_all = torch.empty((C, w.local_len), dtype=torch.int64, device=dev)
            self.pos = list(self.pos_all.unbind(0))
            self.out = torch.empty((w.batch, w.local_len, w.heads_q, w.head_dim), dtype=torch.float32, device=dev)
            self.lse = torch.empty((w.batch, w.heads_q, w.local_len), dtype=torch.float32, device=dev)
            if mode == "unfused":
                self.tout = torch.empty_like(self.out)
                self.tlse = torch.empty_like(self.lse)
            t = w.chunk_len
            for r in self.ranks:
                for step in range(C):
                    owner = (r - step) % C
                    pairs = 2 * t * t + t if owner == r else 2 * t * t
                    self.attn_flops.append(4.0 * w.batch * w.heads_q * w.head_dim * pairs)
        elif w.kind == "allgather":
            gather = [c for rr in range(C) for c in (rr, 2 * C - 1 - rr)]
            self.kg = synthetic.chunks("k", gather, heads=w.heads_kv, **kw).to(dev)
            self.vg = synthetic.chunks("v", gather, heads=w.heads_kv, **kw).to(dev)
            self.kseq = torch.empty_like(self.kg)
            self.vseq = torch.empty_like(self.vg)
            self.qs = [synthetic.chunks("q", [rr, 2 * C - 1 - rr], heads=w.heads_q, **kw).to(dev) for rr in range(C)]
            # every owner's positions, one row each, written by one launch per step
            self.pos_all = torch.empty((C, w.local_len), dtype=torch.int64, device=dev)
            self.pos = list(self.pos_all.unbind(0))
            self.gpos = torch.arange(w.seq_len, device=dev)
            self.out = torch.empty((w.batch, w.local_len, w.heads_q, w.head_dim), dtype=torch.float32, device=dev)
            self.lse = torch.empty((w.batch, w.heads_q, w.local_len), dtype=torch.float32, device=dev)
            t = w.chunk_len
            for rr in range(C):
                pairs = 2 * C * t * t + t
                self.attn_flops.append(4.0 * w.batch * w.heads_q * w.head_dim * pairs)
        elif w.kind == "ulysses":
            s, g = w.local_len, w.group
            if w.zigzag:
                # rank src's shard: chunks src and 2C-1-src
                shard = lambda name, H, src: synthetic.chunks(name, [src, 2 * C - 1 - src], heads=H, **kw)
                stack_z = lambda name, H: torch.stack([shard(name, H, src) for src in range(C)]).to(dev)
                self.qst = stack_z("q", w.heads_q)
                self.kst = stack_z("k", w.heads_kv)
                self.vst = stack_z("v", w.heads_kv)
            else:
                stack = lambda x: x.reshape(w.batch, C, s, *x.shape[2:]).transpose(0, 1).contiguous()
                ids = range(2 * C)
                self.qst = stack(synthetic.chunks("q", ids, heads=w.heads_q, **kw)).to(dev)
                self.kst = stack(synthetic.chunks("k", ids, heads=w.heads_kv, **kw)).to(dev)
                self.vst = stack(synthetic.chunks("v", ids, heads=w.heads_kv, **kw)).to(dev)
            hq, hk = w.heads_q // C, w.heads_kv // C
            self.qg = torch.empty((w.batch, w.seq_len, hq, w.head_dim), dtype=td, device=dev)
            self.kgp = torch.empty((w.batch, w.seq_len, hk, w.head_dim), dtype=td, device=dev)
            self.vgp = torch.empty_like(self.kgp)
            self.gpos = torch.arange(w.seq_len, device=dev)
            self.og = torch.empty((w.batch, w.seq_len, hq, w.head_dim), dtype=torch.float32, device=dev)
            self.lg = torch.empty((w.batch, hq, w.seq_len), dtype=torch.float32, device=dev)
            self.ost = torch.zeros((C, w.batch, s, w.heads_q, w.head_dim), dtype=torch.float32, device=dev)
            S = w.seq_len
            # one batch, contiguous shards: global row i of the group is row i of the stacked
            # buffers at the group's head offset, so the attention reads and writes them in place
            self.rows = mode == "fused" and w.batch == 1 and not w.zigzag and td == torch.bfloat16
            if self.rows:
                Hq, Hk = w.heads_q, w.heads_kv
                self.qrows = self.qst.view(S, Hq, w.head_dim)[:, g * hq:(g + 1) * hq]
                self.krows = self.kst.view(S, Hk, w.head_dim)[:, g * hk:(g + 1) * hk]
                self.vrows = self.vst.view(S, Hk, w.head_dim)[:, g * hk:(g + 1) * hk]
                self.orows = self.ost.view(S, Hq, w.head_dim)[:, g * hq:(g + 1) * hq]
            self.attn_flops.append(4.0 * w.batch * hq * w.head_dim * (S * (S + 1) // 2))
        elif w.kind == "usp":
            A = w.a2a
            R = C // A
            self.R, self.g, self.a = R, w.rank // A, w.rank % A
            shard = lambda name, H, r: synthetic.chunks(name, [r, 2 * C - 1 - r], heads=H, **kw)
            # A2A group o's stacked shards (its A ranks o*A .. o*A+A-1)
            grp = lambda name, H, o: torch.stack([shard(name, H, o * A + j) for j in range(A)]).to(dev)
            self.qst = grp("q", w.heads_q, self.g)
            self.ksts = [grp("k", w.heads_kv, o) for o in range(R)]
            self.vsts = [grp("v", w.heads_kv, o) for o in range(R)]
            n = w.seq_len // R
            hq, hk = w.heads_q // A, w.heads_kv // A
            self.qh = torch.empty((w.batch, n, hq, w.head_dim), dtype=td, device=dev)
            self.kh = [torch.empty((w.batch, n, hk, w.head_dim), dtype=td, device=dev) for _ in range(R)]
            self.vh = [torch.empty((w.batch, n, hk, w.head_dim), dtype=td, device=dev) for _ in range(R)]
            self.pos_all = torch.empty((R, n), dtype=torch.int64, device=dev)
            self.pos = list(self.pos_all.unbind(0))
            self.out = torch.empty((w.batch, n, hq, w.head_dim), dtype=torch.float32, device=dev)
            self.lse = torch.empty((w.batch, hq, n), dtype=torch.float32, device=dev)
            self.ost = torch.zeros((A, w.batch, w.local_len, w.heads_q, w.head_dim), dtype=torch.float32,
                                   device=dev)
            t2 = w.seq_len // (2 * R)
            for step in range(R):
                owner = (self.g - step) % R
                pairs = 2 * t2 * t2 + t2 if owner == self.g else 2 * t2 * t2
                self.attn_flops.append(4.0 * w.batch * hq * w.head_dim * pairs)
        else:
            raise ValueError(w.kind)
        self.backward = False
        if backward:
            if w.kind != "ring_share" or w.rank is None:
                raise ValueError("--pass bwd needs a ring_share workload with a rank")
            # the saved forward state comes from this library's forward, run once here
            r = w.rank
            self.step()
            torch.cuda.synchronize()
            self.dout = synthetic.chunks("dout", [r, 2 * C - 1 - r], heads=w.heads_q, **kw).to(dev)
            self.dq = torch.empty_like(self.out)
            self.dks = [torch.empty(k.shape, dtype=torch.float32, device=dev) for k in self.k]
            self.dvs = [torch.empty(v.shape, dtype=torch.float32, device=dev) for v in self.v]
            self.delta = torch.empty_like(self.lse)
            # algorithmic backward FLOPs: 10*D per visible pair and query head (S = QK^T
            # recomputed, dP = dO V^T, dV = P^T dO, dQ = dS K, dK = dS^T Q)
            self.attn_flops = [f * 2.5 for f in self.attn_flops]
            # "unfused": one cpattn_block_bwd per ring step; otherwise the share's one
            # cpattn_ring_share_bwd call (dq per step, one dk/dv launch over all blocks), timed
            # as one unit
            self.bwd_steps = mode == "unfused"
            if not self.bwd_steps:
                self.attn_flops = [sum(self.attn_flops)]
            self.backward = True
        self.flops = sum(self.attn_flops)
        self.hbm_ev = []  # (kernel, bytes, start, end) of the timed steps' bandwidth-bound kernels

    def step(self, ev=None):
        """Launch one step on the current stream.  ev: list to which (start, end) event
        pairs around each block attention launch are appended."""
        cp, torch, w = self.cp, self.torch, self.w
        C = w.cp_size
        if getattr(self, "backward", False):
            return self.step_bwd(ev)

        def attn(*a, fn=cp.block_fwd):
            if ev is not None:
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                fn(*a)
                e.record()
                ev.append((s, e))
            else:
                fn(*a)

        def hbm(name, nbytes, fn, *a, **kw):
            """A bandwidth-bound layout or merge kernel, timed when the step is timed."""
            if ev is not None:
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                fn(*a, **kw)
                e.record()
                self.hbm_ev.append((name, nbytes, s, e))
            else:
                fn(*a, **kw)

        if self.kind == "ring_share":
            cp.zigzag_index_all(w.seq_len, C, out=self.pos_all)
            for r in self.ranks:
                q = self.qs[r]
                order = [(r - step) % C for step in range(C)]
                if self.mode == "single":
                    attn(q, [self.k[o] for o in order], [self.v[o] for o in order], [self.pos[o] for o in order],
                         self.pos[r], w.scale, self.out, self.lse, fn=cp.ring_blocks_fwd)
                    continue
                for step, owner in enumerate(order):
                    a = (q, self.k[owner], self.v[owner], self.pos[r], self.pos[owner], w.scale)
                    if step == 0:
                        attn(*a, self.out, self.lse)
                    elif self.mode == "fused":
                        attn(*a, self.out, self.lse, fn=cp.block_fwd_merge)
                    else:
                        attn(*a, self.tout, self.tlse)
                        hbm("lse_merge_kernel", 3 * (self.out.numel() + self.lse.numel()) * 4,
                            cp.lse_merge, self.out, self.lse, self.tout, self.tlse)
        elif self.kind == "allgather":
            nb = 2 * self.kg.numel() * self.kg.element_size()
            hbm("reorder_kernel", nb, cp.reorder_gathered, self.kg, C, cp.RANK_TO_SEQ, out=self.kseq)
            hbm("reorder_kernel", nb, cp.reorder_gathered, self.vg, C, cp.RANK_TO_SEQ, out=self.vseq)
            cp.zigzag_index_all(w.seq_len, C, out=self.pos_all)
            for rr in range(C):
                attn(self.qs[rr], self.kseq, self.vseq, self.pos[rr], self.gpos, w.scale, self.out, self.lse)
        elif self.kind == "ulysses" and self.rows:
            attn(self.qrows, self.krows, self.vrows, self.gpos, self.gpos, w.scale, self.orows, self.lg,
                 fn=cp.block_fwd_rows)
        elif self.kind == "ulysses":
            g, zz = w.group, w.zigzag
            nb = lambda x: 2 * x.numel() * x.element_size()  # noqa: E731  (read + write)
            for src, dst in ((self.qst, self.qg), (self.kst, self.kgp), (self.vst, self.vgp)):
                hbm("ulysses_kernel", nb(dst), cp.ulysses_seq_to_heads, src, g, out=dst, zigzag=zz)
            attn(self.qg, self.kgp, self.vgp, self.gpos, self.gpos, w.scale, self.og, self.lg)
            hbm("ulysses_kernel", nb(self.og), cp.ulysses_heads_to_seq, self.og, g, self.ost, zigzag=zz)
        else:
            # the group's exchange for this rank's head group (every ring owner's K/V
            # exchange included, although on a mesh each group does its own), then the
            # ring over the R owners and the inverse exchange of the output
            R, g, a = self.R, self.g, self.a
            nb = lambda x: 2 * x.numel() * x.element_size()  # noqa: E731  (read + write)
            hbm("ulysses_kernel", nb(self.qh), cp.ulysses_seq_to_heads, self.qst, a, out=self.qh, zigzag=True)
            for o in range(R):
                hbm("ulysses_kernel", nb(self.kh[o]), cp.ulysses_seq_to_heads, self.ksts[o], a, out=self.kh[o],
                    zigzag=True)
                hbm("ulysses_kernel", nb(self.vh[o]), cp.ulysses_seq_to_heads, self.vsts[o], a, out=self.vh[o],
                    zigzag=True)
            cp.zigzag_index_all(w.seq_len, R, out=self.pos_all)
            for step in range(R):
                owner = (g - step) % R
                a_ = (self.qh, self.kh[owner], self.vh[owner], self.pos[g], self.pos[owner], w.scale)
                if step == 0:
                    attn(*a_, self.out, self.lse)
                else:
                    attn(*a_, self.out, self.lse, fn=cp.block_fwd_merge)
            hbm("ulysses_kernel", nb(self.out), cp.ulysses_heads_to_seq, self.out, a, self.ost, zigzag=True)


    def hbm_calls(self):
        """The bandwidth-bound kernels of this plan's step, each as (kernel, algorithmic bytes,
        callable launching it once on the current stream), for timing them one at a time."""
        cp, w = self.cp, self.w
        C = w.cp_size
        nb = lambda x: 2 * x.numel() * x.element_size()  # noqa: E731  (read + write)
        calls = []
        if self.backward:
            n = self.out.numel() * 4 + self.dout.numel() * self.dout.element_size() + self.delta.numel() * 4
            calls.append(("delta_kernel", n, lambda: cp.attn_bwd_delta(self.out, self.dout, self.delta)))
        elif self.kind == "ring_share" and self.mode == "unfused":
            n = 3 * (self.out.numel() + self.lse.numel()) * 4
            calls.append(("lse_merge_kernel", n, lambda: cp.lse_merge(self.out, self.lse, self.tout, self.tlse)))
        elif self.kind == "allgather":
            calls.append(("reorder_kernel", nb(self.kg),
                          lambda: cp.reorder_gathered(self.kg, C, cp.RANK_TO_SEQ, out=self.kseq)))
        elif self.kind == "ulysses" and not self.rows:
            g, zz = w.group, w.zigzag
            for name, src, dst in (("q", self.qst, self.qg), ("k", self.kst, self.kgp), ("v", self.vst, self.vgp)):
                calls.append((f"ulysses_kernel ({name})", nb(dst),
                              lambda src=src, dst=dst: cp.ulysses_seq_to_heads(src, g, out=dst, zigzag=zz)))
            calls.append(("ulysses_kernel (out, inverse)", nb(self.og),
                          lambda: cp.ulysses_heads_to_seq(self.og, g, self.ost, zigzag=zz)))
        return calls

    def step_bwd(self, ev=None):
        """One rank share of the ring backward: delta, then the share's backward in one call
        (cpattn_ring_share_bwd), or ("unfused") the block backward of each ring step (dq
        written at step 0 and added after; each owner's dk, dv written by its step)."""
        cp, torch, w = self.cp, self.torch, self.w
        C, r = w.cp_size, w.rank
        nb = self.out.numel() * 4 + self.dout.numel() * self.dout.element_size() + self.delta.numel() * 4
        if ev is not None:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            cp.attn_bwd_delta(self.out, self.dout, self.delta)
            e.record()
            self.hbm_ev.append(("delta_kernel", nb, s, e))
        else:
            cp.attn_bwd_delta(self.out, self.dout, self.delta)
        q = self.qs[r]
        if not self.bwd_steps:
            order = [(r - step) % C for step in range(C)]
            a = (q, self.dout, [self.k[o] for o in order], [self.v[o] for o in order], [self.pos[o] for o in order],
                 self.pos[r], w.scale, self.lse, self.delta, self.dq, [self.dks[o] for o in order],
                 [self.dvs[o] for o in order])
            if ev is not None:
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                cp.ring_blocks_bwd(*a)
                e.record()
                ev.append((s, e))
            else:
                cp.ring_blocks_bwd(*a)
            return
        for step in range(C):
            owner = (r - step) % C
            flags = cp.BWD_WRITE_DKV | (cp.BWD_WRITE_DQ if step == 0 else 0)
            a = (q, self.k[owner], self.v[owner], self.dout, self.pos[r], self.pos[owner], w.scale, self.lse,
                 self.delta, self.dq, self.dks[owner], self.dvs[owner], flags)
            if ev is not None:
                s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                s.record()
                cp.block_bwd(*a)
                e.record()
                ev.append((s, e))
            else:
                cp.block_bwd(*a)


def _pci_bdf(index: int):
    """PCI address of HIP device ``index`` ("0000:05:00.0"), or None."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        buf = ctypes.create_string_buffer(64)
        if hip.hipDeviceGetPCIBusId(buf, 64, index) != 0:
            return None
        return buf.value.decode().lower()
    except OSError:
        return None


def _hip_max_sclk_mhz(index: int):
    """The device's maximum graphics clock (hipDeviceAttributeClockRate, kHz) in MHz, or None."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, index) != 0 or v.value <= 0:
            return None
        return v.value / 1000.0
    except OSError:
        return None


def sclk_under_load(plan, index: int, seconds: float = 2.0, settle: float = 1.0):
    """Graphics clock of the benchmarked GPU while it runs this workload: the steps are
    repeated (untimed) for ``seconds`` while a thread reads the per-XCD clocks from the amdsmi
    GPU metrics every 50 ms; readings from the first ``settle`` seconds are dropped, since the
    telemetry refreshes about once a second.  None-valued where the telemetry is unreadable."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
    except Exception as e:  # telemetry is optional
        return {"mhz_mean": None, "note": f"amdsmi unavailable: {type(e).__name__}"}
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        bdf = _pci_bdf(index)
        match = [h for h in handles if bdf and str(amdsmi.amdsmi_get_gpu_device_bdf(h)).lower() == bdf]
        h = match[0] if match else (handles[0] if len(handles) == 1 else None)
        if h is None:
            return {"mhz_mean": None, "note": "benchmarked GPU not found among amdsmi devices"}
        samples, stop = [], threading.Event()
        t0 = time.perf_counter()

        def run():
            while not stop.is_set():
                if time.perf_counter() - t0 >= settle:
                    try:
                        xs = [float(x) for x in amdsmi.amdsmi_get_gpu_metrics_info(h)["current_gfxclks"]
                              if isinstance(x, (int, float))]
                        if xs:
                            samples.append(xs)
                    except Exception:
                        pass
                stop.wait(0.05)
        th = threading.Thread(target=run, daemon=True)
        th.start()
        while time.perf_counter() - t0 < seconds:
            plan.step()
            torch.cuda.synchronize()
        stop.set()
        th.join()
        if not samples:
            return {"mhz_mean": None, "note": "no readings"}
        per_xcd = [sum(col) / len(col) for col in zip(*samples)]
        return {"mhz_mean": round(sum(per_xcd) / len(per_xcd), 1),
                "mhz_per_xcd": [round(x) for x in per_xcd], "samples": len(samples),
                "source": f"amdsmi GPU metrics current_gfxclks over {seconds - settle:.0f} s of extra untimed steps"}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def profiled_traffic(workload: str, kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter summary of
    this workload, or None when there is none or the kernel source changed since."""
    import hashlib
    f = ROOT / "profiles" / f"block_fwd_bf16_{workload}_traffic.txt"
    src = ROOT / "context_causal_attention_amd" / "csrc" / "block_fwd_bf16.hip"
    if not f.exists() or not src.exists():
        return None
    sha = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    recorded, value = None, None
    for line in f.read_text().splitlines():
        if line.startswith("kernel_source:"):
            recorded = line.split()[-1]
        if line.startswith(f"traffic_bytes_per_launch {kernel}:"):
            value = float(line.split()[-1])
    return value if recorded == sha else None


def cpu_baseline(w, budget_s: float, total_pairs: float):
    """The CPU oracle (as it stands) on a bounded sample of the same workload: direct causal
    attention of a seeded sample of the share's query rows, all heads, fp64."""
    import numpy as np
    import oracle
    from context_causal_attention_amd import synthetic
    import torch

    td = {"bf16": torch.bfloat16, "fp32": torch.float32}[w.dtype]
    kw = dict(batch=w.batch, chunk_len=w.chunk_len, head_dim=w.head_dim, dtype=td)
    C, S = w.cp_size, w.seq_len
    if w.kind == "ulysses":
        hq, hk = w.heads_q // C, w.heads_kv // C
        g = w.group
        ids = list(range(2 * C))
        q = synthetic.chunks("q", ids, heads=w.heads_q, **kw)[:, :, g * hq:(g + 1) * hq].float().numpy()
        k = synthetic.chunks("k", ids, heads=w.heads_kv, **kw)[:, :, g * hk:(g + 1) * hk].float().numpy()
        v = synthetic.chunks("v", ids, heads=w.heads_kv, **kw)[:, :, g * hk:(g + 1) * hk].float().numpy()
        qpos = np.arange(S, dtype=np.int64)
        heads = hq
    elif w.kind == "usp":
        A = w.a2a
        R = C // A
        g, a = w.rank // A, w.rank % A
        hq, hk = w.heads_q // A, w.heads_kv // A
        ids = list(range(2 * C))
        qpos = np.sort(np.concatenate([np.arange(c * w.chunk_len, (c + 1) * w.chunk_len)
                                       for j in range(A) for c in (g * A + j, 2 * C - 1 - g * A - j)]))
        q = synthetic.chunks("q", ids, heads=w.heads_q, **kw)[:, qpos, a * hq:(a + 1) * hq].float().numpy()
        k = synthetic.chunks("k", ids, heads=w.heads_kv, **kw)[:, :, a * hk:(a + 1) * hk].float().numpy()
        v = synthetic.chunks("v", ids, heads=w.heads_kv, **kw)[:, :, a * hk:(a + 1) * hk].float().numpy()
        qpos = qpos.astype(np.int64)
        heads = hq
    else:
        r = w.rank if w.rank is not None else C - 1  # one rank stands for all: equal work per rank
        q = synthetic.chunks("q", [r, 2 * C - 1 - r], heads=w.heads_q, **kw).float().numpy()
        k = synthetic.chunks("k", range(2 * C), heads=w.heads_kv, **kw).float().numpy()
        v = synthetic.chunks("v", range(2 * C), heads=w.heads_kv, **kw).float().numpy()
        qpos = oracle.zigzag_positions(S, C, r)
        heads = w.heads_q
    kvpos = np.arange(S, dtype=np.int64)
    threads = oracle.default_threads()
    rng = np.random.default_rng(0)
    n_all = q.shape[1]

    def run(n):
        rows = np.sort(rng.choice(n_all, size=n, replace=False)).astype(np.int64)
        pairs = int(np.searchsorted(kvpos, qpos[rows], side="right").sum()) * w.batch * heads
        t0 = time.perf_counter()
        oracle.attention_rows(q, k, v, qpos, kvpos, w.scale, rows=rows, nthreads=threads)
        return pairs, time.perf_counter() - t0

    pairs, dt = run(max(1, threads))                # calibration
    n = int(max(1, min(n_all, threads * budget_s / max(dt, 1e-3))))
    pairs, dt = run(n)
    flops = 4.0 * w.head_dim * pairs
    # one thread on a few rows, for the per-core rate
    rows1 = np.sort(rng.choice(n_all, size=2, replace=False)).astype(np.int64)
    pairs1 = int(np.searchsorted(kvpos, qpos[rows1], side="right").sum()) * w.batch * heads
    t0 = time.perf_counter()
    oracle.attention_rows(q, k, v, qpos, kvpos, w.scale, rows=rows1, nthreads=1)
    dt1 = time.perf_counter() - t0
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of {n_all} local query rows (seeded), all {heads} query heads, "
                      f"{pairs} visible pairs, fp64, {dt:.1f} s",
            "pairs_per_s": pairs / dt, "pairs_per_s_1_thread": pairs1 / max(dt1, 1e-9), "cpu_model": model,
            "extrapolated_full_share_s": total_pairs / (pairs / dt)}


def measure(plan, steps: int, warmup: int, graph_mode: bool = False):
    """Warm up, then time exactly ``steps`` steps with an event at every step boundary (and,
    without a graph, events around every block attention launch)."""
    import torch
    for _ in range(warmup):
        plan.step()
    torch.cuda.synchronize()
    ev = []
    plan.hbm_ev = []
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    graph = None
    if graph_mode:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            plan.step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            plan.step()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
    marks[0].record()
    for i in range(steps):
        if graph is not None:
            graph.replay()
        else:
            plan.step(ev)
        marks[i + 1].record()
    torch.cuda.synchronize()
    ms_total = marks[0].elapsed_time(marks[-1])
    ms_steps = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    if graph is not None:  # no events inside the graph: the whole step stands for its launches
        attn_ms = [m / len(plan.attn_flops) for m in ms_steps for _ in plan.attn_flops]
    else:
        attn_ms = [s.elapsed_time(e) for s, e in ev]
    hbm = {}
    for name, nbytes, s_, e_ in plan.hbm_ev:
        d = hbm.setdefault(name, [0, 0.0, 0.0])
        d[0] += 1
        d[1] += s_.elapsed_time(e_)
        d[2] += nbytes
    hbm_kernels = [{"kernel": k, "calls": c, "bytes_per_call": b / c, "avg_ms": round(ms / c, 4),
                    "GB/s": round(b / (ms * 1e-3) / 1e9, 1), "frac_of_hbm_peak": round(b / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                   for k, (c, ms, b) in hbm.items()]
    ms_step = ms_total / steps
    attn_flops = plan.attn_flops * steps
    return {"ms_step": ms_step, "ms_steps": ms_steps, "value": plan.flops / (ms_step * 1e-3) / 1e12,
            "attn_ms": attn_ms, "achieved": sum(attn_flops) / (sum(attn_ms) * 1e-3) / 1e12,
            "hbm_kernels": hbm_kernels, "graph": graph is not None}


def hbm_flushed(plan, reps: int = 5, flush_mib: int = 1024):
    """Each bandwidth-bound kernel of the plan timed alone, ``reps`` times, with a write of a
    ``flush_mib`` MiB scratch buffer before every repetition (outside the timed events), so
    that neither the 256 MB MALL nor the L2 holds its inputs when it starts."""
    import torch
    calls = plan.hbm_calls()
    if not calls:
        return []
    scratch = torch.empty((flush_mib << 20) // 4, dtype=torch.float32, device=plan.dev)
    out = []
    for name, nbytes, fn in calls:
        fn()  # warm
        ms = []
        for i in range(reps):
            scratch.fill_(float(i))
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            ms.append(s.elapsed_time(e))
        ms.sort()
        med = ms[len(ms) // 2]
        out.append({"kernel": name, "bytes_per_call": nbytes, "median_ms": round(med, 4), "min_ms": round(ms[0], 4),
                    "GB/s": round(nbytes / (med * 1e-3) / 1e9, 1),
                    "frac_of_hbm_peak": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "flush": f"{flush_mib} MiB scratch write before each of {reps} repetitions"})
    # the runtime's own device copy of the largest and the smallest call's bytes under the same
    # flush: what a plain copy of that size reaches on this chip, beside the kernels
    sizes = sorted({c[1] for c in calls})
    src = torch.empty(sizes[-1] // 2, dtype=torch.uint8, device=plan.dev)
    dst = torch.empty_like(src)
    for nbytes in sorted({sizes[0], sizes[-1]}):
        sv, dv = src[: nbytes // 2], dst[: nbytes // 2]
        dv.copy_(sv)  # warm
        ms = []
        for i in range(reps):
            scratch.fill_(float(i))
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            dv.copy_(sv)
            e.record()
            torch.cuda.synchronize()
            ms.append(s.elapsed_time(e))
        ms.sort()
        med = ms[len(ms) // 2]
        out.append({"kernel": "device copy, reference (torch copy_)", "bytes_per_call": nbytes,
                    "median_ms": round(med, 4), "min_ms": round(ms[0], 4),
                    "GB/s": round(nbytes / (med * 1e-3) / 1e9, 1),
                    "frac_of_hbm_peak": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                    "flush": f"{flush_mib} MiB scratch write before each of {reps} repetitions"})
    del src, dst
    del scratch
    return out


def workload_name(w, mode: str, bwd: bool, graph: bool) -> str:
    return (w.name + (f"_{mode}" if mode != "single" and w.kind in ("ring_share", "ulysses") else "")
            + ("_bwd" if bwd else "") + ("_graph" if graph else ""))


def extra_line(name: str, mode: str, steps: int, warmup: int, dev):
    """One more workload of the same run, reported beside the headline: its step time and
    TFLOP/s, the attention kernel's own rate and fraction of the bf16 peak, and its
    bandwidth-bound kernels (in the step, and alone under the MALL flush)."""
    import torch
    from context_causal_attention_amd.workloads import WORKLOADS
    w = WORKLOADS[name]
    bwd = mode == "bwd"  # the workload's backward (its one-launch forward saved first), 10*D FLOPs per pair
    plan = Plan(w, dev, mode="single" if bwd else mode, backward=bwd)
    m = measure(plan, steps, warmup)
    res = {"workload": workload_name(w, "single" if bwd else mode, bwd, False), "steps": steps,
           "ms_per_step": round(m["ms_step"], 4),
           "ms_per_step_median": round(m["ms_steps"][len(m["ms_steps"]) // 2], 4),
           "value": round(m["value"], 3), "unit": "TFLOP/s", "pct_of_bf16_peak": round(100.0 * m["value"] / PEAK_BF16_TFLOPS, 2),
           "attention": {"kernel": "block_bwd_dq_kernel+block_bwd_dkdv_kernel" if bwd else "block_fwd_bf16",
                         "achieved": round(m["achieved"], 3), "peak": PEAK_BF16_TFLOPS,
                         "frac": round(m["achieved"] / PEAK_BF16_TFLOPS, 4),
                         "avg_launch_ms": round(sum(m["attn_ms"]) / len(m["attn_ms"]), 4), "launches": len(m["attn_ms"])},
           "hbm_kernels": m["hbm_kernels"], "hbm_kernels_flushed": hbm_flushed(plan),
           "config": {"seq_len": w.seq_len, "cp_size": w.cp_size, "rank": w.rank, "group": w.group,
                      "sharding": w.sharding, "heads_q": w.heads_q, "heads_kv": w.heads_kv, "head_dim": w.head_dim,
                      "unmasked_flops_per_step": plan.flops}}
    del plan
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main(argv=None) -> int:
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the rank share runs all ring steps on one device).", file=sys.stderr)
        return 2
    import torch
    from context_causal_attention_amd.workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    plan = Plan(w, dev, mode=args.mode, backward=args.which == "bwd")
    if args.copy_calibration_mib > 0:
        # the library's layout kernels stream with non-temporal accesses, which the byte
        # counters report differently; the reference is a plain cached copy
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)  # reads n bytes, writes n bytes
        del src, dst
    torch.cuda.synchronize()
    m = measure(plan, args.steps, args.warmup, graph_mode=args.graph)
    sclk = {"mhz_mean": None, "note": "skipped (--no-sclk)"} if args.no_sclk else sclk_under_load(plan, dev.index or 0)
    bwd = args.which == "bwd"
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    kernel = ("block_bwd_dq_kernel+block_bwd_dkdv_kernel" if bwd else "block_fwd_bf16") \
        if w.dtype == "bf16" else ("bwd_dq_f32_kernel+bwd_dkdv_f32_kernel" if bwd else "block_fwd_f32_kernel")
    props = torch.cuda.get_device_properties(dev)
    max_mhz = _hip_max_sclk_mhz(dev.index or 0)
    device = {"name": props.name, "arch": props.gcnArchName, "cus": props.multi_processor_count,
              "max_sclk_mhz": max_mhz or None,
              # 4096 dense bf16 FLOPs per CU and clock: 256 CUs at 2.4 GHz give the published peak
              "bf16_peak_from_device_tflops": round(props.multi_processor_count * 4096 * max_mhz * 1e6 / 1e12, 1)
              if max_mhz else None,
              "sclk_under_load": sclk}
    value, ms_step, ms_steps = m["value"], m["ms_step"], m["ms_steps"]
    result = {
        "metric": METRIC_BWD if bwd else METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_median": round(ms_steps[len(ms_steps) // 2], 4),
        "ms_per_step_min": round(ms_steps[0], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded iid N(0,1), per-chunk generators)",
        "config": {"workload": workload_name(w, args.mode, bwd, m["graph"]),
                   "batch": w.batch, "a2a": w.a2a, "sharding": w.sharding, "seq_len": w.seq_len, "cp_size": w.cp_size,
                   "rank": w.rank, "group": w.group, "heads_q": w.heads_q, "heads_kv": w.heads_kv,
                   "head_dim": w.head_dim, "unmasked_flops_per_step": plan.flops},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "kernel": kernel,
                     "achieved": round(m["achieved"], 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(m["achieved"] / peak, 4),
                     "traffic": profiled_traffic(w.name, "block_fwd_bf16") if w.dtype == "bf16" and not bwd
                     else None,
                     "avg_launch_ms": round(sum(m["attn_ms"]) / len(m["attn_ms"]), 4), "launches": len(m["attn_ms"])},
        "hbm_kernels": m["hbm_kernels"],
        "hbm_kernels_flushed": hbm_flushed(plan) if not args.no_flush else [],
        "device": device,
    }
    if bwd:
        result["cpu_baseline"] = None  # the oracle baseline is quoted for the forward line
    elif not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, plan.flops / (4.0 * w.head_dim))
    if args.extras is None:
        extras = EXTRAS if (args.workload == "ring_share_256k" and args.mode == "single" and not bwd
                            and not args.graph) else []
    else:
        extras = [tuple(e.split(":")) if ":" in e else (e, "single") for e in args.extras.split(",") if e]
    if extras:
        del plan
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["extra"] = [extra_line(name, mode, args.steps, args.warmup, dev) for name, mode in extras]
    print(json.dumps(result), flush=True)
    return 0


# Measured beside the default line, in the same run: the Ulysses group with the workload's
# explicit permute, attention and inverse permute ("On Context Parallelism", All-to-all); the
# same group as the library's Ulysses share runs it, the exchanges folded into the attention's
# row addressing; the long-context ring share in its per-step form, one attention launch per
# ring step into a tile and the merge kernel after each ("On Context Parallelism",
# Peer-to-peer / Forward); and that share's backward, delta once, one dq launch per ring step
# and one dk/dv launch over all the blocks ("On Context Parallelism", Peer-to-peer / Backward).
EXTRAS = [("ulysses_gqa_128k", "single"), ("ulysses_gqa_128k", "fused"), ("ring_share_256k", "unfused"),
          ("ring_share_256k", "bwd")]


if __name__ == "__main__":
    sys.exit(main())

"""HIP attention backward against the oracle: the row term D, the block backward (both
dtypes, head dims 128 and 64, GQA, every zigzag step class, sparse positions with empty rows,
ragged tails; small
launches run the dq kernel with its keys split over two wave groups), the write/accumulate
flags, launch-size blocks with ragged ends (the 4-wave dq kernel), and the ring-share backward
at the 8K and 256K workloads (sampled rows and keys, in the launch sequence the benchmark
times; at launch size the saved forward state is synthetic, since the oracle cannot run that
forward for every row).

Tolerances: fp32, 1e-5 times max(1, largest reference magnitude).  bf16: p and ds are
rounded to bf16 (relative error <= 2^-9 each) before the products that use them; on these
inputs that moves a gradient by about 2^-9 of the largest entry, and the comparisons with the
exact backward allow 2^-7 of it.  The roundings themselves are pinned by comparing the bf16
kernels with the oracle's model of them (``bf16_pds``) at 2^-11 of the largest entry."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import context_causal_attention_amd as cp
import oracle
from context_causal_attention_amd.workloads import WORKLOADS, Workload
from helpers import gen, max_abs, sample_rows, zigzag_chunks

pytestmark = pytest.mark.gpu
DEV = "cuda"
TDT = {"bf16": torch.bfloat16, "fp32": torch.float32}


def _tol(dtype, ref):
    m = float(np.max(np.abs(ref))) if ref.size else 0.0
    return 1e-5 * max(1.0, m) if dtype == "fp32" else 2.0 ** -7 * max(m, 1e-2)


def _rand(seed, shape, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(TDT[dtype])


def _check(name, got, ref, dtype):
    got = got.cpu().numpy() if isinstance(got, torch.Tensor) else got
    err, tol = max_abs(got, ref), _tol(dtype, ref)
    assert err <= tol, f"{name}: max abs err {err:.3g} > {tol:.3g}"


def _block_case(seed, B, Sq, Skv, Hq, Hkv, D, dtype, qpos, kvpos):
    """One block that is the whole key set: out and lse from the oracle's forward."""
    q, k, v, g = (_rand(seed + i, s, dtype) for i, s in
                  enumerate(((B, Sq, Hq, D), (B, Skv, Hkv, D), (B, Skv, Hkv, D), (B, Sq, Hq, D))))
    scale = 1 / math.sqrt(D)
    qf, kf, vf, gf = (x.float().numpy() for x in (q, k, v, g))
    out, lse = oracle.attention_rows(qf, kf, vf, qpos, kvpos, scale)
    ref = oracle.block_bwd(qf, kf, vf, gf, out, lse, qpos, kvpos, scale)
    d = lambda x: x.to(DEV)  # noqa: E731
    tq, tk = torch.from_numpy(qpos).to(DEV), torch.from_numpy(kvpos).to(DEV)
    o_t = torch.from_numpy(out.astype(np.float32)).to(DEV)
    l_t = torch.from_numpy(lse.astype(np.float32)).to(DEV)
    delta = cp.attn_bwd_delta(o_t, d(g))
    dq = torch.full((B, Sq, Hq, D), 7.0, device=DEV)  # overwritten: WRITE flags
    dk = torch.full((B, Skv, Hkv, D), 7.0, device=DEV)
    dv = torch.full((B, Skv, Hkv, D), 7.0, device=DEV)
    cp.block_bwd(d(q), d(k), d(v), d(g), tq, tk, scale, l_t, delta, dq, dk, dv,
                 cp.BWD_WRITE_DQ | cp.BWD_WRITE_DKV)
    torch.cuda.synchronize()
    return (dq, dk, dv), ref, (d(q), d(k), d(v), d(g), tq, tk, scale, l_t, delta)


CASES = [
    # B, Sq, Skv, Hq, Hkv
    (1, 256, 256, 2, 2),
    (2, 200, 333, 4, 2),
    (1, 130, 70, 8, 1),
    (1, 97, 300, 6, 2),
    (1, 1, 1, 1, 1),
    (3, 45, 513, 4, 4),
]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 128), ("bf16", 64)])
@pytest.mark.parametrize("case", CASES)
def test_block_bwd_causal_contiguous(case, dtype, D):
    B, Sq, Skv, Hq, Hkv = case
    qpos = np.arange(Skv - Sq, Skv, dtype=np.int64) if Skv >= Sq else np.arange(Sq, dtype=np.int64)
    kvpos = np.arange(Skv, dtype=np.int64)
    got, ref, _ = _block_case(10, B, Sq, Skv, Hq, Hkv, D, dtype, qpos, kvpos)
    for name, x, r in zip(("dq", "dk", "dv"), got, ref):
        _check(name, x, r, dtype)


# The bf16 kernels against the oracle's model of their two roundings (p and ds to bf16,
# nearest-even, ds formed from the unrounded p; all else fp64): what remains is fp32
# arithmetic (accumulation, exp2, and ds = p (dp - D) where dp and D nearly cancel) and the
# bf16 roundings it tips the other way; measured at most 1.5e-4 (D = 128) and 3.1e-4 (D = 64)
# of the largest entry, against 0.9e-3 - 2.9e-3 (about 2^-9) between the kernels and the exact
# backward.  The tolerance is
# 2^-11 of the largest entry, and the kernels must sit at least 4x closer to the model than to
# the exact backward, so that a rounding left out, added or placed elsewhere shows.
MODEL_TOL = 2.0 ** -11
MODEL_CASES = [
    # B, Sq, Skv, Hq, Hkv, positions
    (1, 256, 256, 2, 2, "causal"),
    (2, 200, 333, 4, 2, "causal"),
    (1, 130, 70, 8, 1, "causal"),
    (1, 128, 128, 4, 2, "zigzag"),
    (1, 150, 260, 4, 2, "sparse"),
]


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("case", MODEL_CASES)
def test_block_bwd_bf16_matches_rounding_model(case, D):
    B, Sq, Skv, Hq, Hkv, kind = case
    if kind == "causal":
        qpos = np.arange(Skv - Sq, Skv, dtype=np.int64) if Skv >= Sq else np.arange(Sq, dtype=np.int64)
        kvpos = np.arange(Skv, dtype=np.int64)
    elif kind == "zigzag":
        qpos = oracle.zigzag_positions(4 * 64 * 2, 4, 3)[:Sq]
        kvpos = oracle.zigzag_positions(4 * 64 * 2, 4, 1)[:Skv]
    else:
        rng = np.random.default_rng(4)
        qpos = np.sort(rng.choice(5000, Sq, replace=False)).astype(np.int64)
        kvpos = np.sort(rng.choice(np.arange(1000, 6000), Skv, replace=False)).astype(np.int64)
    got, exact, args = _block_case(50, B, Sq, Skv, Hq, Hkv, D, "bf16", qpos, kvpos)
    q, k, v, g = (x.float().cpu().numpy() for x in args[:4])
    out, lse = oracle.attention_rows(q, k, v, qpos, kvpos, args[6])
    model = oracle.block_bwd(q, k, v, g, out, lse, qpos, kvpos, args[6], bf16_pds=True)
    for name, x, m, e in zip(("dq", "dk", "dv"), got, model, exact):
        x = x.cpu().numpy()
        big = max(float(np.max(np.abs(m))), 1e-2)
        err_m, err_e = max_abs(x, m), max_abs(x, e)
        print(f"{kind} D={D} {case[:5]} {name}: vs model {err_m / big:.3g}, vs exact {err_e / big:.3g} "
              f"of the largest entry")
        assert err_m <= MODEL_TOL * big, f"{name}: {err_m:.3g} > {MODEL_TOL * big:.3g}"
        assert err_e >= 4 * err_m, f"{name}: not closer to the rounding model ({err_m:.3g}, {err_e:.3g})"


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 128), ("bf16", 64)])
@pytest.mark.parametrize("C,t", [(4, 64), (2, 100)])
def test_block_bwd_every_zigzag_step_class(C, t, dtype, D):
    S = 2 * C * t
    for r in (0, C - 1):
        qpos = oracle.zigzag_positions(S, C, r)
        for o in range(C):
            kvpos = oracle.zigzag_positions(S, C, o)
            got, ref, _ = _block_case(20 + o, 1, 2 * t, 2 * t, 4, 2, D, dtype, qpos, kvpos)
            for name, x, rr in zip(("dq", "dk", "dv"), got, ref):
                _check(f"r{r} o{o} {name}", x, rr, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_block_bwd_sparse_positions_and_empty_rows(dtype):
    rng = np.random.default_rng(4)
    qpos = np.sort(rng.choice(5000, 150, replace=False)).astype(np.int64)
    kvpos = np.sort(rng.choice(np.arange(1000, 6000), 260, replace=False)).astype(np.int64)
    got, ref, _ = _block_case(30, 1, 150, 260, 4, 2, 128, dtype, qpos, kvpos)
    empty = kvpos[0] > qpos
    assert empty.any()
    assert torch.count_nonzero(got[0][:, torch.from_numpy(empty).to(DEV)]) == 0
    for name, x, r in zip(("dq", "dk", "dv"), got, ref):
        _check(name, x, r, dtype)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp32", 64), ("bf16", 64)])
def test_head_dim_and_accumulate_flag(dtype, D):
    pos = np.arange(96, dtype=np.int64)
    got, ref, args = _block_case(40, 1, 96, 96, 2, 1, D, dtype, pos, pos)
    # a second call without flags adds the same part again: exactly twice the first result
    first = [x.clone() for x in got]
    cp.block_bwd(*args, *got, 0)
    torch.cuda.synchronize()
    for a, b2 in zip(first, got):
        assert torch.equal(b2, 2 * a)
    for name, x, r in zip(("dq", "dk", "dv"), first, ref):
        _check(name, x, r, dtype)


def test_no_keys_with_write_flags_gives_zeros():
    q = _rand(1, (1, 40, 2, 128), "bf16").to(DEV)
    k = torch.empty((1, 0, 2, 128), dtype=torch.bfloat16, device=DEV)
    pos = torch.arange(40, device=DEV)
    lse = torch.full((1, 2, 40), -math.inf, device=DEV)
    delta = torch.zeros((1, 2, 40), device=DEV)
    dq = torch.full((1, 40, 2, 128), 3.0, device=DEV)
    dk = torch.empty((1, 0, 2, 128), device=DEV)
    cp.block_bwd(q, k, k, q, pos, pos[:0], 0.1, lse, delta, dq, dk, dk.clone(), cp.BWD_WRITE_DQ)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dq) == 0


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_delta_matches_oracle(dtype):
    out = _rand(50, (2, 77, 3, 128), "fp32")
    g = _rand(51, (2, 77, 3, 128), dtype)
    got = cp.attn_bwd_delta(out.to(DEV), g.to(DEV)).cpu().numpy()
    ref = np.einsum("bshd,bshd->bhs", out.double().numpy(), g.double().numpy())
    assert max_abs(got, ref) <= 1e-5 * max(1.0, float(np.abs(ref).max()))


def _synthetic_saved(w, qf, kf, zz):
    """Saved forward state for a full-size check: out is seeded N(0,1) and lse an upper bound
    of each row's log-sum-exp (scale*|q_i|*max_j|k_j| + ln(visible keys)), so every weight
    p = exp(s - lse) stays below 1.  The block backward is a function of these inputs whatever
    their origin, and the oracle evaluates the same function."""
    B, s, H, D = qf.shape
    out = torch.randn((B, s, H, D), generator=torch.Generator().manual_seed(77)).numpy()
    kmax = float(np.sqrt((kf.astype(np.float64) ** 2).sum(-1)).max())
    qn = np.sqrt((qf.astype(np.float64) ** 2).sum(-1))  # [B, s, H]
    lse = (w.scale * qn * kmax + np.log(zz + 1.0)[None, :, None]).transpose(0, 2, 1)
    return out.astype(np.float32), np.ascontiguousarray(lse.astype(np.float32))


def _ring_bwd_check(w, rows_per_chunk, key_samples, exact_forward):
    C, r = w.cp_size, w.rank
    S = w.seq_len
    pos = [cp.zigzag_index(S, C, o, device=DEV) for o in range(C)]
    ks = [gen(w, "k", zigzag_chunks(C, o), w.heads_kv).to(DEV) for o in range(C)]
    vs = [gen(w, "v", zigzag_chunks(C, o), w.heads_kv).to(DEV) for o in range(C)]
    q = gen(w, "q", zigzag_chunks(C, r), w.heads_q)
    g = gen(w, "dout", zigzag_chunks(C, r), w.heads_q)
    ids = range(2 * C)
    kf, vf = gen(w, "k", ids, w.heads_kv).float().numpy(), gen(w, "v", ids, w.heads_kv).float().numpy()
    zz = oracle.zigzag_positions(S, C, r)
    gpos = np.arange(S, dtype=np.int64)
    qf, gf = q.float().numpy(), g.float().numpy()
    if exact_forward:  # the complete forward of every local row, from the oracle
        out, lse = oracle.attention_rows(qf, kf, vf, zz, gpos, w.scale)
    else:
        out, lse = _synthetic_saved(w, qf, kf, zz)
    print(f"{w.name}: saved forward state ready", flush=True)
    o_t = torch.from_numpy(np.ascontiguousarray(out, dtype=np.float32)).to(DEV)
    l_t = torch.from_numpy(np.ascontiguousarray(lse, dtype=np.float32)).to(DEV)
    dq, dks, dvs = cp.ring_share_bwd(q.to(DEV), ks, vs, pos, r, w.scale, o_t, l_t, g.to(DEV))
    torch.cuda.synchronize()
    print(f"{w.name}: HIP ring backward done", flush=True)
    del ks, vs
    qrows = sample_rows(w.local_len, w.chunk_len, seed=r, per_chunk_random=rows_per_chunk)
    ref_dq, _, _ = oracle.block_bwd(qf, kf, vf, gf, out, lse, zz, gpos, w.scale, qrows=qrows,
                                    krows=np.zeros(0, dtype=np.int64))
    _check("dq", dq[:, torch.from_numpy(qrows).to(DEV)], ref_dq, w.dtype)
    print(f"{w.name}: dq checked on {len(qrows)} rows", flush=True)
    rng = np.random.default_rng(9)
    for o in range(C):
        kz = oracle.zigzag_positions(S, C, o)
        krows = np.unique(np.concatenate([[0, w.chunk_len - 1, w.chunk_len, 2 * w.chunk_len - 1],
                                          rng.integers(0, 2 * w.chunk_len, key_samples)])).astype(np.int64)
        _, rdk, rdv = oracle.block_bwd(qf, kf[:, kz], vf[:, kz], gf, out, lse, zz, kz, w.scale,
                                       qrows=np.zeros(0, dtype=np.int64), krows=krows)
        kidx = torch.from_numpy(krows).to(DEV)
        _check(f"dk owner {o}", dks[o][:, kidx], rdk, w.dtype)
        _check(f"dv owner {o}", dvs[o][:, kidx], rdv, w.dtype)
        print(f"{w.name}: owner {o} dk, dv checked on {len(krows)} keys", flush=True)


@pytest.mark.parametrize("dtype,C,t,Hq,Hkv,D,B,rank", [
    ("bf16", 4, 100, 4, 2, 128, 1, 1),   # ragged tiles, GQA
    ("bf16", 3, 70, 8, 8, 64, 2, 2),     # head dim 64, batch 2, the last rank
    ("bf16", 8, 256, 32, 8, 128, 1, 3),  # whole tiles, the long share's head layout
    ("fp32", 2, 33, 4, 2, 64, 1, 0),
    # 16384 local rows: the dq launches (4096 blocks) and the one dk/dv launch (4096 blocks)
    # take their work from queues across the XCDs, the per-step dk/dv launches (1024 blocks)
    # do not, so this also pins the queue order's bits to the static order's
    ("bf16", 4, 8192, 32, 8, 128, 1, 3),
])
def test_ring_share_bwd_single_equals_steps(dtype, C, t, Hq, Hkv, D, B, rank):
    """The share's backward in one call (cpattn_ring_share_bwd: dq per step, dk and dv of all
    blocks in one launch) gives the same bits as one cpattn_block_bwd per ring step."""
    S = 2 * C * t
    pos = [cp.zigzag_index(S, C, o, device=DEV) for o in range(C)]
    ks = [_rand(300 + o, (B, 2 * t, Hkv, D), dtype).to(DEV) for o in range(C)]
    vs = [_rand(400 + o, (B, 2 * t, Hkv, D), dtype).to(DEV) for o in range(C)]
    q, g = _rand(1, (B, 2 * t, Hq, D), dtype).to(DEV), _rand(2, (B, 2 * t, Hq, D), dtype).to(DEV)
    scale = 1 / math.sqrt(D)
    out, lse = cp.ring_share_fwd(q, ks, vs, pos, rank, scale)
    res = {}
    for mode in ("single", "steps"):
        dq = torch.full((B, 2 * t, Hq, D), 7.0, device=DEV)  # every buffer is overwritten
        dks = [torch.full(k.shape, 7.0, device=DEV) for k in ks]
        dvs = [torch.full(v.shape, 7.0, device=DEV) for v in vs]
        res[mode] = cp.ring_share_bwd(q, ks, vs, pos, rank, scale, out, lse, g, dq=dq, dk_blocks=dks,
                                      dv_blocks=dvs, mode=mode)
    torch.cuda.synchronize()
    a, b = res["single"], res["steps"]
    assert torch.equal(a[0], b[0])
    for o in range(C):
        assert torch.equal(a[1][o], b[1][o]) and torch.equal(a[2][o], b[2][o]), o


@pytest.mark.parametrize("lens", [[500, 0, 130, 257], [64 + 37 * o for o in range(16)]])
def test_ring_blocks_bwd_unequal_and_empty_blocks(lens):
    """Blocks of different lengths (the dk/dv launch is sized by the longest; shorter blocks'
    missing key blocks do nothing), a block without keys, and the most blocks one call takes
    (16), against per-block calls."""
    B, Sq, Hq, Hkv, D = 1, 300, 4, 2, 128
    qpos = torch.arange(600, 600 + Sq, device=DEV)
    kpos = [torch.sort(torch.randperm(900, generator=torch.Generator().manual_seed(o))[:n]).values.to(DEV)
            for o, n in enumerate(lens)]
    ks = [_rand(500 + o, (B, n, Hkv, D), "bf16").to(DEV) for o, n in enumerate(lens)]
    vs = [_rand(600 + o, (B, n, Hkv, D), "bf16").to(DEV) for o, n in enumerate(lens)]
    q, g = _rand(3, (B, Sq, Hq, D), "bf16").to(DEV), _rand(4, (B, Sq, Hq, D), "bf16").to(DEV)
    scale = 1 / math.sqrt(D)
    out, lse = cp.ring_blocks_fwd(q, ks, vs, kpos, qpos, scale)
    delta = cp.attn_bwd_delta(out, g)
    dq = torch.full((B, Sq, Hq, D), 7.0, device=DEV)
    dks = [torch.full(k.shape, 7.0, device=DEV) for k in ks]
    dvs = [torch.full(v.shape, 7.0, device=DEV) for v in vs]
    cp.ring_blocks_bwd(q, g, ks, vs, kpos, qpos, scale, lse, delta, dq, dks, dvs)
    rq = torch.empty_like(dq)
    rk = [torch.empty_like(x) for x in dks]
    rv = [torch.empty_like(x) for x in dvs]
    for o in range(len(lens)):
        cp.block_bwd(q, ks[o], vs[o], g, qpos, kpos[o], scale, lse, delta, rq, rk[o], rv[o],
                     cp.BWD_WRITE_DKV | (cp.BWD_WRITE_DQ if o == 0 else 0))
    torch.cuda.synchronize()
    assert torch.equal(dq, rq)
    for o in range(len(lens)):
        assert torch.equal(dks[o], rk[o]) and torch.equal(dvs[o], rv[o]), o


def test_ring_share_bwd_8k():
    _ring_bwd_check(WORKLOADS["rank_share_8k"], rows_per_chunk=12, key_samples=12, exact_forward=True)


def test_ring_share_bwd_head_dim_64():
    """The ring-share backward through the binding with bf16 and head dim 64: a zigzag rank's
    share (S = 2048, C = 4, rank 1, 8 query / 2 K/V heads), every step's block backward."""
    w = Workload("ring_bwd_d64", "ring_share", 1, 2048, 8, 2, 64, "bf16", 4, rank=1)
    _ring_bwd_check(w, rows_per_chunk=12, key_samples=12, exact_forward=True)


def test_ring_share_bwd_256k_sampled():
    _ring_bwd_check(WORKLOADS["ring_share_256k"], rows_per_chunk=2, key_samples=4, exact_forward=False)


@pytest.mark.parametrize("B,S,Hq,Hkv,D", [(1, 9000, 32, 8, 128), (2, 5000, 16, 8, 128), (1, 9000, 32, 8, 64)])
def test_block_bwd_launch_size_sampled(B, S, Hq, Hkv, D):
    """Causal self-attention backward at launch size (the 4-wave dq kernel, at least 512
    blocks; ragged last tiles), from a synthetic saved state (seeded out; an upper bound of
    each row's lse, so every weight stays below 1).  Sampled dq rows and dk, dv keys against
    the oracle."""
    scale = 1 / math.sqrt(D)
    q, k, v, g = (_rand(S + i, s, "bf16") for i, s in
                  enumerate(((B, S, Hq, D), (B, S, Hkv, D), (B, S, Hkv, D), (B, S, Hq, D))))
    qf, kf, vf, gf = (x.float().numpy() for x in (q, k, v, g))
    pos = np.arange(S, dtype=np.int64)
    out = torch.randn((B, S, Hq, D), generator=torch.Generator().manual_seed(78)).numpy().astype(np.float32)
    kmax = float(np.sqrt((kf.astype(np.float64) ** 2).sum(-1)).max())
    qn = np.sqrt((qf.astype(np.float64) ** 2).sum(-1))  # [B, S, Hq]
    lse = np.ascontiguousarray((scale * qn * kmax + np.log(pos + 1.0)[None, :, None]).transpose(0, 2, 1),
                               dtype=np.float32)
    tp = torch.from_numpy(pos).to(DEV)
    o_t, l_t = torch.from_numpy(out).to(DEV), torch.from_numpy(lse).to(DEV)
    gd = g.to(DEV)
    delta = cp.attn_bwd_delta(o_t, gd)
    dq = torch.empty((B, S, Hq, D), device=DEV)
    dk = torch.empty((B, S, Hkv, D), device=DEV)
    dv = torch.empty((B, S, Hkv, D), device=DEV)
    cp.block_bwd(q.to(DEV), k.to(DEV), v.to(DEV), gd, tp, tp, scale, l_t, delta, dq, dk, dv,
                 cp.BWD_WRITE_DQ | cp.BWD_WRITE_DKV)
    torch.cuda.synchronize()
    rng = np.random.default_rng(S)
    edges = [0, 1, 31, 32, 63, 64, 127, 128, S - 65, S - 64, S - 33, S - 2, S - 1]
    rows = np.unique(np.concatenate([edges, rng.integers(0, S, 12)])).astype(np.int64)
    ref_dq, _, _ = oracle.block_bwd(qf, kf, vf, gf, out, lse, pos, pos, scale, qrows=rows,
                                    krows=np.zeros(0, dtype=np.int64))
    _check("dq", dq[:, torch.from_numpy(rows).to(DEV)], ref_dq, "bf16")
    _, rdk, rdv = oracle.block_bwd(qf, kf, vf, gf, out, lse, pos, pos, scale,
                                   qrows=np.zeros(0, dtype=np.int64), krows=rows)
    kidx = torch.from_numpy(rows).to(DEV)
    _check("dk", dk[:, kidx], rdk, "bf16")
    _check("dv", dv[:, kidx], rdv, "bf16")


@pytest.mark.parametrize("seed", range(10))
def test_block_bwd_random_shapes(seed):
    """Seeded random small shapes (batch 1-2, K/V heads 1-4, head ratios 1-4, causal or sparse
    increasing positions, ragged sizes), both dtypes: every dq, dk, dv entry against the
    oracle, from the oracle's own forward."""
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 3))
    hkv = int(rng.choice([1, 2, 4]))
    hq = hkv * int(rng.choice([1, 2, 3, 4]))
    sq, skv = int(rng.integers(1, 260)), int(rng.integers(1, 330))
    if rng.integers(0, 2):
        qpos = np.sort(rng.choice(3 * (sq + skv), sq, replace=False)).astype(np.int64)
        kvpos = np.sort(rng.choice(3 * (sq + skv), skv, replace=False)).astype(np.int64)
    else:
        n = max(sq, skv)
        kvpos = np.arange(n - skv, n, dtype=np.int64)
        qpos = np.arange(n - sq, n, dtype=np.int64)
    for dtype in ("bf16", "fp32"):
        got, ref, _ = _block_case(200 + seed, B, sq, skv, hq, hkv, 128, dtype, qpos, kvpos)
        for name, x, r in zip(("dq", "dk", "dv"), got, ref):
            _check(f"seed {seed} {dtype} B={B} Sq={sq} Skv={skv} Hq={hq} Hkv={hkv} {name}", x, r, dtype)

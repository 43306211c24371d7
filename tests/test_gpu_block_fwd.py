"""HIP block attention against the oracle element by element, on small seeded cases that
span several tiles with ragged tails: both dtypes, grouped-query ratios, batch > 1, every
zigzag step class (diagonal / entirely visible / entirely hidden), sparse positions, empty
rows and empty key sets."""
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


def _inputs(seed, B, Sq, Skv, Hq, Hkv, D, dtype):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((B, Sq, Hq, D), generator=g).to(dtype)
    k = torch.randn((B, Skv, Hkv, D), generator=g).to(dtype)
    v = torch.randn((B, Skv, Hkv, D), generator=g).to(dtype)
    return q, k, v


def _run_and_compare(q, k, v, qpos, kvpos, scale, dtype_name):
    out, lse = cp.block_fwd(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(qpos).to(DEV),
                            torch.from_numpy(kvpos).to(DEV), scale)
    ref_o, ref_l = oracle.attention_rows(q.float().numpy(), k.float().numpy(), v.float().numpy(), qpos,
                                         kvpos, scale)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    tol_o, tol_l = TOL[dtype_name]
    eo, el = max_abs(o, ref_o), max_abs(l, ref_l)
    assert eo <= tol_o and el <= tol_l, f"max abs err O {eo:.3g} lse {el:.3g}"
    # rows with no visible key: exactly (0, -inf)
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(l), empty)
    assert np.all(o.transpose(0, 2, 1, 3)[empty] == 0.0)
    return eo, el


CASES = [
    # B, Sq, Skv, Hq, Hkv, D
    (1, 256, 256, 2, 2, 128),
    (2, 200, 333, 4, 2, 128),
    (1, 130, 70, 8, 1, 128),
    (1, 97, 300, 6, 2, 128),    # ratio 3: one query head per block row group
    (1, 64, 128, 16, 2, 128),   # ratio 8: two head groups per K/V head
    (1, 1, 1, 1, 1, 128),
    (3, 45, 513, 4, 4, 128),
]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("case", CASES)
def test_causal_contiguous(case, dtype):
    B, Sq, Skv, Hq, Hkv, D = case
    q, k, v = _inputs(hash(case) % 1000, B, Sq, Skv, Hq, Hkv, D, torch.bfloat16 if dtype == "bf16" else torch.float32)
    # queries are the last Sq positions of a Skv-long sequence (a prefix-cache shape)
    kvpos = np.arange(Skv, dtype=np.int64)
    qpos = np.arange(Skv - Sq, Skv, dtype=np.int64) if Sq <= Skv else np.arange(Sq, dtype=np.int64)
    _run_and_compare(q, k, v, qpos, kvpos, 1.0 / math.sqrt(D), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("C,t", [(4, 96), (8, 40), (2, 200)])
def test_zigzag_every_step_class(C, t, dtype):
    """Rank r's local queries against every owner's shard: owner == r (diagonal chunks),
    owner < r (early chunk fully visible), owner > r (early queries see nothing)."""
    S = 2 * C * t
    Hq, Hkv, D = 4, 2, 128
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, _, _ = _inputs(C * t, 1, S // C, 1, Hq, Hkv, D, td)
    for r in (0, C // 2, C - 1):
        for o in range(C):
            _, k, v = _inputs(1000 * o + r, 1, 1, S // C, Hq, Hkv, D, td)
            _run_and_compare(q, k, v, oracle.zigzag_positions(S, C, r), oracle.zigzag_positions(S, C, o),
                             0.088, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_sparse_positions_and_empty_rows(dtype):
    rng = np.random.default_rng(5)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    for trial in range(4):
        Sq, Skv = int(rng.integers(1, 300)), int(rng.integers(1, 400))
        qpos = np.sort(rng.choice(5000, Sq, replace=False)).astype(np.int64)
        kvpos = np.sort(rng.choice(5000, Skv, replace=False)).astype(np.int64)
        q, k, v = _inputs(trial, 2, Sq, Skv, 8, 2, 128, td)
        _run_and_compare(q, k, v, qpos, kvpos, 0.1, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_all_hidden_and_no_keys(dtype):
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = _inputs(9, 1, 100, 150, 4, 4, 128, td)
    # every key later than every query: all rows empty
    _run_and_compare(q, k, v, np.arange(100, dtype=np.int64), np.arange(1000, 1150, dtype=np.int64), 0.1, dtype)
    # no keys at all
    out, lse = cp.block_fwd(q.to(DEV), k[:, :0].contiguous().to(DEV), v[:, :0].contiguous().to(DEV),
                            torch.arange(100, device=DEV), torch.zeros(0, dtype=torch.int64, device=DEV), 0.1)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_fp32_head_dim_64():
    q, k, v = _inputs(11, 2, 150, 150, 2, 1, 64, torch.float32)
    pos = np.arange(150, dtype=np.int64)
    _run_and_compare(q, k, v, pos, pos, 0.125, "fp32")


def test_repeat_calls_are_identical():
    """Same inputs, same outputs bit for bit (no dependence on scheduling)."""
    q, k, v = _inputs(12, 1, 512, 512, 8, 2, 128, torch.bfloat16)
    pos = torch.arange(512, device=DEV)
    a = cp.block_fwd(q.to(DEV), k.to(DEV), v.to(DEV), pos, pos, 0.09)
    b = cp.block_fwd(q.to(DEV), k.to(DEV), v.to(DEV), pos, pos, 0.09)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def _rows(n: int, seed: int, extra: int = 24) -> np.ndarray:
    """Rows to compare at launch sizes: both ends, rows around the 64- and 96-row block edges
    at both ends, and seeded random rows."""
    rng = np.random.default_rng(seed)
    rows = {0, 1, 31, 32, 63, 64, 95, 96, 127, n - 97, n - 96, n - 65, n - 64, n - 33, n - 32, n - 2, n - 1}
    rows.update(rng.integers(0, n, extra).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < n), dtype=np.int64)


def _check_rows(out, lse, rows, ref_o, ref_l, what):
    o = out[:, rows].cpu().numpy()
    lv = lse[:, :, rows].cpu().numpy()
    tol_o, tol_l = TOL["bf16"]
    eo, el = max_abs(o, ref_o), max_abs(lv, ref_l)
    assert eo <= tol_o and el <= tol_l, f"{what}: max abs err O {eo:.3g} lse {el:.3g}"


# launches of at least 512 eight-wave blocks (the 8- and 12-wave kernels), ragged last
# blocks, grouped-query ratios 4, 2 and 3: (B, S, Hq, Hkv)
LARGE = [(1, 6000, 32, 8), (2, 4100, 32, 8), (1, 9000, 16, 8), (1, 11000, 12, 4)]


@pytest.mark.parametrize("case", LARGE)
def test_large_causal_launches(case):
    """Causal self-attention at launch sizes: with one positions tensor for queries and keys
    (the 12-wave kernel) and with the same positions in a second tensor (the 8-wave kernel);
    sampled rows against the oracle."""
    B, S, Hq, Hkv = case
    D = 128
    scale = 1 / math.sqrt(D)
    q, k, v = _inputs(S % 997, B, S, S, Hq, Hkv, D, torch.bfloat16)
    pos = np.arange(S, dtype=np.int64)
    rows = _rows(S, S)
    ref_o, ref_l = oracle.attention_rows(q.float().numpy(), k.float().numpy(), v.float().numpy(), pos, pos,
                                         scale, rows=rows)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    tp = torch.from_numpy(pos).to(DEV)
    for name, kvp in (("shared positions", tp), ("separate positions", tp.clone())):
        out, lse = cp.block_fwd(qd, kd, vd, tp, kvp, scale)
        torch.cuda.synchronize()
        _check_rows(out, lse, rows, ref_o, ref_l, name)


def test_large_zigzag_steps_and_share():
    """A zigzag rank's queries at launch size (C = 4, t = 3000: 6000 local rows, 32/8 heads)
    against an earlier, its own and a later owner's keys, one launch per step, and the whole
    share in one launch; sampled rows against the oracle."""
    C, t, Hq, Hkv, D = 4, 3000, 32, 8, 128
    S, r = 2 * C * t, 1
    scale = 1 / math.sqrt(D)
    q_full, k_full, v_full = _inputs(77, 1, S, S, Hq, Hkv, D, torch.bfloat16)
    pos = [oracle.zigzag_positions(S, C, o) for o in range(C)]
    tpos = [torch.from_numpy(p).to(DEV) for p in pos]
    q = q_full[:, pos[r]].contiguous().to(DEV)
    ks = [k_full[:, p].contiguous().to(DEV) for p in pos]
    vs = [v_full[:, p].contiguous().to(DEV) for p in pos]
    rows = _rows(2 * t, 5)
    qf, kf, vf = q_full.float().numpy(), k_full.float().numpy(), v_full.float().numpy()
    for o in (0, r, C - 1):
        ref_o, ref_l = oracle.attention_rows(qf[:, pos[r]], kf[:, pos[o]], vf[:, pos[o]], pos[r], pos[o], scale,
                                             rows=rows)
        out, lse = cp.block_fwd(q, ks[o], vs[o], tpos[r], tpos[o], scale)
        torch.cuda.synchronize()
        _check_rows(out, lse, rows, ref_o, ref_l, f"owner {o}")
    gpos = np.arange(S, dtype=np.int64)
    ref_o, ref_l = oracle.attention_rows(qf, kf, vf, gpos, gpos, scale, rows=pos[r][rows])
    out, lse = cp.ring_share_fwd(q, ks, vs, tpos, r, scale)
    torch.cuda.synchronize()
    _check_rows(out, lse, rows, ref_o, ref_l, "one-launch share")


def _random_case(seed: int):
    """A seeded shape: batch, sizes, head ratio, positions (contiguous causal, a shared
    positions tensor, or sparse increasing sets), small or at launch size."""
    rng = np.random.default_rng(seed)
    hkv = int(rng.choice([1, 2, 4, 8]))
    ratio = int(rng.choice([1, 2, 3, 4, 8]))
    hq = hkv * ratio
    B = int(rng.integers(1, 3))
    large = bool(rng.integers(0, 2))
    # at launch size the 8-wave blocks (256/G positions of G query heads) number >= 512
    G = 4 if ratio % 4 == 0 else (2 if ratio % 2 == 0 else 1)
    cols = B * hkv * (ratio // G)
    if large:
        sq = max(1, -(-520 // cols) * (256 // G) + int(rng.integers(-90, 90)))
    else:
        sq = int(rng.integers(1, 700))
    kind = str(rng.choice(["shared", "causal", "sparse"]))
    if kind == "sparse":
        skv = int(rng.integers(1, 2 * sq + 2))
        qpos = np.sort(rng.choice(4 * (sq + skv), sq, replace=False)).astype(np.int64)
        kvpos = np.sort(rng.choice(4 * (sq + skv), skv, replace=False)).astype(np.int64)
    else:
        skv = sq if kind == "shared" else sq + int(rng.integers(0, 300))
        kvpos = np.arange(skv, dtype=np.int64)
        qpos = kvpos[skv - sq:].copy()
    return B, sq, skv, hq, hkv, kind, qpos, kvpos


@pytest.mark.parametrize("seed", range(16))
def test_random_shapes_sampled(seed):
    """Seeded random shapes through whichever kernel the launcher picks; sampled rows (every
    row when small) against the oracle, and empty rows exactly (0, -inf)."""
    B, sq, skv, hq, hkv, kind, qpos, kvpos = _random_case(seed)
    D, scale = 128, 1 / math.sqrt(128)
    q, k, v = _inputs(7000 + seed, B, sq, skv, hq, hkv, D, torch.bfloat16)
    rows = _rows(sq, seed) if sq > 700 else np.arange(sq, dtype=np.int64)
    ref_o, ref_l = oracle.attention_rows(q.float().numpy(), k.float().numpy(), v.float().numpy(), qpos, kvpos,
                                         scale, rows=rows)
    tq = torch.from_numpy(qpos).to(DEV)
    tk = tq if kind == "shared" else torch.from_numpy(kvpos).to(DEV)
    out, lse = cp.block_fwd(q.to(DEV), k.to(DEV), v.to(DEV), tq, tk, scale)
    torch.cuda.synchronize()
    _check_rows(out, lse, rows, ref_o, ref_l, f"seed {seed}: B={B} Sq={sq} Skv={skv} Hq={hq} Hkv={hkv} {kind}")
    lv = lse[:, :, rows].cpu().numpy()
    empty = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(lv), empty)
    assert np.all(out[:, rows].cpu().numpy().transpose(0, 2, 1, 3)[empty] == 0.0)


@pytest.mark.parametrize("S,Hq,Hkv,shared", [(6000, 32, 8, True), (6000, 32, 8, False), (300, 8, 2, True),
                                             (777, 4, 4, False)])
def test_block_fwd_rows_equals_dense(S, Hq, Hkv, shared):
    """cpattn_block_fwd_rows on one head group of wider rows (q, k, v read in place; out written
    into a wider buffer) gives the bits of cpattn_block_fwd on dense copies, and leaves the
    other heads of out untouched."""
    D, scale = 128, 1 / math.sqrt(128)
    q_all, k_all, v_all = _inputs(S + Hq, 1, S, S, 2 * Hq, 2 * Hkv, D, torch.bfloat16)
    q_all, k_all, v_all = (x[0].to(DEV) for x in (q_all, k_all, v_all))
    qv, kv, vv = q_all[:, Hq:], k_all[:, Hkv:], v_all[:, Hkv:]
    out_all = torch.full((S, 2 * Hq, D), 7.0, device=DEV)
    ov = out_all[:, Hq:]
    tp = torch.arange(S, device=DEV)
    tk = tp if shared else tp.clone()
    _, lse = cp.block_fwd_rows(qv, kv, vv, tp, tk, scale, ov)
    ref_o, ref_l = cp.block_fwd(qv.contiguous()[None], kv.contiguous()[None], vv.contiguous()[None], tp, tk, scale)
    torch.cuda.synchronize()
    assert torch.equal(ov, ref_o[0]) and torch.equal(lse, ref_l)
    assert bool((out_all[:, :Hq] == 7.0).all())


def test_block_fwd_rows_no_keys():
    q = _inputs(3, 1, 50, 1, 8, 2, 128, torch.bfloat16)[0][0].to(DEV)
    out = torch.full((50, 16, 128), 5.0, device=DEV)
    _, lse = cp.block_fwd_rows(q[:, :], torch.empty((0, 2, 128), dtype=torch.bfloat16, device=DEV),
                               torch.empty((0, 2, 128), dtype=torch.bfloat16, device=DEV),
                               torch.arange(50, device=DEV), torch.zeros(0, dtype=torch.int64, device=DEV), 0.1,
                               out[:, 8:])
    torch.cuda.synchronize()
    assert torch.count_nonzero(out[:, 8:]) == 0 and bool((out[:, :8] == 5.0).all())
    assert bool(torch.isneginf(lse).all())


# bf16 with head dim 64: the same kernels instantiated for 128-byte rows (their own LDS
# swizzles), small launches (keys split over two wave groups) and launch sizes (the
# software-pipelined kernel)
@pytest.mark.parametrize("case", [(1, 256, 256, 2, 2), (2, 200, 333, 4, 2), (1, 97, 300, 6, 2), (3, 45, 513, 8, 4)])
def test_bf16_head_dim_64_small(case):
    B, Sq, Skv, Hq, Hkv = case
    q, k, v = _inputs(64 + Sq, B, Sq, Skv, Hq, Hkv, 64, torch.bfloat16)
    kvpos = np.arange(Skv, dtype=np.int64)
    qpos = np.arange(Skv - Sq, Skv, dtype=np.int64) if Sq <= Skv else np.arange(Sq, dtype=np.int64)
    _run_and_compare(q, k, v, qpos, kvpos, 0.125, "bf16")


def test_bf16_head_dim_64_zigzag_steps():
    C, t, Hq, Hkv = 4, 96, 4, 2
    S = 2 * C * t
    q, _, _ = _inputs(640, 1, S // C, 1, Hq, Hkv, 64, torch.bfloat16)
    for r in (0, C - 1):
        for o in range(C):
            _, k, v = _inputs(650 + o, 1, 1, S // C, Hq, Hkv, 64, torch.bfloat16)
            _run_and_compare(q, k, v, oracle.zigzag_positions(S, C, r), oracle.zigzag_positions(S, C, o), 0.125,
                             "bf16")


@pytest.mark.parametrize("case", [(1, 6000, 32, 8), (2, 4100, 16, 4)])
def test_bf16_head_dim_64_large(case):
    B, S, Hq, Hkv = case
    D = 64
    scale = 1 / math.sqrt(D)
    q, k, v = _inputs(S % 991, B, S, S, Hq, Hkv, D, torch.bfloat16)
    pos = np.arange(S, dtype=np.int64)
    rows = _rows(S, S + 1)
    ref_o, ref_l = oracle.attention_rows(q.float().numpy(), k.float().numpy(), v.float().numpy(), pos, pos,
                                         scale, rows=rows)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    tp = torch.from_numpy(pos).to(DEV)
    for name, kvp in (("shared positions", tp), ("separate positions", tp.clone())):
        out, lse = cp.block_fwd(qd, kd, vd, tp, kvp, scale)
        torch.cuda.synchronize()
        _check_rows(out, lse, rows, ref_o, ref_l, name)


def test_bf16_head_dim_64_ring_share():
    """A zigzag rank's whole share in one launch at D = 64, sampled rows against the oracle."""
    C, t, Hq, Hkv, D = 4, 1500, 16, 4, 64
    S, r = 2 * C * t, 2
    scale = 1 / math.sqrt(D)
    q_full, k_full, v_full = _inputs(78, 1, S, S, Hq, Hkv, D, torch.bfloat16)
    pos = [oracle.zigzag_positions(S, C, o) for o in range(C)]
    tpos = [torch.from_numpy(p).to(DEV) for p in pos]
    q = q_full[:, pos[r]].contiguous().to(DEV)
    ks = [k_full[:, p].contiguous().to(DEV) for p in pos]
    vs = [v_full[:, p].contiguous().to(DEV) for p in pos]
    rows = _rows(2 * t, 6)
    gpos = np.arange(S, dtype=np.int64)
    ref_o, ref_l = oracle.attention_rows(q_full.float().numpy(), k_full.float().numpy(), v_full.float().numpy(),
                                         gpos, gpos, scale, rows=pos[r][rows])
    for mode in ("single", "fused"):
        out, lse = cp.ring_share_fwd(q, ks, vs, tpos, r, scale, mode=mode)
        torch.cuda.synchronize()
        _check_rows(out, lse, rows, ref_o, ref_l, f"D=64 share ({mode})")

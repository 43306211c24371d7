"""Pins for the oracle's attention backward: automatic differentiation of the forward
definition (torch fp64 on the CPU, an independent derivation of the same derivative), central
finite differences, the ring decomposition (blocks add up to the whole gradient), and the
contribution pattern the pages print for rank 1 at C = 4."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from conftest import read_golden


def _inputs(seed, B, S, Hq, Hkv, D, dyadic=False):
    rng = np.random.default_rng(seed)
    shapes = [(B, S, Hq, D), (B, S, Hkv, D), (B, S, Hkv, D), (B, S, Hq, D)]
    xs = [rng.standard_normal(s) for s in shapes]
    if dyadic:  # few mantissa bits: exact in fp32, so perturbations by 2^-12 are exact too
        xs = [np.round(x * 64) / 64 for x in xs]
    return [x.astype(np.float32) for x in xs]


def _autograd(q, k, v, dout, q_pos, kv_pos, scale):
    """Gradients of L = sum(out * dout) for causal attention written with torch ops."""
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    G = q.shape[2] // k.shape[2]
    kk = tk.repeat_interleave(G, dim=2)
    vv = tv.repeat_interleave(G, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", tq, kk) * scale
    vis = torch.tensor(kv_pos[None, :] <= q_pos[:, None])
    s = s.masked_fill(~vis, float("-inf"))
    p = torch.softmax(s, dim=-1)
    out = torch.einsum("bhij,bjhd->bihd", p, vv)
    (out * torch.tensor(dout, dtype=torch.float64)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("Hq,Hkv,pos_kind", [(2, 2, "causal"), (4, 2, "causal"), (3, 1, "sparse")])
def test_backward_matches_autograd(Hq, Hkv, pos_kind):
    B, S, D, scale = 2, 24, 8, 0.35
    q, k, v, dout = _inputs(1, B, S, Hq, Hkv, D)
    if pos_kind == "causal":
        q_pos = kv_pos = np.arange(S, dtype=np.int64)
    else:
        rng = np.random.default_rng(2)
        q_pos = np.sort(rng.choice(100, S, replace=False)).astype(np.int64)
        kv_pos = np.sort(rng.choice(100, S, replace=False)).astype(np.int64)
    out, lse = oracle.attention_rows(q, k, v, q_pos, kv_pos, scale)
    dq, dk, dv = oracle.block_bwd(q, k, v, dout, out, lse, q_pos, kv_pos, scale)
    if pos_kind == "sparse":  # rows with no visible key have no gradient at all
        empty = kv_pos[0] > q_pos
        assert np.all(dq[:, empty] == 0)
        q_use = ~empty
    else:
        q_use = np.ones(S, dtype=bool)
    gq, gk, gv = _autograd(q[:, q_use], k, v, dout[:, q_use], q_pos[q_use], kv_pos, scale)
    assert np.max(np.abs(dq[:, q_use] - gq)) < 1e-10
    assert np.max(np.abs(dk - gk)) < 1e-10
    assert np.max(np.abs(dv - gv)) < 1e-10


def test_backward_matches_finite_differences():
    B, S, Hq, Hkv, D, scale = 1, 6, 2, 1, 4, 0.5
    q, k, v, dout = _inputs(3, B, S, Hq, Hkv, D, dyadic=True)
    pos = np.arange(S, dtype=np.int64)
    out, lse = oracle.attention_rows(q, k, v, pos, pos, scale)
    dq, dk, dv = oracle.block_bwd(q, k, v, dout, out, lse, pos, pos, scale)

    def loss(q_, k_, v_):
        o, _ = oracle.attention_rows(q_, k_, v_, pos, pos, scale)
        return float(np.sum(o * dout.astype(np.float64)))

    eps = 2.0 ** -12
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        arrs = [q, k, v]
        for idx in [(0, 0, 0, 0), (0, 3, 0, 2), (0, 5, grad.shape[2] - 1, 3), (0, 2, 0, 1)]:
            plus = [a.copy() for a in arrs]
            minus = [a.copy() for a in arrs]
            plus[which][idx] += eps
            minus[which][idx] -= eps
            fd = (loss(*plus) - loss(*minus)) / (2 * eps)
            assert fd == pytest.approx(grad[idx], abs=1e-6), (which, idx)


def test_ring_backward_adds_up_to_the_whole_gradient():
    B, C, t, Hq, Hkv, D, scale = 1, 4, 4, 4, 2, 8, 0.3
    S = 2 * C * t
    q, k, v, dout = _inputs(5, B, S, Hq, Hkv, D)
    pos = np.arange(S, dtype=np.int64)
    out, lse = oracle.attention_rows(q, k, v, pos, pos, scale)
    dq_all, dk_all, dv_all = oracle.block_bwd(q, k, v, dout, out, lse, pos, pos, scale)
    dk_sum, dv_sum = np.zeros_like(dk_all), np.zeros_like(dv_all)
    for r in range(C):
        zz = oracle.zigzag_positions(S, C, r)
        dq_r, contrib = oracle.ring_rank_share_bwd(q[:, zz], k, v, dout[:, zz], out[:, zz], lse[:, :, zz],
                                                   S, C, r, scale)
        assert np.max(np.abs(dq_r - dq_all[:, zz])) < 1e-12
        for o, (dko, dvo) in contrib.items():
            kz = oracle.zigzag_positions(S, C, o)
            dk_sum[:, kz] += dko
            dv_sum[:, kz] += dvo
    assert np.max(np.abs(dk_sum - dk_all)) < 1e-12
    assert np.max(np.abs(dv_sum - dv_all)) < 1e-12


def test_backward_contribution_pattern_rank1():
    # which of rank 1's query chunks send gradient to each K/V chunk (C = 4)
    B, C, t, H, D, scale = 1, 4, 4, 1, 4, 0.5
    S = 2 * C * t
    q, k, v, dout = _inputs(7, B, S, H, H, D)
    pos = np.arange(S, dtype=np.int64)
    out, lse = oracle.attention_rows(q, k, v, pos, pos, scale)
    reach = {c: [] for c in range(2 * C)}
    for qc in (1, 2 * C - 2):
        rows = np.arange(qc * t, (qc + 1) * t)
        _, dk, dv = oracle.block_bwd(q[:, rows], k, v, dout[:, rows], out[:, rows], lse[:, :, rows],
                                     pos[rows], pos, scale)
        for c in range(2 * C):
            if np.any(dv[:, c * t:(c + 1) * t] != 0) or np.any(dk[:, c * t:(c + 1) * t] != 0):
                reach[c].append(qc)
    g = read_golden("backward_contrib_rank1_c4.txt")
    for key, qchunks in g.items():
        assert reach[int(key.split()[1])] == [int(c) for c in qchunks]


# ---- the bf16 rounding model (p and ds rounded to bf16 before the products that use them)
def test_round_bf16_matches_torch_conversion():
    """The rounding primitive against torch's float32 -> bfloat16 conversion (round to nearest,
    ties to even) on fp32 values: random magnitudes over the whole exponent range, exact ties
    (low 16 bits 0x8000, both parities of the kept bit), and subnormals."""
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.0e38)]
    ties = ((bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties) & (np.abs(ties) < 3.0e38)]
    sub = (rng.integers(1, 2 ** 23, 2000, dtype=np.uint64).astype(np.uint32)).view(np.float32)
    for vals in (x, ties, sub, -sub, np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875])):
        want = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
        got = oracle.round_bf16(vals.astype(np.float64))
        np.testing.assert_array_equal(got, want)


def test_bwd_bf16_model_within_rounding_bound():
    """Each term of a gradient sum carries one bf16 rounding (of p in dv, of ds in dq and dk),
    at most 2^-9 of itself; on these N(0,1) inputs the model stays within 2^-6 of the largest
    entry of the exact backward, and the rounding does take effect (the results differ)."""
    B, S, Hq, Hkv, D, scale = 1, 40, 4, 2, 16, 0.25
    q, k, v, dout = _inputs(21, B, S, Hq, Hkv, D)
    pos = np.arange(S, dtype=np.int64)
    out, lse = oracle.attention_rows(q, k, v, pos, pos, scale)
    exact = oracle.block_bwd(q, k, v, dout, out, lse, pos, pos, scale)
    model = oracle.block_bwd(q, k, v, dout, out, lse, pos, pos, scale, bf16_pds=True)
    for e, m in zip(exact, model):
        diff = float(np.max(np.abs(e - m)))
        assert 0.0 < diff <= 2.0 ** -6 * float(np.max(np.abs(e)))


def test_bwd_bf16_model_exact_when_p_is_one():
    """One query that sees one key: p = 1 and ds = 0 are bf16 values, so the model equals the
    exact backward (dq = dk = 0, dv = dout)."""
    q, k, v, dout = _inputs(22, 1, 1, 2, 1, 8)
    pos = np.zeros(1, dtype=np.int64)
    out, lse = oracle.attention_rows(q, k, v, pos, pos, 0.5)
    exact = oracle.block_bwd(q, k, v, dout, out, lse, pos, pos, 0.5)
    model = oracle.block_bwd(q, k, v, dout, out, lse, pos, pos, 0.5, bf16_pds=True)
    for e, m in zip(exact, model):
        np.testing.assert_array_equal(e, m)
    np.testing.assert_array_equal(model[2][0, 0, 0], dout[0, 0].astype(np.float64).sum(axis=0))

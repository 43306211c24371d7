"""Pins for the oracle's zigzag Ulysses exchange and two-dimensional mesh functions, against
what the pages fix (the mesh's group lists, the rank-order gather) and against brute force
on tiny inputs."""
from __future__ import annotations

import numpy as np
import pytest

import oracle


def test_usp_groups_match_page(golden):
    g = golden("usp_groups_c8.txt")
    C, A, R = int(g["C"][0]), int(g["A"][0]), int(g["R"][0])
    assert C == A * R
    a2a, p2p = oracle.usp_groups(C, A)
    assert a2a == [[int(x) for x in grp.split(",")] for grp in g["a2a"]]
    assert p2p == [[int(x) for x in grp.split(",")] for grp in g["p2p"]]


@pytest.mark.parametrize("S,A,R", [(64, 2, 4), (96, 3, 2), (128, 4, 2), (48, 1, 3), (80, 5, 1)])
def test_group_positions_are_a_zigzag_partition_over_R(S, A, R):
    seen = []
    for g in range(R):
        pos = oracle.group_positions(S, A, R, g)
        assert np.array_equal(pos, oracle.zigzag_positions(S, R, g))
        seen.append(pos)
    assert np.array_equal(np.sort(np.concatenate(seen)), np.arange(S))


def _labelled_stack(C, B, t, H, D):
    """Stacked zigzag shards whose elements encode (b, position, head, d)."""
    st = np.empty((C, B, 2 * t, H, D), dtype=np.int64)
    for r in range(C):
        for b in range(B):
            for i in range(2 * t):
                p = r * t + i if i < t else (2 * C - 1 - r) * t + (i - t)
                for h in range(H):
                    for d in range(D):
                        st[r, b, i, h, d] = ((b * 1000 + p) * 100 + h) * 10 + d
    return st


@pytest.mark.parametrize("C,B,t,H,D", [(3, 2, 2, 6, 2), (4, 1, 3, 4, 3)])
def test_zigzag_exchange_brute_force(C, B, t, H, D):
    st = _labelled_stack(C, B, t, H, D)
    S, hg = 2 * C * t, H // C
    for g in range(C):
        got = oracle.ulysses_zigzag_seq_to_heads(st, C, g)
        want = np.empty((B, S, hg, D), dtype=np.int64)
        for b in range(B):
            for p in range(S):
                for h in range(hg):
                    for d in range(D):
                        want[b, p, h, d] = ((b * 1000 + p) * 100 + g * hg + h) * 10 + d
        assert np.array_equal(got, want)
        back = np.zeros_like(st)
        oracle.ulysses_zigzag_heads_to_seq(got, C, g, back)
        assert np.array_equal(back[:, :, :, g * hg:(g + 1) * hg], st[:, :, :, g * hg:(g + 1) * hg])
        assert not back[:, :, :, :g * hg].any() and not back[:, :, :, (g + 1) * hg:].any()


def test_plain_exchange_of_zigzag_shards_is_rank_order(golden):
    # without the reorder, the exchange leaves the chunks in the page's rank-gather order
    C, t = 4, 2
    st = _labelled_stack(C, 1, t, C, 1)
    grouped = oracle.ulysses_seq_to_heads(st, C, 0)
    chunk_of_row = (grouped[0, :, 0, 0] // 1000 % 1000) // t
    order = [int(x) for x in golden("gather_order_c4.txt")["order"]]
    assert list(chunk_of_row[::t]) == order


@pytest.mark.parametrize("A,R", [(2, 4), (4, 2), (1, 8)])
def test_usp_share_ring_matches_direct(A, R):
    rng = np.random.default_rng(7)
    B, S, Hq, Hkv, D = 1, 64, 8, 4, 8
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    scale = 0.3
    for r in range(A * R):
        g, a = oracle.usp_rank_coords(r, A)
        d_out, d_lse = oracle.usp_rank_share(q, k, v, S, A, R, r, scale)
        pos = oracle.group_positions(S, A, R, g)
        hq, hk = Hq // A, Hkv // A
        r_out, r_lse, _ = oracle.ring_rank_share(q[:, pos][:, :, a * hq:(a + 1) * hq],
                                                 k[:, :, a * hk:(a + 1) * hk], v[:, :, a * hk:(a + 1) * hk],
                                                 S, R, g, scale)
        assert np.max(np.abs(d_out - r_out)) < 1e-12
        assert np.max(np.abs(d_lse - r_lse)) < 1e-12

"""Pins of the CPU oracle to what the pages and the mathematics fix (no GPU).

Every check here compares the oracle with something other than itself: values the pages
print (fixtures under tests/golden, each citing its page and section), closed forms,
invariants, or a library routine that a special case reduces to (torch's fp64
scaled_dot_product_attention on the CPU).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle

from conftest import read_golden


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------------------
# Zigzag ownership and the all-gather order
# ----------------------------------------------------------------------------------------
def test_zigzag_c4_matches_pages():
    g = read_golden("zigzag_c4.txt")
    t = 5
    for r in range(4):
        pos = oracle.zigzag_positions(8 * t, 4, r)
        chunk_ids = list(dict.fromkeys((pos // t).tolist()))  # chunk ids in local order
        assert chunk_ids == [int(x) for x in g[str(r)]]


@pytest.mark.parametrize("C", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("t", [1, 3, 16])
def test_zigzag_is_a_balanced_partition(C, t):
    S = 2 * C * t
    all_pos = []
    for r in range(C):
        pos = oracle.zigzag_positions(S, C, r)
        assert pos.shape == (S // C,)
        assert np.all(np.diff(pos) > 0), "local positions must be strictly increasing"
        assert pos[0] == r * t and pos[t] == (2 * C - 1 - r) * t  # early chunk first
        all_pos.append(pos)
    cat = np.concatenate(all_pos)
    assert np.array_equal(np.sort(cat), np.arange(S)), "disjoint and covering [0, S)"


def test_zigzag_rejects_bad_shapes():
    with pytest.raises(ValueError):
        oracle.zigzag_positions(30, 4, 0)  # S not divisible by 2C
    with pytest.raises(ValueError):
        oracle.zigzag_positions(32, 4, 4)  # rank out of range


def test_gather_order_c4_matches_pages():
    g = read_golden("gather_order_c4.txt")
    t = 3
    gp = oracle.gathered_positions(8 * t, 4)
    order = (gp[::t] // t).tolist()
    assert order == [int(x) for x in g["order"]]


@pytest.mark.parametrize("C", [1, 2, 4, 8])
def test_reorder_reads_back_the_permutation(C):
    t, B = 4, 2
    S = 2 * C * t
    gp = oracle.gathered_positions(S, C)
    # rows carry their own global position: reordering to sequence order gives an iota
    x = np.broadcast_to(gp[None, :, None], (B, S, 3)).astype(np.int64).copy()
    y = oracle.reorder(x, C, 0)
    assert np.array_equal(y[:, :, 0], np.broadcast_to(np.arange(S), (B, S)))
    # and the inverse direction puts an iota back into rank order
    z = oracle.reorder(y, C, 1)
    assert np.array_equal(z, x)


def test_reorder_round_trip_on_random_bytes():
    rng = _rng(1)
    for C, t, row in [(4, 3, 7), (8, 2, 16), (3, 5, 1)]:
        S = 2 * C * t
        x = rng.integers(0, 256, size=(2, S, row), dtype=np.uint8)
        assert np.array_equal(oracle.reorder(oracle.reorder(x, C, 0), C, 1), x)
        assert np.array_equal(oracle.reorder(oracle.reorder(x, C, 1), C, 0), x)


# ----------------------------------------------------------------------------------------
# Which keys each query sees: the mask on global positions
# ----------------------------------------------------------------------------------------
def _chunk_visibility(S, C, r, t):
    """Run the oracle with zero keys (all scores equal) and one-hot chunk-id values, so
    out[i, c] = (#keys of chunk c visible to query i) / (#visible keys)."""
    q_pos = oracle.zigzag_positions(S, C, r)
    kv_pos = np.arange(S, dtype=np.int64)
    n_chunks = 2 * C
    q = _rng(2).standard_normal((1, S // C, 1, n_chunks)).astype(np.float32)
    k = np.zeros((1, S, 1, n_chunks), np.float32)
    v = np.zeros((1, S, 1, n_chunks), np.float32)
    v[0, np.arange(S), 0, np.arange(S) // t] = 1.0
    out, lse = oracle.attention_rows(q, k, v, q_pos, kv_pos, 0.125)
    return q_pos, out[0, :, 0, :], lse[0, 0]


def test_visible_chunks_rank1_matches_pages():
    C, t = 4, 6
    S = 2 * C * t
    q_pos, frac, lse = _chunk_visibility(S, C, 1, t)
    # exact fractions: keys of chunk c visible to a query at position p, over p + 1
    for i, p in enumerate(q_pos):
        counts = np.array([max(0, min(p + 1, (c + 1) * t) - c * t) for c in range(2 * C)])
        np.testing.assert_allclose(frac[i], counts / (p + 1), rtol=0, atol=1e-15)
        assert lse[i] == pytest.approx(math.log(p + 1), abs=1e-14)  # all scores are 0
    g = read_golden("visible_chunks_rank1_c4.txt")
    for key, chunks in g.items():
        qc = int(key.split()[1])
        rows = np.where(q_pos // t == qc)[0]
        seen = sorted(set(np.nonzero(frac[rows].sum(axis=0) > 0)[0].tolist()))
        assert seen == [int(c) for c in chunks]
    g = read_golden("backward_contrib_rank1_c4.txt")
    for key, qchunks in g.items():
        kc = int(key.split()[1])
        reach = sorted({int(q_pos[i] // t) for i in range(len(q_pos)) if frac[i, kc] > 0})
        assert reach == [int(c) for c in qchunks]


def test_first_position_sees_only_itself():
    rng = _rng(3)
    q = rng.standard_normal((1, 4, 1, 8)).astype(np.float32)
    k = rng.standard_normal((1, 4, 1, 8)).astype(np.float32)
    v = rng.standard_normal((1, 4, 1, 8)).astype(np.float32)
    pos = np.arange(4, dtype=np.int64)
    out, lse = oracle.attention_rows(q, k, v, pos, pos, 0.5)
    assert np.array_equal(out[0, 0, 0], v[0, 0, 0].astype(np.float64))
    assert lse[0, 0, 0] == pytest.approx(0.5 * float(np.dot(q[0, 0, 0].astype(np.float64),
                                                              k[0, 0, 0].astype(np.float64))), abs=1e-14)


def test_two_identical_keys_average_and_add_ln2():
    rng = _rng(4)
    q = rng.standard_normal((1, 1, 1, 8)).astype(np.float32)
    kk = rng.standard_normal(8).astype(np.float32)
    k = np.stack([kk, kk])[None, :, None, :]
    v = rng.standard_normal((1, 2, 1, 8)).astype(np.float32)
    out, lse = oracle.attention_rows(q, k, v, np.array([5]), np.array([3, 5]), 0.3)
    np.testing.assert_allclose(out[0, 0, 0], v[0, :, 0].astype(np.float64).mean(axis=0), atol=1e-15)
    s = 0.3 * float(np.dot(q[0, 0, 0].astype(np.float64), kk.astype(np.float64)))
    assert lse[0, 0, 0] == pytest.approx(s + math.log(2.0), abs=1e-14)


def test_row_without_visible_key_is_empty():
    rng = _rng(5)
    q = rng.standard_normal((1, 2, 1, 4)).astype(np.float32)
    k = rng.standard_normal((1, 3, 1, 4)).astype(np.float32)
    v = rng.standard_normal((1, 3, 1, 4)).astype(np.float32)
    out, lse = oracle.attention_rows(q, k, v, np.array([1, 10]), np.array([2, 3, 4]), 1.0)
    assert np.all(out[0, 0] == 0.0) and lse[0, 0, 0] == -np.inf
    assert np.isfinite(lse[0, 0, 1])


# ----------------------------------------------------------------------------------------
# Direct attention against torch's fp64 scaled_dot_product_attention (CPU)
# ----------------------------------------------------------------------------------------
def _sdpa(q, k, v, mask, scale):
    """Library routine in fp64 on [B,S,H,D] inputs; kv heads expanded by repeat."""
    Hq, Hkv = q.shape[2], k.shape[2]
    tq = torch.from_numpy(q.astype(np.float64)).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    tv = torch.from_numpy(v.astype(np.float64)).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(
        tq.contiguous(), tk.contiguous(), tv.contiguous(), attn_mask=torch.from_numpy(mask), scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 1), (4, 2), (8, 2)])
def test_direct_matches_sdpa_full_causal(Hq, Hkv):
    rng = _rng(6)
    B, S, D = 2, 37, 16
    q = rng.standard_normal((B, S, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, S, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((B, S, Hkv, D)).astype(np.float32)
    pos = np.arange(S, dtype=np.int64)
    scale = 1.0 / math.sqrt(D)
    out, _ = oracle.attention_rows(q, k, v, pos, pos, scale)
    ref = _sdpa(q, k, v, np.tril(np.ones((S, S), dtype=bool)), scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-13)


def test_direct_matches_sdpa_on_zigzag_positions():
    rng = _rng(7)
    C, t, H, D = 4, 8, 3, 8
    S = 2 * C * t
    k = rng.standard_normal((1, S, H, D)).astype(np.float32)
    v = rng.standard_normal((1, S, H, D)).astype(np.float32)
    for r in range(C):
        q_pos = oracle.zigzag_positions(S, C, r)
        q = rng.standard_normal((1, S // C, H, D)).astype(np.float32)
        out, _ = oracle.attention_rows(q, k, v, q_pos, np.arange(S), 0.37)
        mask = np.arange(S)[None, :] <= q_pos[:, None]
        np.testing.assert_allclose(out, _sdpa(q, k, v, mask, 0.37), rtol=0, atol=1e-13)


def test_lse_matches_sdpa_with_a_sink_key():
    """Append a key of score 0 whose value is a one-hot in an extra column: SDPA gives it
    weight w = 1 / (1 + e^lse), so lse = ln((1 - w) / w) independently of the oracle."""
    rng = _rng(8)
    B, S, H, D = 1, 20, 2, 8
    q = rng.standard_normal((B, S, H, D)).astype(np.float32)
    k = rng.standard_normal((B, S, H, D)).astype(np.float32)
    v = rng.standard_normal((B, S, H, D)).astype(np.float32)
    pos = np.arange(S, dtype=np.int64)
    scale = 0.6
    _, lse = oracle.attention_rows(q, k, v, pos, pos, scale)
    k2 = np.concatenate([np.zeros((B, 1, H, D), np.float32), k], axis=1)
    v2 = np.concatenate([np.zeros((B, S + 1, H, 1), np.float32),
                         np.concatenate([np.zeros((B, 1, H, D), np.float32), v], axis=1)], axis=3)
    v2[:, 0, :, 0] = 1.0
    q2 = q
    mask = np.concatenate([np.ones((S, 1), bool), np.tril(np.ones((S, S), bool))], axis=1)
    tq = torch.from_numpy(q2.astype(np.float64)).permute(0, 2, 1, 3).contiguous()
    tk = torch.from_numpy(k2.astype(np.float64)).permute(0, 2, 1, 3).contiguous()
    tv = torch.from_numpy(v2.astype(np.float64)).permute(0, 2, 1, 3).contiguous()
    # SDPA requires equal head dims for q and k only; v may be wider
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(mask), scale=scale)
    w = o[..., 0].numpy()  # [B, H, S]
    np.testing.assert_allclose(lse, np.log((1.0 - w) / w), rtol=0, atol=1e-11)


# ----------------------------------------------------------------------------------------
# The merge
# ----------------------------------------------------------------------------------------
def _rand_partial(rng, B, s, H, D):
    return rng.standard_normal((B, s, H, D)), rng.standard_normal((B, H, s)) * 3.0


def test_merge_scales_sum_to_one_and_identity():
    rng = _rng(9)
    o1, l1 = _rand_partial(rng, 1, 6, 2, 4)
    o2, l2 = _rand_partial(rng, 1, 6, 2, 4)
    # a tile of constant ones exposes the tile weight; a zero tile exposes the old weight
    ones = np.ones_like(o1)
    zero = np.zeros_like(o1)
    a, _ = oracle.merge(ones, l1, zero, l2)   # = old_scale
    c, _ = oracle.merge(zero, l1, ones, l2)   # = tile_scale
    np.testing.assert_allclose(a + c, 1.0, rtol=0, atol=1e-15)
    # merging an empty tile (0, -inf) changes nothing, bit for bit
    o, L = oracle.merge(o1, l1, zero, np.full_like(l1, -np.inf))
    assert np.array_equal(o, o1) and np.array_equal(L, l1)
    # two empty sides stay empty and never produce NaN
    o, L = oracle.merge(zero, np.full_like(l1, -np.inf), zero, np.full_like(l1, -np.inf))
    assert np.all(o == 0) and np.all(L == -np.inf)


def test_merge_commutes_and_associates():
    rng = _rng(10)
    a = _rand_partial(rng, 2, 5, 3, 4)
    b = _rand_partial(rng, 2, 5, 3, 4)
    c = _rand_partial(rng, 2, 5, 3, 4)
    ab = oracle.merge(*a, *b)
    ba = oracle.merge(*b, *a)
    assert np.array_equal(ab[0], ba[0]) and np.array_equal(ab[1], ba[1])
    left = oracle.merge(*ab, *c)
    right = oracle.merge(*a, *oracle.merge(*b, *c))
    np.testing.assert_allclose(left[0], right[0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(left[1], right[1], rtol=0, atol=1e-14)


def test_merge_of_identical_tiles_adds_ln2():
    rng = _rng(11)
    o, l = _rand_partial(rng, 1, 7, 2, 4)
    mo, ml = oracle.merge(o, l, o, l)
    np.testing.assert_allclose(mo, o, rtol=0, atol=1e-15)
    np.testing.assert_allclose(ml, l + math.log(2.0), rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------------------
# Block-wise equals direct, and the two block combines agree
# ----------------------------------------------------------------------------------------
def _full_inputs(S, Hq, Hkv, D, seed):
    rng = _rng(seed)
    return (rng.standard_normal((1, S, Hq, D)).astype(np.float32),
            rng.standard_normal((1, S, Hkv, D)).astype(np.float32),
            rng.standard_normal((1, S, Hkv, D)).astype(np.float32))


@pytest.mark.parametrize("C,t,Hq,Hkv,D", [(4, 32, 2, 2, 64), (3, 7, 4, 2, 16), (8, 4, 2, 1, 8)])
def test_ring_share_equals_direct_fp64(C, t, Hq, Hkv, D):
    g = read_golden("blockwise_vs_direct.txt")
    S = 2 * C * t
    q, k, v = _full_inputs(S, Hq, Hkv, D, 12)
    pos = np.arange(S, dtype=np.int64)
    scale = 1.0 / math.sqrt(D)
    direct, dlse = oracle.attention_rows(q, k, v, pos, pos, scale)
    worst = 0.0
    for r in range(C):
        zz = oracle.zigzag_positions(S, C, r)
        out, lse, blocks = oracle.ring_rank_share(q[:, zz], k, v, S, C, r, scale)
        worst = max(worst, float(np.abs(out - direct[:, zz]).max()), float(np.abs(lse - dlse[:, :, zz]).max()))
        # every final row sees at least its own key: lse finite
        assert np.all(np.isfinite(lse))
        cf, cflse = oracle.closed_form_share(q[:, zz], k, v, S, C, r, scale)
        np.testing.assert_allclose(cf, out, rtol=0, atol=float(g["bound"][0]))
        np.testing.assert_allclose(cflse, lse, rtol=0, atol=float(g["bound"][0]))
    print(f"block-wise vs direct, fp64: max abs diff {worst:.2e} (pages quote {g['quoted'][0]})")
    assert worst <= float(g["bound"][0])


def test_zigzag_tile_cases_per_step():
    """Per ring step, rank r's pairs with owner o's shard: o == r gives 2t^2 + t,
    any other owner gives 2t^2; the first local chunk sees nothing of a later owner."""
    C, t = 4, 6
    S = 2 * C * t
    for r in range(C):
        q_pos = oracle.zigzag_positions(S, C, r)
        for o in range(C):
            kv_pos = oracle.zigzag_positions(S, C, o)
            pairs = oracle.visible_pairs(q_pos, kv_pos)
            assert pairs == (2 * t * t + t if o == r else 2 * t * t)
            if o > r:
                assert oracle.visible_pairs(q_pos[:t], kv_pos) == 0


def test_contiguous_ring_p4_matches_pages():
    """The pages' own check: 4 ranks, S=32, H=8, D=16, contiguous shards, future blocks
    skipped; each rank matches single-process causal attention, and the blocks actually
    computed per rank are [1, 2, 3, 4]."""
    g = read_golden("ring_blocks_p4.txt")
    S, H, D, P = 32, 8, 16, 4
    q, k, v = _full_inputs(S, H, H, D, 13)
    pos = np.arange(S, dtype=np.int64)
    direct, _ = oracle.attention_rows(q, k, v, pos, pos, 1.0 / math.sqrt(D))
    computed = []
    for r in range(P):
        mine = oracle.contiguous_positions(S, P, r)
        out, _, blocks = oracle.ring_rank_share(q[:, mine], k, v, S, P, r, 1.0 / math.sqrt(D),
                                                layout="contiguous")
        np.testing.assert_allclose(out, direct[:, mine], rtol=0, atol=1e-5)
        computed.append(sum(1 for _, _, tl in blocks if np.isfinite(tl).any()))
    assert computed == [int(x) for x in g["blocks"]]
    assert oracle.contiguous_ring_blocks(P) == computed


# ----------------------------------------------------------------------------------------
# Work models
# ----------------------------------------------------------------------------------------
def test_imbalance_table_matches_pages():
    g = read_golden("imbalance_contiguous.txt")
    for key, (ratio,) in g.items():
        P = int(key.split()[1])
        w = oracle.block_work_diag_one(P, "contiguous")
        assert w == [float(p + 1) for p in range(P)]
        assert f"{max(w) / (sum(w) / P):.2f}" == ratio
        assert max(w) / (sum(w) / P) == pytest.approx(2 * P / (P + 1))


def test_zigzag_load_matches_pages():
    g = read_golden("zigzag_load_p4.txt")
    assert oracle.block_work_diag_one(4, "zigzag") == [float(x) for x in g["load"]]
    for P in (2, 3, 8, 16):
        assert oracle.block_work_diag_one(P, "zigzag") == [2.0 * P + 1] * P


def test_work_per_rank_matches_pages_and_exact_pairs():
    g = read_golden("work_per_rank_p4.txt")
    P = 4
    contiguous = {r: [2 * r, 2 * r + 1] for r in range(P)}
    zigzag = {r: [r, 2 * P - 1 - r] for r in range(P)}
    assert [oracle.chunk_work_diag_half(contiguous[r]) for r in range(P)] == [float(x) for x in g["contiguous"]]
    assert [oracle.chunk_work_diag_half(zigzag[r]) for r in range(P)] == [float(x) for x in g["zigzag"]]
    # exact pair counts: (model) * t^2 + (number of chunks) * t / 2
    for t in (1, 2, 7, 64):
        S = 2 * P * t
        kv = np.arange(S)
        for r in range(P):
            zz = oracle.zigzag_positions(S, P, r)
            assert zz[0] // t == zigzag[r][0] and zz[-1] // t == zigzag[r][1]
            assert oracle.visible_pairs(zz, kv) == oracle.chunk_work_diag_half(zigzag[r]) * t * t + t


@pytest.mark.parametrize("C", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("t", [1, 5, 32])
def test_zigzag_pairs_equal_for_every_rank(C, t):
    S = 2 * C * t
    kv = np.arange(S)
    counts = [oracle.visible_pairs(oracle.zigzag_positions(S, C, r), kv) for r in range(C)]
    assert counts == [2 * C * t * t + t] * C
    assert sum(counts) == S * (S + 1) // 2


# ----------------------------------------------------------------------------------------
# Ulysses
# ----------------------------------------------------------------------------------------
def _replay_all_to_all(shards, P):
    """NumPy replay of the sequence->heads exchange as the handbook describes it: each rank
    splits its [S/P, H, D] shard by destination head group (group p = the p-th share of the
    heads), ships group p to rank p, and rank p stacks what it receives in source-rank
    order to get the whole sequence for its heads."""
    s, H, D = shards[0].shape
    send = [x.reshape(s, P, H // P, D).swapaxes(0, 1) for x in shards]   # [P(dest), s, H/P, D]
    return [np.concatenate([send[src][dest] for src in range(P)], axis=0) for dest in range(P)]


def test_ulysses_shapes_match_pages():
    g = read_golden("ulysses_shapes.txt")
    S, H, D, P = (int(g[x][0]) for x in ("S", "H", "D", "P"))
    stacked = np.zeros((P, 1, S // P, H, D), np.float32)
    out = oracle.ulysses_seq_to_heads(stacked, P, 0)
    assert tuple(stacked.shape[2:]) == tuple(int(x) for x in g["input"])
    assert tuple(out.shape[1:]) == tuple(int(x) for x in g["attention"])


@pytest.mark.parametrize("P,S,H,D", [(4, 32, 8, 16), (2, 6, 4, 3), (8, 16, 8, 2)])
def test_ulysses_permute_matches_replay_and_round_trips(P, S, H, D):
    rng = _rng(14)
    full = rng.standard_normal((S, H, D)).astype(np.float32)
    shards = [full[p * (S // P):(p + 1) * (S // P)] for p in range(P)]
    stacked = np.stack(shards)[:, None]          # [P, B=1, S/P, H, D]
    replay = _replay_all_to_all(shards, P)
    back = np.zeros_like(stacked)
    for g in range(P):
        grouped = oracle.ulysses_seq_to_heads(stacked, P, g)
        assert np.array_equal(grouped[0], replay[g])
        # contiguous shards: the grouped tensor is the global sequence for group g's heads
        assert np.array_equal(grouped[0], full[:, g * (H // P):(g + 1) * (H // P)])
        oracle.ulysses_heads_to_seq(grouped, P, g, back)
    assert np.array_equal(back, stacked)


def test_ulysses_attention_equals_direct():
    """Sequence->heads, full causal attention per head group, heads->sequence equals direct
    causal attention on the whole tensor (the handbook's single-process check)."""
    rng = _rng(15)
    P, S, H, Hkv, D = 4, 32, 8, 4, 16
    q = rng.standard_normal((1, S, H, D)).astype(np.float32)
    k = rng.standard_normal((1, S, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((1, S, Hkv, D)).astype(np.float32)
    pos = np.arange(S, dtype=np.int64)
    scale = 1.0 / math.sqrt(D)
    ref, _ = oracle.attention_rows(q, k, v, pos, pos, scale)
    st = lambda x: x.reshape(1, P, S // P, *x.shape[2:]).swapaxes(0, 1).copy()  # contiguous shards
    out_stacked = np.zeros((P, 1, S // P, H, D), np.float64)
    for g in range(P):
        qg = oracle.ulysses_seq_to_heads(st(q), P, g)
        kg = oracle.ulysses_seq_to_heads(st(k), P, g)
        vg = oracle.ulysses_seq_to_heads(st(v), P, g)
        og, _ = oracle.attention_rows(qg, kg, vg, pos, pos, scale)
        oracle.ulysses_heads_to_seq(og, P, g, out_stacked)
    out = out_stacked.swapaxes(0, 1).reshape(1, S, H, D)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)

"""Zigzag Ulysses exchange and the two-dimensional mesh on the HIP path, against the oracle:
the exchange bit for bit, the shares within the attention tolerances (every row at small
sizes, sampled rows at the workloads' full sizes, in the launch sequence the benchmark
times)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import context_causal_attention_amd as cp
import oracle
from context_causal_attention_amd.workloads import WORKLOADS, Workload
from helpers import TOL, gen, max_abs, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _zz_stack(w, name, heads, ranks):
    """Stacked zigzag shards [len(ranks), B, S/C, H, D] of the given ranks, CPU."""
    C = w.cp_size
    return torch.stack([gen(w, name, [r, 2 * C - 1 - r], heads) for r in ranks])


@pytest.mark.parametrize("dtype,C,B,t,H,D", [(torch.bfloat16, 4, 2, 8, 8, 16), (torch.float32, 3, 1, 5, 6, 4),
                                            (torch.float32, 2, 1, 3, 2, 3)])
def test_zigzag_exchange_bit_exact(dtype, C, B, t, H, D):
    g = torch.Generator().manual_seed(11)
    st = torch.randn((C, B, 2 * t, H, D), generator=g).to(dtype)
    for grp in range(C):
        got = cp.ulysses_seq_to_heads(st.to(DEV), grp, zigzag=True).cpu()
        want = oracle.ulysses_zigzag_seq_to_heads(st.view(torch.int16 if dtype == torch.bfloat16 else torch.int32)
                                                  .numpy(), C, grp)
        assert np.array_equal(got.view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy(), want)
        back = torch.zeros_like(st).to(DEV)
        cp.ulysses_heads_to_seq(got.to(DEV), grp, back, zigzag=True)
        ref = np.zeros(st.shape, dtype=want.dtype)
        oracle.ulysses_zigzag_heads_to_seq(want, C, grp, ref)
        itype = torch.int16 if dtype == torch.bfloat16 else torch.int32
        assert np.array_equal(back.cpu().view(itype).numpy(), ref)


def _small(name, kind, S, C, Hq, Hkv, **kw):
    return Workload(name, kind, 1, S, Hq, Hkv, 128, "bf16", C, **kw)


def test_ulysses_zigzag_share_small_every_row():
    w = _small("uz_small", "ulysses", 1024, 4, 8, 4, group=1, zigzag=True)
    C, g = w.cp_size, w.group
    qs, ks, vs = (_zz_stack(w, n, h, range(C)) for n, h in (("q", w.heads_q), ("k", w.heads_kv), ("v", w.heads_kv)))
    out_st = torch.zeros((C, 1, w.local_len, w.heads_q, 128), device=DEV)
    og, lse = cp.ulysses_share_fwd(qs.to(DEV), ks.to(DEV), vs.to(DEV), g, w.scale, out_st, zigzag=True)
    torch.cuda.synchronize()
    hq, hk = w.heads_q // C, w.heads_kv // C
    ids = range(2 * C)
    qf, kf, vf = (gen(w, n, ids, h).float().numpy() for n, h in (("q", w.heads_q), ("k", w.heads_kv), ("v", w.heads_kv)))
    pos = np.arange(w.seq_len, dtype=np.int64)
    ref_o, ref_l = oracle.attention_rows(qf[:, :, g * hq:(g + 1) * hq], kf[:, :, g * hk:(g + 1) * hk],
                                         vf[:, :, g * hk:(g + 1) * hk], pos, pos, w.scale)
    tol_o, tol_l = TOL["bf16"]
    assert max_abs(og.cpu().numpy(), ref_o) <= tol_o
    assert max_abs(lse.cpu().numpy(), ref_l) <= tol_l
    # the inverse exchange puts every row back on its shard, bit for bit
    ref_st = np.zeros(tuple(out_st.shape), dtype=np.float32)
    oracle.ulysses_zigzag_heads_to_seq(og.cpu().numpy(), C, g, ref_st)
    assert np.array_equal(out_st.cpu().numpy(), ref_st)


@pytest.mark.parametrize("B,fused", [(1, None), (1, False), (2, None)])
def test_ulysses_contiguous_share_small_every_row(B, fused):
    # contiguous shards: with B = 1 the exchanges fold into the attention's row addressing,
    # with B = 2 (or fused=False) they run as explicit permutes; both against the oracle
    w = Workload("u_small", "ulysses", B, 1024, 8, 4, 128, "bf16", 4, group=2)
    C, g, s = w.cp_size, w.group, w.local_len
    ids = range(2 * C)
    full = {n: gen(w, n, ids, h) for n, h in (("q", w.heads_q), ("k", w.heads_kv), ("v", w.heads_kv))}
    stack = lambda x: x.reshape(B, C, s, *x.shape[2:]).transpose(0, 1).contiguous().to(DEV)
    out_st = torch.zeros((C, B, s, w.heads_q, 128), device=DEV)
    og, lse = cp.ulysses_share_fwd(stack(full["q"]), stack(full["k"]), stack(full["v"]), g, w.scale, out_st,
                                   zigzag=False, fused=fused)
    torch.cuda.synchronize()
    hq, hk = w.heads_q // C, w.heads_kv // C
    pos = np.arange(w.seq_len, dtype=np.int64)
    ref_o, ref_l = oracle.attention_rows(full["q"][:, :, g * hq:(g + 1) * hq].float().numpy(),
                                         full["k"][:, :, g * hk:(g + 1) * hk].float().numpy(),
                                         full["v"][:, :, g * hk:(g + 1) * hk].float().numpy(), pos, pos, w.scale)
    tol_o, tol_l = TOL["bf16"]
    assert max_abs(og.cpu().numpy(), ref_o) <= tol_o
    assert max_abs(lse.cpu().numpy(), ref_l) <= tol_l
    # the group's heads of every shard hold the group output, the other heads stay zero
    back = out_st.transpose(0, 1).reshape(B, w.seq_len, w.heads_q, 128).cpu()
    assert torch.equal(back[:, :, g * hq:(g + 1) * hq], og.cpu())
    assert torch.count_nonzero(back[:, :, :g * hq]) == 0 and torch.count_nonzero(back[:, :, (g + 1) * hq:]) == 0


def _usp_inputs(w):
    A, C = w.a2a, w.cp_size
    R = C // A
    grp = lambda n, h, o: _zz_stack(w, n, h, [o * A + j for j in range(A)]).to(DEV)
    return ([grp("q", w.heads_q, o) for o in range(R)], [grp("k", w.heads_kv, o) for o in range(R)],
            [grp("v", w.heads_kv, o) for o in range(R)])


def test_usp_share_small_every_rank_every_row():
    w = _small("usp_small", "usp", 2048, 8, 8, 4, a2a=2)
    A, C = w.a2a, w.cp_size
    qsts, ksts, vsts = _usp_inputs(w)
    ids = range(2 * C)
    qf, kf, vf = (gen(w, n, ids, h).float().numpy() for n, h in (("q", w.heads_q), ("k", w.heads_kv), ("v", w.heads_kv)))
    tol_o, tol_l = TOL["bf16"]
    for r in range(C):
        g, a = oracle.usp_rank_coords(r, A)
        out_st = torch.zeros((A, 1, w.local_len, w.heads_q, 128), device=DEV)
        out, lse = cp.usp_share_fwd(qsts[g], ksts, vsts, g, a, w.scale, out_st)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle.usp_rank_share(qf, kf, vf, w.seq_len, A, C // A, r, w.scale)
        eo, el = max_abs(out.cpu().numpy(), ref_o), max_abs(lse.cpu().numpy(), ref_l)
        assert eo <= tol_o and el <= tol_l, f"rank {r}: O {eo:.3g} lse {el:.3g}"
        ref_st = np.zeros(tuple(out_st.shape), dtype=np.float32)
        oracle.ulysses_zigzag_heads_to_seq(out.cpu().numpy(), A, a, ref_st)
        assert np.array_equal(out_st.cpu().numpy(), ref_st)


def test_ulysses_zz_128k_sampled():
    w = WORKLOADS["ulysses_zz_128k"]
    C, g = w.cp_size, w.group
    qs, ks, vs = (_zz_stack(w, n, h, range(C)).to(DEV) for n, h in (("q", w.heads_q), ("k", w.heads_kv), ("v", w.heads_kv)))
    out_st = torch.zeros((C, 1, w.local_len, w.heads_q, 128), device=DEV)
    og, lse = cp.ulysses_share_fwd(qs, ks, vs, g, w.scale, out_st, zigzag=True)
    torch.cuda.synchronize()
    del qs, ks, vs
    hq, hk = w.heads_q // C, w.heads_kv // C
    ids = range(2 * C)
    qf = gen(w, "q", ids, w.heads_q)[:, :, g * hq:(g + 1) * hq].float().numpy()
    kf = gen(w, "k", ids, w.heads_kv)[:, :, g * hk:(g + 1) * hk].float().numpy()
    vf = gen(w, "v", ids, w.heads_kv)[:, :, g * hk:(g + 1) * hk].float().numpy()
    rows = sample_rows(w.seq_len, w.chunk_len, seed=5, per_chunk_random=4)
    pos = np.arange(w.seq_len, dtype=np.int64)
    ref_o, ref_l = oracle.attention_rows(qf, kf, vf, pos, pos, w.scale, rows=rows)
    ridx = torch.from_numpy(rows).to(DEV)
    eo, el = max_abs(og[:, ridx].cpu().numpy(), ref_o), max_abs(lse[:, :, ridx].cpu().numpy(), ref_l)
    print(f"ulysses_zz_128k: max abs err O {eo:.3g}, lse {el:.3g} over {len(rows)} rows")
    tol_o, tol_l = TOL[w.dtype]
    assert eo <= tol_o and el <= tol_l


def test_usp_128k_sampled():
    w = WORKLOADS["usp_128k"]
    A, C = w.a2a, w.cp_size
    R = C // A
    g, a = oracle.usp_rank_coords(w.rank, A)
    qsts, ksts, vsts = _usp_inputs(w)
    out_st = torch.zeros((A, 1, w.local_len, w.heads_q, 128), device=DEV)
    out, lse = cp.usp_share_fwd(qsts[g], ksts, vsts, g, a, w.scale, out_st)
    torch.cuda.synchronize()
    del qsts, ksts, vsts
    ids = range(2 * C)
    qf, kf, vf = (gen(w, n, ids, h).float().numpy() for n, h in (("q", w.heads_q), ("k", w.heads_kv), ("v", w.heads_kv)))
    n = w.seq_len // R
    rows = sample_rows(n, w.chunk_len, seed=3, per_chunk_random=3)
    ref_o, ref_l = oracle.usp_rank_share(qf, kf, vf, w.seq_len, A, R, w.rank, w.scale, rows=rows)
    ridx = torch.from_numpy(rows).to(DEV)
    eo, el = max_abs(out[:, ridx].cpu().numpy(), ref_o), max_abs(lse[:, :, ridx].cpu().numpy(), ref_l)
    print(f"usp_128k: max abs err O {eo:.3g}, lse {el:.3g} over {len(rows)} rows")
    tol_o, tol_l = TOL[w.dtype]
    assert eo <= tol_o and el <= tol_l

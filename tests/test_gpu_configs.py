"""The five workloads end to end on the HIP path, against the oracle.

Small workloads are compared on every row; the large ones on sampled rows (chunk edges,
tile edges, seeded random rows; all heads), with layout outputs compared in full and bit
for bit.  Each test launches exactly the kernels the benchmark times."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import context_causal_attention_amd as cp
import oracle
from context_causal_attention_amd.workloads import WORKLOADS
from helpers import TOL, f32np, gen, max_abs, sample_rows, zigzag_chunks

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _owner_blocks(w, heads):
    """Every owner's K and V shard (zigzag chunks o and 2C-1-o), on the device."""
    ks, vs = [], []
    for o in range(w.cp_size):
        ks.append(gen(w, "k", zigzag_chunks(w.cp_size, o), heads).to(DEV))
        vs.append(gen(w, "v", zigzag_chunks(w.cp_size, o), heads).to(DEV))
    return ks, vs


def _full_kv_f32(w, heads):
    ids = range(2 * w.cp_size)
    return gen(w, "k", ids, heads).float().numpy(), gen(w, "v", ids, heads).float().numpy()


def _ring_share(w, r, ks, vs, mode="single"):
    """Rank r's share: one launch over the C blocks ("single"), or the ring's per-step form,
    one launch per step merging in its epilogue ("fused") or into a tile followed by the
    merge kernel ("unfused")."""
    C = w.cp_size
    pos = [cp.zigzag_index(w.seq_len, C, o, device=DEV) for o in range(C)]
    q = gen(w, "q", zigzag_chunks(C, r), w.heads_q)
    out, lse = cp.ring_share_fwd(q.to(DEV), ks, vs, pos, r, w.scale, mode=mode)
    torch.cuda.synchronize()
    return q, out, lse


def test_tiny_fp32_every_rank_and_step():
    w = WORKLOADS["tiny_fp32"]
    C = w.cp_size
    ks, vs = _owner_blocks(w, w.heads_kv)
    kf, vf = _full_kv_f32(w, w.heads_kv)
    qf_full = gen(w, "q", range(2 * C), w.heads_q).float().numpy()
    gpos = np.arange(w.seq_len, dtype=np.int64)
    direct, dlse = oracle.attention_rows(qf_full, kf, vf, gpos, gpos, w.scale)
    tol_o, tol_l = TOL["fp32"]
    for r in range(C):
        q, out, lse = _ring_share(w, r, ks, vs)
        zz = oracle.zigzag_positions(w.seq_len, C, r)
        assert max_abs(out.cpu().numpy(), direct[:, zz]) <= tol_o
        assert max_abs(lse.cpu().numpy(), dlse[:, :, zz]) <= tol_l
        # each ring step's tile against the oracle's block attention
        for o in range(C):
            kvp = oracle.zigzag_positions(w.seq_len, C, o)
            t_out, t_lse = cp.block_fwd(q.to(DEV), ks[o], vs[o], torch.from_numpy(zz).to(DEV),
                                        torch.from_numpy(kvp).to(DEV), w.scale)
            r_out, r_lse = oracle.attention_rows(q.numpy(), kf[:, kvp], vf[:, kvp], zz, kvp, w.scale)
            assert max_abs(t_out.cpu().numpy(), r_out) <= tol_o
            assert max_abs(t_lse.cpu().numpy(), r_lse) <= tol_l


def test_rank_share_8k_all_rows():
    """Every row of the 8K rank share against the oracle, in the one-launch form and in the
    ring's per-step forms (the per-step tile merges of "On Context Parallelism",
    Peer-to-peer / Forward); the two per-step forms give the same bits."""
    w = WORKLOADS["rank_share_8k"]
    ks, vs = _owner_blocks(w, w.heads_kv)
    kf, vf = _full_kv_f32(w, w.heads_kv)
    zz = oracle.zigzag_positions(w.seq_len, w.cp_size, w.rank)
    q = gen(w, "q", zigzag_chunks(w.cp_size, w.rank), w.heads_q)
    ref_o, ref_l = oracle.attention_rows(q.float().numpy(), kf, vf, zz, np.arange(w.seq_len), w.scale)
    tol_o, tol_l = TOL[w.dtype]
    res = {}
    for mode in ("single", "fused", "unfused"):
        _, out, lse = _ring_share(w, w.rank, ks, vs, mode)
        eo, el = max_abs(out.cpu().numpy(), ref_o), max_abs(lse.cpu().numpy(), ref_l)
        print(f"rank_share_8k ({mode}): max abs err O {eo:.3g}, lse {el:.3g}")
        assert eo <= tol_o and el <= tol_l, mode
        res[mode] = (out, lse)
    assert torch.equal(res["fused"][0], res["unfused"][0]) and torch.equal(res["fused"][1], res["unfused"][1])


def test_allgather_32k_reorder_then_attend():
    w = WORKLOADS["allgather_32k"]
    C = w.cp_size
    gather_ids = [c for r in range(C) for c in zigzag_chunks(C, r)]  # rank-order concatenation
    kg = gen(w, "k", gather_ids, w.heads_kv)
    vg = gen(w, "v", gather_ids, w.heads_kv)
    k_seq = cp.reorder_gathered(kg.to(DEV), C, cp.RANK_TO_SEQ)
    v_seq = cp.reorder_gathered(vg.to(DEV), C, cp.RANK_TO_SEQ)
    ref_k = oracle.reorder(kg.view(torch.int16).numpy(), C, 0)
    assert np.array_equal(k_seq.cpu().view(torch.int16).numpy(), ref_k)
    assert np.array_equal(v_seq.cpu().view(torch.int16).numpy(), oracle.reorder(vg.view(torch.int16).numpy(), C, 0))
    kf, vf = _full_kv_f32(w, w.heads_kv)  # oracle inputs straight from the generator
    gpos = torch.arange(w.seq_len, device=DEV)
    tol_o, tol_l = TOL[w.dtype]
    for r in range(C):
        q = gen(w, "q", zigzag_chunks(C, r), w.heads_q)
        zz = cp.zigzag_index(w.seq_len, C, r, device=DEV)
        out, lse = cp.block_fwd(q.to(DEV), k_seq, v_seq, zz, gpos, w.scale)
        rows = sample_rows(w.local_len, w.chunk_len, seed=r, per_chunk_random=8)
        ref_o, ref_l = oracle.attention_rows(q.float().numpy(), kf, vf,
                                             oracle.zigzag_positions(w.seq_len, C, r),
                                             np.arange(w.seq_len), w.scale, rows=rows)
        eo = max_abs(out[:, torch.from_numpy(rows).to(DEV)].cpu().numpy(), ref_o)
        el = max_abs(lse[:, :, torch.from_numpy(rows).to(DEV)].cpu().numpy(), ref_l)
        print(f"allgather_32k rank {r}: max abs err O {eo:.3g}, lse {el:.3g} over {len(rows)} rows")
        assert eo <= tol_o and el <= tol_l


def test_ulysses_gqa_128k_group():
    w = WORKLOADS["ulysses_gqa_128k"]
    C, g = w.cp_size, w.group
    s = w.local_len
    ids = range(2 * C)
    # contiguous sharding: rank src holds rows [src*s, (src+1)*s); stacked = [C, B, s, H, D]
    qfull = gen(w, "q", ids, w.heads_q)
    kfull = gen(w, "k", ids, w.heads_kv)
    vfull = gen(w, "v", ids, w.heads_kv)
    stack = lambda x: x.reshape(w.batch, C, s, *x.shape[2:]).transpose(0, 1).contiguous()
    qg = cp.ulysses_seq_to_heads(stack(qfull).to(DEV), g)
    kg = cp.ulysses_seq_to_heads(stack(kfull).to(DEV), g)
    vg = cp.ulysses_seq_to_heads(stack(vfull).to(DEV), g)
    hq, hk = w.heads_q // C, w.heads_kv // C
    assert torch.equal(qg.cpu(), qfull[:, :, g * hq:(g + 1) * hq])
    assert torch.equal(kg.cpu(), kfull[:, :, g * hk:(g + 1) * hk])
    pos = torch.arange(w.seq_len, device=DEV)
    og, lseg = cp.block_fwd(qg, kg, vg, pos, pos, w.scale)
    out_stacked = torch.zeros((C, w.batch, s, w.heads_q, w.head_dim), device=DEV)
    cp.ulysses_heads_to_seq(og, g, out_stacked)
    # inverse permute, bit for bit: the group's heads of every shard hold the group output
    back = out_stacked.transpose(0, 1).reshape(w.batch, w.seq_len, w.heads_q, w.head_dim)
    assert torch.equal(back[:, :, g * hq:(g + 1) * hq], og)
    assert torch.count_nonzero(back[:, :, :g * hq]) == 0
    rows = sample_rows(w.seq_len, w.chunk_len, seed=g, per_chunk_random=6)
    npos = np.arange(w.seq_len, dtype=np.int64)
    # oracle inputs straight from the generator: the group's heads of the full tensors
    ref_o, ref_l = oracle.attention_rows(qfull[:, :, g * hq:(g + 1) * hq].float().numpy(),
                                         kfull[:, :, g * hk:(g + 1) * hk].float().numpy(),
                                         vfull[:, :, g * hk:(g + 1) * hk].float().numpy(), npos, npos,
                                         w.scale, rows=rows)
    ridx = torch.from_numpy(rows).to(DEV)
    eo, el = max_abs(og[:, ridx].cpu().numpy(), ref_o), max_abs(lseg[:, :, ridx].cpu().numpy(), ref_l)
    print(f"ulysses_gqa_128k: max abs err O {eo:.3g}, lse {el:.3g} over {len(rows)} rows")
    tol_o, tol_l = TOL[w.dtype]
    assert eo <= tol_o and el <= tol_l
    # the exchanges folded into the attention's row addressing (the bench's --mode fused form):
    # the same bits in the same stacked output, the other groups' heads untouched
    out_rows = torch.zeros_like(out_stacked)
    og_r, lse_r = cp.ulysses_share_fwd(stack(qfull).to(DEV), stack(kfull).to(DEV), stack(vfull).to(DEV), g,
                                       w.scale, out_rows, zigzag=False)
    torch.cuda.synchronize()
    assert torch.equal(out_rows, out_stacked) and torch.equal(lse_r, lseg) and torch.equal(og_r, og)


def test_ring_share_256k_sampled():
    """Sampled rows of the long-context ring share against the oracle: the one-launch form
    and the ring's per-step forms (8 launches, the 7 merges fused into the epilogue or run
    by the merge kernel)."""
    w = WORKLOADS["ring_share_256k"]
    ks, vs = _owner_blocks(w, w.heads_kv)
    kf, vf = _full_kv_f32(w, w.heads_kv)
    zz = oracle.zigzag_positions(w.seq_len, w.cp_size, w.rank)
    q = gen(w, "q", zigzag_chunks(w.cp_size, w.rank), w.heads_q)
    rows = sample_rows(w.local_len, w.chunk_len, seed=w.rank, per_chunk_random=12)
    ref_o, ref_l = oracle.attention_rows(q.float().numpy(), kf, vf, zz, np.arange(w.seq_len), w.scale,
                                         rows=rows)
    del kf, vf
    ridx = torch.from_numpy(rows).to(DEV)
    tol_o, tol_l = TOL[w.dtype]
    for mode in ("single", "fused", "unfused"):
        _, out, lse = _ring_share(w, w.rank, ks, vs, mode)
        assert torch.isfinite(lse).all() and torch.isfinite(out).all()
        eo, el = max_abs(out[:, ridx].cpu().numpy(), ref_o), max_abs(lse[:, :, ridx].cpu().numpy(), ref_l)
        print(f"ring_share_256k ({mode}): max abs err O {eo:.3g}, lse {el:.3g} over {len(rows)} rows")
        assert eo <= tol_o and el <= tol_l, mode
        del out, lse
        torch.cuda.empty_cache()

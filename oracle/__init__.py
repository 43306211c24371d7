"""Plain fp64 CPU oracle for one context-parallel rank's share of causal attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The library under
``context_causal_attention_amd`` never imports it, and it imports nothing from there.

The arithmetic lives in ``oracle.c`` (plain loops, fp64, pthreads), loaded with ctypes.
This module adds argument marshalling plus three pieces of plain Python that follow
the pages step by step:

* ``ring_rank_share``: the ring forward of "On Context Parallelism", section
  "Peer-to-peer" / "Forward": for each step the K/V shard of owner (rank - step) mod C
  is attended with global positions and folded in with the pairwise LSE merge.
* ``closed_form_share``: the same blocks folded at once with the boxed combine of
  "Context parallelism -- splitting the sequence across GPUs", section "How do partial
  softmax results combine?".
* ``ring_rank_share_bwd``: the ring backward of "On Context Parallelism", section
  "Peer-to-peer" / "Backward": per step the block backward of the local queries against
  owner (rank - step) mod C's shard, dq summed over the steps, dk and dv kept per owner.
* the zigzag Ulysses exchange (the all-to-all's rank-order concatenation followed by the
  chunk reorder) and the two-dimensional mesh of "On Context Parallelism", section
  "Peer-to-peer + All-to-all" (group positions, rank coordinates, the group's share).
* the work models of "Context Parallelism & Ring Attention" ("The causal load-imbalance
  problem", "The zigzag fix") and of "Context parallelism: Ring Attention and Ulysses"
  ("The zigzag partition", "Ring Attention").

``block_bwd(..., bf16_pds=True)`` (with ``round_bf16``, its rounding) is not a step of the
pages, which fix no precision: it models a bf16 backward that rounds its two self-formed
product operands, p and ds, to bf16, so that such a kernel's rounding can be checked
exactly rather than only bounded.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "oracle.c"
_LIB_PATH = _HERE / "liboracle.so"
_lib = None


def build(force: bool = True) -> Path:
    """Compile oracle.c with gcc into liboracle.so (IEEE fp64, no fast-math)."""
    if force or not _LIB_PATH.exists():
        tmp = _LIB_PATH.with_suffix(".so.tmp")
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fno-fast-math", "-shared", "-fPIC", str(_SRC),
             "-o", str(tmp), "-lm", "-lpthread"],
            check=True,
        )
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not _LIB_PATH.exists():
        build(force=False)
    L = ctypes.CDLL(str(_LIB_PATH))
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    L.orc_zigzag_positions.argtypes = [i64, i32, i32, P]
    L.orc_contiguous_positions.argtypes = [i64, i32, i32, P]
    L.orc_gathered_positions.argtypes = [i64, i32, P]
    L.orc_reorder.argtypes = [P, P, i32, i64, i64, i32, i32]
    L.orc_ulysses_permute.argtypes = [P, P, i32, i32, i64, i32, i32, i32, i32, i32]
    L.orc_attention_rows.argtypes = [P, P, P, i32, i64, i64, i32, i32, i32, P, P, f64, P, i64,
                                     P, P, i32]
    L.orc_block_stats.argtypes = [P, P, P, i32, i64, i64, i32, i32, i32, P, P, f64, P, i64,
                                  P, P, P]
    L.orc_merge.argtypes = [P, P, P, P, i32, i64, i32, i32]
    L.orc_combine_blocks.argtypes = [P, P, P, i32, i64, i32, P, P]
    L.orc_block_bwd.argtypes = [P, P, P, P, P, P, i32, i64, i64, i32, i32, i32, P, P, f64, P, i64, P,
                                i64, P, P, P, i32, i32]
    L.orc_round_bf16.argtypes = [P, P, i64]
    for name in ("orc_zigzag_positions", "orc_contiguous_positions", "orc_gathered_positions",
                 "orc_reorder", "orc_ulysses_permute", "orc_attention_rows", "orc_block_stats",
                 "orc_merge", "orc_combine_blocks", "orc_block_bwd", "orc_round_bf16"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle: invalid arguments to {what}")


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


# ----------------------------------------------------------------------------------------
# Positions and layouts
# ----------------------------------------------------------------------------------------
def zigzag_positions(S: int, C: int, r: int) -> np.ndarray:
    out = np.empty(S // max(C, 1), dtype=np.int64)
    _check(_load().orc_zigzag_positions(S, C, r, _ptr(out)), "zigzag_positions")
    return out


def contiguous_positions(S: int, P: int, p: int) -> np.ndarray:
    out = np.empty(S // max(P, 1), dtype=np.int64)
    _check(_load().orc_contiguous_positions(S, P, p, _ptr(out)), "contiguous_positions")
    return out


def gathered_positions(S: int, C: int) -> np.ndarray:
    out = np.empty(S, dtype=np.int64)
    _check(_load().orc_gathered_positions(S, C, _ptr(out)), "gathered_positions")
    return out


def reorder(x: np.ndarray, C: int, direction: int) -> np.ndarray:
    """x: [B, S, ...] any dtype; rows are everything after the sequence axis."""
    x = np.ascontiguousarray(x)
    B, S = x.shape[0], x.shape[1]
    row_bytes = x.nbytes // (B * S)
    out = np.empty_like(x)
    _check(_load().orc_reorder(_ptr(x), _ptr(out), B, S, row_bytes, C, direction), "reorder")
    return out


def ulysses_seq_to_heads(stacked: np.ndarray, C: int, g: int) -> np.ndarray:
    """stacked: [C, B, S/C, H, D] -> group g's [B, S, H/C, D]."""
    x = np.ascontiguousarray(stacked)
    Cc, B, s, H, D = x.shape
    assert Cc == C
    out = np.empty((B, s * C, H // C, D), dtype=x.dtype)
    _check(_load().orc_ulysses_permute(_ptr(x), _ptr(out), x.itemsize, B, s * C, H, D, C, g, 0),
           "ulysses_permute")
    return out


def ulysses_heads_to_seq(grouped: np.ndarray, C: int, g: int, out: np.ndarray) -> np.ndarray:
    """grouped: [B, S, H/C, D] -> writes group g's heads of stacked out [C, B, S/C, H, D]."""
    x = np.ascontiguousarray(grouped)
    B, S, hg, D = x.shape
    assert out.flags.c_contiguous and out.shape == (C, B, S // C, hg * C, D) and out.dtype == x.dtype
    _check(_load().orc_ulysses_permute(_ptr(x), _ptr(out), x.itemsize, B, S, hg * C, D, C, g, 1),
           "ulysses_permute")
    return out


def ulysses_zigzag_seq_to_heads(stacked: np.ndarray, C: int, g: int) -> np.ndarray:
    """Zigzag shards [C, B, S/C, H, D] through the Ulysses exchange for head group g.

    "On Context Parallelism", section "All-to-all": the exchange concatenates the C shards
    in rank order; with zigzag shards that is the rank-order layout of section "All-gather"
    ([c0, c2C-1, c1, c2C-2, ...]), which the chunk reorder turns into global order."""
    return reorder(ulysses_seq_to_heads(stacked, C, g), C, 0)


def ulysses_zigzag_heads_to_seq(grouped: np.ndarray, C: int, g: int, out: np.ndarray) -> np.ndarray:
    """Inverse of ``ulysses_zigzag_seq_to_heads``: global order back to rank order, then the
    exchange back to group g's heads of the stacked shards ``out``."""
    return ulysses_heads_to_seq(reorder(grouped, C, 1), C, g, out)


# ----------------------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------------------
def _f32(a) -> np.ndarray:
    a = np.asarray(a)
    return np.ascontiguousarray(a, dtype=np.float32)


def attention_rows(q, k, v, q_pos, kv_pos, scale: float, rows=None, nthreads: int | None = None):
    """Direct causal attention (definition) for query rows ``rows`` (default: all).

    q [B,Sq,Hq,D]; k, v [B,Skv,Hkv,D] (fp32 values); positions int64.
    Returns out [B,len(rows),Hq,D] and lse [B,Hq,len(rows)], both fp64.
    """
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    assert k.shape == v.shape == (B, Skv, Hkv, D)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int64)
    kv_pos = np.ascontiguousarray(kv_pos, dtype=np.int64)
    assert q_pos.shape == (Sq,) and kv_pos.shape == (Skv,)
    rows = np.arange(Sq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.shape[0]
    out = np.zeros((B, n, Hq, D), dtype=np.float64)
    lse = np.zeros((B, Hq, n), dtype=np.float64)
    nt = default_threads() if nthreads is None else nthreads
    _check(_load().orc_attention_rows(_ptr(q), _ptr(k), _ptr(v), B, Sq, Skv, Hq, Hkv, D,
                                      _ptr(q_pos), _ptr(kv_pos), float(scale), _ptr(rows), n,
                                      _ptr(out), _ptr(lse), nt), "attention_rows")
    return out, lse


def block_stats(q, k, v, q_pos, kv_pos, scale: float, rows=None):
    """Unnormalised per-block statistics (m_r, l_r, z_r) for every selected row."""
    q, k, v = _f32(q), _f32(k), _f32(v)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int64)
    kv_pos = np.ascontiguousarray(kv_pos, dtype=np.int64)
    rows = np.arange(Sq, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.shape[0]
    m = np.zeros((B, Hq, n)); l = np.zeros((B, Hq, n)); z = np.zeros((B, n, Hq, D))
    _check(_load().orc_block_stats(_ptr(q), _ptr(k), _ptr(v), B, Sq, Skv, Hq, Hkv, D,
                                   _ptr(q_pos), _ptr(kv_pos), float(scale), _ptr(rows), n,
                                   _ptr(m), _ptr(l), _ptr(z)), "block_stats")
    return m, l, z


def merge(out, lse, out_t, lse_t):
    """Pairwise LSE merge; returns new arrays.  out [B,s,H,D], lse [B,H,s] (fp64)."""
    o = np.array(out, dtype=np.float64, order="C", copy=True)
    L = np.array(lse, dtype=np.float64, order="C", copy=True)
    ot = np.ascontiguousarray(out_t, dtype=np.float64)
    Lt = np.ascontiguousarray(lse_t, dtype=np.float64)
    B, s, H, D = o.shape
    assert L.shape == Lt.shape == (B, H, s) and ot.shape == o.shape
    _check(_load().orc_merge(_ptr(o), _ptr(L), _ptr(ot), _ptr(Lt), B, s, H, D), "merge")
    return o, L


def combine_blocks(m, l, z):
    """Closed-form combine.  m, l: [R, n]; z: [R, n, D] -> (out [n, D], lse [n])."""
    m = np.ascontiguousarray(m, dtype=np.float64)
    l = np.ascontiguousarray(l, dtype=np.float64)
    z = np.ascontiguousarray(z, dtype=np.float64)
    R, n = m.shape
    D = z.shape[2]
    out = np.zeros((n, D)); lse = np.zeros(n)
    _check(_load().orc_combine_blocks(_ptr(m), _ptr(l), _ptr(z), R, n, D, _ptr(out), _ptr(lse)),
           "combine_blocks")
    return out, lse


def round_bf16(x) -> np.ndarray:
    """Each value rounded to the nearest bf16 value, ties to even (``orc_round_bf16``)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    _check(_load().orc_round_bf16(_ptr(x), _ptr(y), x.size), "round_bf16")
    return y


def block_bwd(q, k, v, dout, out, lse, q_pos, kv_pos, scale: float, qrows=None, krows=None,
              nthreads: int | None = None, bf16_pds: bool = False):
    """Backward of one block (see ``orc_block_bwd``): returns (dq, dk, dv) in fp64 for the
    selected query rows (default all) and key rows (default all).  out and lse are the
    complete forward results of the query rows (fp64 or fp32 values).

    bf16_pds: a model of a bf16 backward that rounds the two operands it forms itself to
    bf16 before the products that use them: p (for dv) and ds = p (dp - D) (for dq and dk,
    formed from the unrounded p); everything else stays fp64."""
    q, k, v, dout = _f32(q), _f32(k), _f32(v), _f32(dout)
    out = np.ascontiguousarray(out, dtype=np.float64)
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    qp = np.ascontiguousarray(q_pos, dtype=np.int64)
    kp = np.ascontiguousarray(kv_pos, dtype=np.int64)
    qr = np.arange(Sq, dtype=np.int64) if qrows is None else np.ascontiguousarray(qrows, dtype=np.int64)
    kr = np.arange(Skv, dtype=np.int64) if krows is None else np.ascontiguousarray(krows, dtype=np.int64)
    dq = np.empty((B, len(qr), Hq, D))
    dk = np.empty((B, len(kr), Hkv, D))
    dv = np.empty((B, len(kr), Hkv, D))
    _check(_load().orc_block_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(out), _ptr(lse), B, Sq, Skv,
                                 Hq, Hkv, D, _ptr(qp), _ptr(kp), float(scale), _ptr(qr), len(qr), _ptr(kr),
                                 len(kr), _ptr(dq), _ptr(dk), _ptr(dv), 1 if bf16_pds else 0,
                                 nthreads or default_threads()), "block_bwd")
    return dq, dk, dv


# ----------------------------------------------------------------------------------------
# The ring, emulated step by step ("On Context Parallelism", "Peer-to-peer" / "Forward")
# ----------------------------------------------------------------------------------------
def owner_positions(S: int, C: int, owner: int, layout: str) -> np.ndarray:
    return zigzag_positions(S, C, owner) if layout == "zigzag" else contiguous_positions(S, C, owner)


def ring_rank_share(q_local, k_full, v_full, S: int, C: int, r: int, scale: float,
                    layout: str = "zigzag", rows=None, nthreads: int | None = None):
    """Rank r's share by the ring: step i attends the shard of owner (r - i) mod C.

    q_local [B, S/C, Hq, D] in the rank's local order; k_full, v_full [B, S, Hkv, D] in
    global order (the owner's shard is gathered from them by its positions).
    Returns (out, lse, blocks) where blocks[i] = (owner, tile_out, tile_lse).
    """
    q_pos = owner_positions(S, C, r, layout)
    out = lse = None
    blocks = []
    for step in range(C):
        owner = (r - step) % C
        kv_pos = owner_positions(S, C, owner, layout)
        kb = np.asarray(k_full)[:, kv_pos]
        vb = np.asarray(v_full)[:, kv_pos]
        t_out, t_lse = attention_rows(q_local, kb, vb, q_pos, kv_pos, scale, rows, nthreads)
        blocks.append((owner, t_out, t_lse))
        if out is None:  # the first completed tile is taken as is
            out, lse = t_out.copy(), t_lse.copy()
        else:
            out, lse = merge(out, lse, t_out, t_lse)
    return out, lse, blocks


def ring_rank_share_bwd(q_local, k_full, v_full, dout_local, out_local, lse_local, S: int, C: int,
                        r: int, scale: float, layout: str = "zigzag"):
    """Rank r's share of the ring backward: step i runs the block backward of the local
    queries against owner (r - i) mod C's shard with the saved (complete) out and lse;
    dq adds up over the steps, and each owner's dk, dv contribution is what travels with
    its K/V.  Returns (dq_local, {owner: (dk_o, dv_o)}) with dk_o, dv_o in the owner's
    local order."""
    q_pos = owner_positions(S, C, r, layout)
    dq = None
    contrib = {}
    for step in range(C):
        owner = (r - step) % C
        kv_pos = owner_positions(S, C, owner, layout)
        t_dq, t_dk, t_dv = block_bwd(q_local, np.asarray(k_full)[:, kv_pos], np.asarray(v_full)[:, kv_pos],
                                     dout_local, out_local, lse_local, q_pos, kv_pos, scale)
        dq = t_dq if dq is None else dq + t_dq
        contrib[owner] = (t_dk, t_dv)
    return dq, contrib


def closed_form_share(q_local, k_full, v_full, S: int, C: int, r: int, scale: float,
                      layout: str = "zigzag", rows=None):
    """Rank r's share by the boxed closed-form combine over all C owners' blocks."""
    q_pos = owner_positions(S, C, r, layout)
    ms, ls, zs = [], [], []
    for owner in range(C):
        kv_pos = owner_positions(S, C, owner, layout)
        m, l, z = block_stats(q_local, np.asarray(k_full)[:, kv_pos], np.asarray(v_full)[:, kv_pos],
                              q_pos, kv_pos, scale, rows)
        ms.append(m); ls.append(l); zs.append(z)
    B, Hq, n = ms[0].shape
    D = zs[0].shape[3]
    out = np.zeros((B, n, Hq, D)); lse = np.zeros((B, Hq, n))
    for b in range(B):
        for h in range(Hq):
            o, L = combine_blocks(np.stack([m[b, h] for m in ms]), np.stack([l[b, h] for l in ls]),
                                  np.stack([z[b, :, h] for z in zs]))
            out[b, :, h] = o
            lse[b, h] = L
    return out, lse


# ----------------------------------------------------------------------------------------
# Two-dimensional mesh ("On Context Parallelism", "Peer-to-peer + All-to-all")
# ----------------------------------------------------------------------------------------
def usp_rank_coords(r: int, A: int) -> tuple[int, int]:
    """Rank r of C = A*R: A2A groups are runs of A consecutive ranks ([0,1], [2,3], ... at
    A=2) and P2P groups collect the ranks at the same place in their A2A group ([0,2,4,6]
    and [1,3,5,7] at C=8, A=2).  Returns (A2A group = position in the P2P ring, place in
    the A2A group = head group)."""
    return r // A, r % A


def usp_groups(C: int, A: int) -> tuple[list[list[int]], list[list[int]]]:
    """(A2A groups, P2P groups) of C ranks, each group's ranks in increasing order."""
    a2a, p2p = {}, {}
    for r in range(C):
        g, a = usp_rank_coords(r, A)
        a2a.setdefault(g, []).append(r)
        p2p.setdefault(a, []).append(r)
    return [a2a[k] for k in sorted(a2a)], [p2p[k] for k in sorted(p2p)]


def group_positions(S: int, A: int, R: int, g: int) -> np.ndarray:
    """Global positions held by A2A group g after its exchange: the union of its A ranks'
    zigzag shards over C = A*R ranks, in increasing order."""
    C = A * R
    return np.sort(np.concatenate([zigzag_positions(S, C, g * A + j) for j in range(A)]))


def usp_rank_share(q_full, k_full, v_full, S: int, A: int, R: int, r: int, scale: float,
                   rows=None, nthreads: int | None = None):
    """Rank r's share on the mesh, by the definition: its A2A group's tokens (in increasing
    position order) and its head group (Hq/A query heads, Hkv/A kv heads) attend the whole
    sequence causally.  q_full [B, S, Hq, D], k_full and v_full [B, S, Hkv, D] in global
    order.  Returns (out [B, S/R, Hq/A, D], lse [B, Hq/A, S/R])."""
    g, a = usp_rank_coords(r, A)
    pos = group_positions(S, A, R, g)
    hq, hk = np.asarray(q_full).shape[2] // A, np.asarray(k_full).shape[2] // A
    q = np.asarray(q_full)[:, pos][:, :, a * hq:(a + 1) * hq]
    k = np.asarray(k_full)[:, :, a * hk:(a + 1) * hk]
    v = np.asarray(v_full)[:, :, a * hk:(a + 1) * hk]
    return attention_rows(q, k, v, pos, np.arange(S, dtype=np.int64), scale, rows, nthreads)


# ----------------------------------------------------------------------------------------
# Work models
# ----------------------------------------------------------------------------------------
def visible_pairs(q_pos, kv_pos) -> int:
    """Number of (query, key) pairs with kv position <= query position (exact count)."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    kv_sorted = np.sort(np.asarray(kv_pos, dtype=np.int64))
    return int(np.searchsorted(kv_sorted, q_pos, side="right").sum())


def block_work_diag_one(P: int, layout: str) -> list[float]:
    """"Context Parallelism & Ring Attention": work in causal key blocks, the diagonal
    block counted as one.  Contiguous: device p does p + 1 blocks.  Zigzag (2P chunks):
    chunk c costs c + 1 units and device p holds chunks p and 2P - 1 - p."""
    if layout == "contiguous":
        return [float(p + 1) for p in range(P)]
    return [float((p + 1) + (2 * P - 1 - p + 1)) for p in range(P)]


def chunk_work_diag_half(query_chunks) -> float:
    """"Context parallelism: Ring Attention and Ulysses", "The zigzag partition": a query
    chunk c attends c earlier KV chunks fully plus half of its own diagonal chunk."""
    return float(sum(c + 0.5 for c in query_chunks))


def contiguous_ring_blocks(P: int) -> list[int]:
    """Blocks a contiguous ring computes per rank when blocks from later ranks are skipped:
    rank r sees owners r, r-1, ..., and computes those not later than itself."""
    counts = []
    for r in range(P):
        counts.append(sum(1 for step in range(P) if (r - step) % P <= r))
    return counts

"""ctypes binding of libcpattn.so: argument marshalling only.

Every function checks devices, dtypes, shapes and contiguity, passes raw device pointers
and the current HIP stream to the C ABI (include/cpattn.h), and raises CpattnError on a
non-zero status.  PyTorch supplies device memory and streams; all arithmetic happens in
the library's kernels.  There is no fallback: without the built library every call fails.
"""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

import torch

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libcpattn.so"
HEADER = _PKG.parent / "include" / "cpattn.h"

CPATTN_F32, CPATTN_BF16 = 0, 1
BWD_WRITE_DQ, BWD_WRITE_DKV = 1, 2
RANK_TO_SEQ, SEQ_TO_RANK = 0, 1
SEQ_TO_HEADS, HEADS_TO_SEQ = 0, 1
STATUS = {0: "CPATTN_OK", 1: "CPATTN_ERR_INVALID_ARG", 2: "CPATTN_ERR_SHAPE",
          3: "CPATTN_ERR_UNSUPPORTED", 4: "CPATTN_ERR_HIP"}

_lib = None


class CpattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def library_path() -> Path:
    return LIB_PATH


def load_library():
    """Load libcpattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m context_causal_attention_amd.build`")
    L = ctypes.CDLL(str(LIB_PATH))
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    L.cpattn_status_string.argtypes = [ctypes.c_int]
    L.cpattn_status_string.restype = ctypes.c_char_p
    L.cpattn_last_error.argtypes = []
    L.cpattn_last_error.restype = ctypes.c_char_p
    L.cpattn_abi_version.argtypes = []
    L.cpattn_abi_version.restype = i32
    L.cpattn_zigzag_index.argtypes = [i64, i32, i32, P, P]
    L.cpattn_zigzag_index_all.argtypes = [i64, i32, P, P]
    L.cpattn_block_fwd.argtypes = [P, P, P, ctypes.c_int, i32, i64, i64, i32, i32, i32, P, P, f32, P, P, P]
    L.cpattn_block_fwd_merge.argtypes = list(L.cpattn_block_fwd.argtypes)
    L.cpattn_block_fwd_rows.argtypes = [P, i64, P, P, i64, i64, i64, i32, i32, i32, P, P, f32, P, i64, P, P]
    L.cpattn_lse_merge.argtypes = [P, P, P, P, i32, i64, i32, i32, P]
    L.cpattn_ring_share_fwd.argtypes = [P, P, P, P, P, i32, ctypes.c_int, i32, i64, i32, i32, i32, P, f32, P, P, P]
    L.cpattn_attn_bwd_delta.argtypes = [P, P, ctypes.c_int, i32, i64, i32, i32, P, P]
    L.cpattn_block_bwd.argtypes = [P, P, P, P, ctypes.c_int, i32, i64, i64, i32, i32, i32, P, P, f32, P, P, P,
                                   P, P, ctypes.c_uint32, P]
    L.cpattn_ring_share_bwd.argtypes = [P, P, P, P, P, P, i32, ctypes.c_int, i32, i64, i32, i32, i32, P, f32, P, P,
                                        P, P, P, P]
    L.cpattn_reorder_gathered.argtypes = [P, P, i32, i64, i64, i32, ctypes.c_int, P]
    L.cpattn_ulysses_permute.argtypes = [P, P, i32, i32, i64, i32, i32, i32, i32, ctypes.c_int, P]
    L.cpattn_ulysses_permute_zigzag.argtypes = list(L.cpattn_ulysses_permute.argtypes)
    for name in ("cpattn_zigzag_index", "cpattn_zigzag_index_all", "cpattn_block_fwd", "cpattn_block_fwd_merge", "cpattn_block_fwd_rows",
                 "cpattn_lse_merge",
                 "cpattn_attn_bwd_delta", "cpattn_block_bwd", "cpattn_ring_share_fwd", "cpattn_ring_share_bwd",
                 "cpattn_reorder_gathered", "cpattn_ulysses_permute", "cpattn_ulysses_permute_zigzag"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def header_entry_points() -> list[str]:
    """Names of the functions declared in include/cpattn.h."""
    text = HEADER.read_text()
    return sorted(set(re.findall(r"\b(cpattn_[a-z0-9_]+)\s*\(", text)))


def _check(status: int):
    if status != 0:
        msg = load_library().cpattn_last_error().decode(errors="replace")
        raise CpattnError(status, msg)


def _ptr(t: torch.Tensor | None):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


def zigzag_index(seq_len: int, cp_size: int, rank: int, out: torch.Tensor | None = None,
                 device=None) -> torch.Tensor:
    """Global positions of rank ``rank``'s local tokens (int64 [seq_len / cp_size])."""
    L = load_library()
    if out is None:
        out = torch.empty(seq_len // max(cp_size, 1), dtype=torch.int64,
                          device=device if device is not None else torch.device("cuda"))
    _need(out, "out", torch.int64)
    _check(L.cpattn_zigzag_index(seq_len, cp_size, rank, _ptr(out), _stream(out.device)))
    return out


def zigzag_index_all(seq_len: int, cp_size: int, out: torch.Tensor | None = None,
                     device=None) -> torch.Tensor:
    """Every rank's zigzag positions in one launch: int64 [cp_size, seq_len / cp_size], row r
    being rank r's local tokens."""
    L = load_library()
    n = seq_len // max(cp_size, 1)
    if out is None:
        out = torch.empty((max(cp_size, 1), n), dtype=torch.int64,
                          device=device if device is not None else torch.device("cuda"))
    _need(out, "out", torch.int64, shape=(cp_size, n))
    _check(L.cpattn_zigzag_index_all(seq_len, cp_size, _ptr(out), _stream(out.device)))
    return out


def _block_fwd_call(entry: str, q, k, v, q_pos, kv_pos, scale, out, lse, alloc: bool):
    L = load_library()
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be bf16 or fp32")
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    _need(q, "q")
    _need(k, "k", q.dtype, (B, Skv, Hkv, D))
    _need(v, "v", q.dtype, (B, Skv, Hkv, D))
    _need(q_pos, "q_pos", torch.int64, (Sq,))
    _need(kv_pos, "kv_pos", torch.int64, (Skv,))
    if alloc and out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=torch.float32, device=q.device)
    if alloc and lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, Sq, Hq, D))
    _need(lse, "lse", torch.float32, (B, Hq, Sq))
    dt = CPATTN_BF16 if q.dtype == torch.bfloat16 else CPATTN_F32
    _check(getattr(L, entry)(_ptr(q), _ptr(k), _ptr(v), dt, B, Sq, Skv, Hq, Hkv, D, _ptr(q_pos),
                             _ptr(kv_pos), float(scale), _ptr(out), _ptr(lse), _stream(q.device)))
    return out, lse


def block_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_pos: torch.Tensor,
              kv_pos: torch.Tensor, scale: float, out: torch.Tensor | None = None,
              lse: torch.Tensor | None = None):
    """One block of causal attention on global positions.

    q [B, Sq, Hq, D]; k, v [B, Skv, Hkv, D] (both bf16 or both fp32); positions int64.
    Returns (out fp32 [B, Sq, Hq, D], lse fp32 [B, Hq, Sq]).
    """
    return _block_fwd_call("cpattn_block_fwd", q, k, v, q_pos, kv_pos, scale, out, lse, alloc=True)


def _rows_view(t: torch.Tensor, name: str, dtype, heads: int | None = None):
    """A [rows, heads, D] view whose rows may be strided; heads and head dims dense."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype or t.dim() != 3:
        raise ValueError(f"{name} must be a 3-d {dtype} view [rows, heads, head_dim]")
    if heads is not None and t.shape[1] != heads:
        raise ValueError(f"{name} must have {heads} heads (got {t.shape[1]})")
    if t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name}: heads and head dims must be dense within a row")
    return t.stride(0)


def block_fwd_rows(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_pos: torch.Tensor,
                   kv_pos: torch.Tensor, scale: float, out: torch.Tensor, lse: torch.Tensor | None = None):
    """cpattn_block_fwd_rows: bf16 block attention (batch 1) on row views.

    q [Sq, Hq, D], k, v [Skv, Hkv, D] (bf16; D = 64 or 128) and out [Sq, Hq, D] (fp32) are views whose
    rows (dim 0) may be strided, e.g. one head group of a stacked buffer; within a row the
    heads and head dims are dense.  Writes out in place; returns (out, lse [1, Hq, Sq]).
    """
    L = load_library()
    Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[0], k.shape[1]
    qs = _rows_view(q, "q", torch.bfloat16)
    ks = _rows_view(k, "k", torch.bfloat16)
    if _rows_view(v, "v", torch.bfloat16, Hkv) != ks or v.shape[0] != Skv:
        raise ValueError("v must have k's shape and row stride")
    os_ = _rows_view(out, "out", torch.float32, Hq)
    if out.shape[0] != Sq:
        raise ValueError("out must have q's rows")
    _need(q_pos, "q_pos", torch.int64, (Sq,))
    _need(kv_pos, "kv_pos", torch.int64, (Skv,))
    if lse is None:
        lse = torch.empty((1, Hq, Sq), dtype=torch.float32, device=q.device)
    _need(lse, "lse", torch.float32, (1, Hq, Sq))
    _check(L.cpattn_block_fwd_rows(_ptr(q), qs, _ptr(k), _ptr(v), ks, Sq, Skv, Hq, Hkv, D, _ptr(q_pos),
                                   _ptr(kv_pos), float(scale), _ptr(out), os_, _ptr(lse), _stream(q.device)))
    return out, lse


def block_fwd_merge(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, q_pos: torch.Tensor,
                    kv_pos: torch.Tensor, scale: float, out: torch.Tensor, lse: torch.Tensor):
    """``block_fwd`` merged in place into the accumulator (out, lse); returns (out, lse)."""
    if out is None or lse is None:
        raise ValueError("block_fwd_merge needs the accumulator tensors out and lse")
    return _block_fwd_call("cpattn_block_fwd_merge", q, k, v, q_pos, kv_pos, scale, out, lse, alloc=False)


def lse_merge(out: torch.Tensor, lse: torch.Tensor, out_tile: torch.Tensor, lse_tile: torch.Tensor):
    """Fold (out_tile, lse_tile) into (out, lse) in place; returns (out, lse)."""
    L = load_library()
    B, S, H, D = out.shape
    _need(out, "out", torch.float32)
    _need(lse, "lse", torch.float32, (B, H, S))
    _need(out_tile, "out_tile", torch.float32, (B, S, H, D))
    _need(lse_tile, "lse_tile", torch.float32, (B, H, S))
    _check(L.cpattn_lse_merge(_ptr(out), _ptr(lse), _ptr(out_tile), _ptr(lse_tile), B, S, H, D,
                              _stream(out.device)))
    return out, lse


def reorder_gathered(x: torch.Tensor, cp_size: int, direction: int = RANK_TO_SEQ,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """Chunk reorder of x [B, S, ...] between all-gather rank order and sequence order."""
    L = load_library()
    _need(x, "x")
    if out is None:
        out = torch.empty_like(x)
    _need(out, "out", x.dtype, tuple(x.shape))
    B, S = x.shape[0], x.shape[1]
    row_bytes = x.numel() * x.element_size() // max(B * S, 1)
    _check(L.cpattn_reorder_gathered(_ptr(x), _ptr(out), B, S, row_bytes, cp_size, direction,
                                     _stream(x.device)))
    return out


def ulysses_seq_to_heads(stacked: torch.Tensor, group: int, out: torch.Tensor | None = None,
                         zigzag: bool = False) -> torch.Tensor:
    """Stacked rank shards [C, B, S/C, H, D] -> head group ``group``'s [B, S, H/C, D].

    ``zigzag``: the shards are zigzag (rank src holds chunks src and 2C-1-src) and the
    result is in global sequence order; otherwise shards are contiguous."""
    L = load_library()
    _need(stacked, "stacked")
    C, B, s, H, D = stacked.shape
    if out is None:
        out = torch.empty((B, s * C, H // C, D), dtype=stacked.dtype, device=stacked.device)
    _need(out, "out", stacked.dtype, (B, s * C, H // C, D))
    fn = L.cpattn_ulysses_permute_zigzag if zigzag else L.cpattn_ulysses_permute
    _check(fn(_ptr(stacked), _ptr(out), stacked.element_size(), B, s * C, H, D, C, group, SEQ_TO_HEADS,
              _stream(stacked.device)))
    return out


def ulysses_heads_to_seq(grouped: torch.Tensor, group: int, out: torch.Tensor,
                         zigzag: bool = False) -> torch.Tensor:
    """Head group ``group``'s [B, S, H/C, D] -> its heads of stacked out [C, B, S/C, H, D]
    (``zigzag`` as in ``ulysses_seq_to_heads``)."""
    L = load_library()
    _need(grouped, "grouped")
    _need(out, "out", grouped.dtype)
    C, B, s, H, D = out.shape
    if tuple(grouped.shape) != (B, s * C, H // C, D):
        raise ValueError(f"grouped must have shape {(B, s * C, H // C, D)}")
    fn = L.cpattn_ulysses_permute_zigzag if zigzag else L.cpattn_ulysses_permute
    _check(fn(_ptr(grouped), _ptr(out), grouped.element_size(), B, s * C, H, D, C, group, HEADS_TO_SEQ,
              _stream(grouped.device)))
    return out


def ring_blocks_fwd(q: torch.Tensor, k_blocks, v_blocks, kv_positions, q_pos: torch.Tensor, scale: float,
                    out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """One launch over K/V blocks taken in the given order (cpattn_ring_share_fwd):
    q [B, Sq, Hq, D]; k_blocks[o], v_blocks[o] [B, S_o, Hkv, D]; kv_positions[o] [S_o]."""
    L = load_library()
    n = len(k_blocks)
    if not (len(v_blocks) == len(kv_positions) == n):
        raise ValueError("k_blocks, v_blocks and kv_positions must have the same length")
    B, Sq, Hq, D = q.shape
    _need(q, "q")
    _need(q_pos, "q_pos", torch.int64, (Sq,))
    Hkv = k_blocks[0].shape[2]
    for o in range(n):
        So = k_blocks[o].shape[1]
        _need(k_blocks[o], f"k_blocks[{o}]", q.dtype, (B, So, Hkv, D))
        _need(v_blocks[o], f"v_blocks[{o}]", q.dtype, (B, So, Hkv, D))
        _need(kv_positions[o], f"kv_positions[{o}]", torch.int64, (So,))
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, (B, Sq, Hq, D))
    _need(lse, "lse", torch.float32, (B, Hq, Sq))
    kp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in k_blocks])
    vp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in v_blocks])
    pp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in kv_positions])
    sq = (ctypes.c_int64 * n)(*[t.shape[1] for t in k_blocks])
    dt = CPATTN_BF16 if q.dtype == torch.bfloat16 else CPATTN_F32
    _check(L.cpattn_ring_share_fwd(_ptr(q), kp, vp, pp, sq, n, dt, B, Sq, Hq, Hkv, D, _ptr(q_pos), float(scale),
                                   _ptr(out), _ptr(lse), _stream(q.device)))
    return out, lse


def ring_share_fwd(q: torch.Tensor, k_blocks, v_blocks, positions, rank: int, scale: float,
                   out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                   tile_out: torch.Tensor | None = None, tile_lse: torch.Tensor | None = None,
                   mode: str = "single"):
    """Rank ``rank``'s share over the C ring steps, on the current stream.

    Step i attends the K/V block of owner (rank - i) mod C ("On Context Parallelism",
    Peer-to-peer / Forward): ``k_blocks[o]``, ``v_blocks[o]`` and ``positions[o]`` are owner
    o's shard and its global positions; ``positions[rank]`` are also the query positions.
    ``mode``:
      "single"  one launch over all C blocks in ring order (one running softmax);
      "fused"   one launch per step, steps >= 1 merged into (out, lse) in the epilogue;
      "unfused" one launch per step into a tile (``tile_out``, ``tile_lse``), then the merge
                kernel.  "fused" and "unfused" give the same bits.
    Returns (out, lse)."""
    C = len(k_blocks)
    B, s, Hq, D = q.shape
    order = [(rank - step) % C for step in range(C)]
    if mode == "single":
        return ring_blocks_fwd(q, [k_blocks[o] for o in order], [v_blocks[o] for o in order],
                               [positions[o] for o in order], positions[rank], scale, out, lse)
    if mode not in ("fused", "unfused"):
        raise ValueError(f"unknown mode {mode!r}")
    if out is None:
        out = torch.empty((B, s, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, s), dtype=torch.float32, device=q.device)
    if C > 1 and mode == "unfused":
        if tile_out is None:
            tile_out = torch.empty_like(out)
        if tile_lse is None:
            tile_lse = torch.empty_like(lse)
    for step, owner in enumerate(order):
        args = (q, k_blocks[owner], v_blocks[owner], positions[rank], positions[owner], scale)
        if step == 0:
            block_fwd(*args, out, lse)
        elif mode == "fused":
            block_fwd_merge(*args, out, lse)
        else:
            block_fwd(*args, tile_out, tile_lse)
            lse_merge(out, lse, tile_out, tile_lse)
    return out, lse


def ulysses_share_fwd(q_st: torch.Tensor, k_st: torch.Tensor, v_st: torch.Tensor, group: int,
                      scale: float, out_st: torch.Tensor, zigzag: bool = True, fused: bool | None = None):
    """Head group ``group``'s share of Ulysses attention from the stacked rank shards
    [C, B, S/C, H, D] of Q, K and V ("On Context Parallelism", All-to-all): the
    sequence-to-heads exchange (zigzag shards: with the chunk reorder folded in), causal
    attention over the whole sequence on global positions, and the inverse exchange of the
    output into the group's heads of ``out_st`` (fp32 [C, B, S/C, Hq, D]).
    Returns (out_grouped [B, S, Hq/C, D], lse [B, Hq/C, S]).

    ``fused`` (default: whenever possible, i.e. B = 1, contiguous shards, bf16, D = 64 or 128): with
    one batch and contiguous shards, global row i of the group is row i of the stacked buffer
    at the group's head offset, so the attention reads Q, K, V in place and writes out_st
    directly (cpattn_block_fwd_rows), with the same bits as the explicit exchanges; out_grouped
    is then a view into out_st."""
    C, B, s, Hq, D = q_st.shape
    S = s * C
    if fused is None:
        fused = (B == 1 and not zigzag and q_st.dtype == torch.bfloat16 and D in (64, 128)
                 and all(t.is_contiguous() for t in (q_st, k_st, v_st, out_st)))
    if fused:
        Hkv = k_st.shape[3]
        hq, hk = Hq // C, Hkv // C
        qv = q_st.view(S, Hq, D)[:, group * hq:(group + 1) * hq]
        kv = k_st.view(S, Hkv, D)[:, group * hk:(group + 1) * hk]
        vv = v_st.view(S, Hkv, D)[:, group * hk:(group + 1) * hk]
        ov = out_st.view(S, Hq, D)[:, group * hq:(group + 1) * hq]
        pos = zigzag_index(S, 1, 0, device=q_st.device)  # 0 .. S-1: global order
        _, lse = block_fwd_rows(qv, kv, vv, pos, pos, scale, ov)
        return ov.unsqueeze(0), lse
    qg = ulysses_seq_to_heads(q_st, group, zigzag=zigzag)
    kg = ulysses_seq_to_heads(k_st, group, zigzag=zigzag)
    vg = ulysses_seq_to_heads(v_st, group, zigzag=zigzag)
    pos = zigzag_index(S, 1, 0, device=q_st.device)  # 0 .. S-1: global order
    og, lse = block_fwd(qg, kg, vg, pos, pos, scale)
    ulysses_heads_to_seq(og, group, out_st, zigzag=zigzag)
    return og, lse


def usp_share_fwd(q_st: torch.Tensor, k_sts, v_sts, ring_rank: int, head_group: int, scale: float,
                  out_st: torch.Tensor):
    """One rank's share of the two-dimensional mesh ("On Context Parallelism", Peer-to-peer
    + All-to-all): C = A*R ranks, A2A groups of A consecutive ranks, P2P rings of the R ranks
    that hold the same head group.

    ``q_st`` is this rank's A2A group's stacked zigzag shards [A, B, S/C, Hq, D];
    ``k_sts[o]`` and ``v_sts[o]`` are A2A group o's stacked shards of K and V, for every
    group o of the ring.  The group's exchange (zigzag, head group ``head_group``) gives
    [B, S/R, H/A, D] in increasing position order, which are exactly the positions of rank
    ``ring_rank`` of a zigzag partition of S over R; the ring share then runs over the R
    owners, and the inverse exchange writes the output into ``out_st`` (fp32
    [A, B, S/C, Hq, D]).  Returns (out [B, S/R, Hq/A, D], lse [B, Hq/A, S/R])."""
    A, B, s, _, _ = q_st.shape
    R = len(k_sts)
    S = s * A * R
    qh = ulysses_seq_to_heads(q_st, head_group, zigzag=True)
    kh = [ulysses_seq_to_heads(k, head_group, zigzag=True) for k in k_sts]
    vh = [ulysses_seq_to_heads(v, head_group, zigzag=True) for v in v_sts]
    pos = list(zigzag_index_all(S, R, device=q_st.device).unbind(0))  # every owner's, one launch
    out, lse = ring_share_fwd(qh, kh, vh, pos, ring_rank, scale)
    ulysses_heads_to_seq(out, head_group, out_st, zigzag=True)
    return out, lse


def attn_bwd_delta(out: torch.Tensor, dout: torch.Tensor, delta: torch.Tensor | None = None) -> torch.Tensor:
    """delta [B, H, S] = <dout, out> per row; out fp32 [B, S, H, D], dout bf16 or fp32."""
    L = load_library()
    B, S, H, D = out.shape
    _need(out, "out", torch.float32)
    _need(dout, "dout", None, (B, S, H, D))
    if dout.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("dout must be bf16 or fp32")
    if delta is None:
        delta = torch.empty((B, H, S), dtype=torch.float32, device=out.device)
    _need(delta, "delta", torch.float32, (B, H, S))
    dt = CPATTN_BF16 if dout.dtype == torch.bfloat16 else CPATTN_F32
    _check(L.cpattn_attn_bwd_delta(_ptr(out), _ptr(dout), dt, B, S, H, D, _ptr(delta), _stream(out.device)))
    return delta


def block_bwd(q, k, v, dout, q_pos, kv_pos, scale: float, lse, delta, dq, dk, dv, flags: int = 0):
    """Backward of one block, added into dq [B, Sq, Hq, D], dk and dv [B, Skv, Hkv, D] (fp32);
    ``flags`` BWD_WRITE_DQ / BWD_WRITE_DKV overwrite instead of adding."""
    L = load_library()
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be bf16 or fp32")
    B, Sq, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    _need(q, "q")
    _need(k, "k", q.dtype, (B, Skv, Hkv, D))
    _need(v, "v", q.dtype, (B, Skv, Hkv, D))
    _need(dout, "dout", q.dtype, (B, Sq, Hq, D))
    _need(q_pos, "q_pos", torch.int64, (Sq,))
    _need(kv_pos, "kv_pos", torch.int64, (Skv,))
    _need(lse, "lse", torch.float32, (B, Hq, Sq))
    _need(delta, "delta", torch.float32, (B, Hq, Sq))
    _need(dq, "dq", torch.float32, (B, Sq, Hq, D))
    _need(dk, "dk", torch.float32, (B, Skv, Hkv, D))
    _need(dv, "dv", torch.float32, (B, Skv, Hkv, D))
    dt = CPATTN_BF16 if q.dtype == torch.bfloat16 else CPATTN_F32
    _check(L.cpattn_block_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), dt, B, Sq, Skv, Hq, Hkv, D, _ptr(q_pos),
                              _ptr(kv_pos), float(scale), _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk), _ptr(dv),
                              int(flags), _stream(q.device)))
    return dq, dk, dv


def ring_blocks_bwd(q, dout, k_blocks, v_blocks, kv_positions, q_pos, scale: float, lse, delta, dq, dk_blocks,
                    dv_blocks):
    """The backward against K/V blocks in one call (cpattn_ring_share_bwd): dq written with the
    sum over the blocks, dk_blocks[o] and dv_blocks[o] written with block o's parts."""
    L = load_library()
    n = len(k_blocks)
    if not (len(v_blocks) == len(kv_positions) == len(dk_blocks) == len(dv_blocks) == n):
        raise ValueError("the block lists must have the same length")
    B, Sq, Hq, D = q.shape
    _need(q, "q")
    _need(dout, "dout", q.dtype, (B, Sq, Hq, D))
    _need(q_pos, "q_pos", torch.int64, (Sq,))
    _need(lse, "lse", torch.float32, (B, Hq, Sq))
    _need(delta, "delta", torch.float32, (B, Hq, Sq))
    _need(dq, "dq", torch.float32, (B, Sq, Hq, D))
    Hkv = k_blocks[0].shape[2]
    for o in range(n):
        So = k_blocks[o].shape[1]
        _need(k_blocks[o], f"k_blocks[{o}]", q.dtype, (B, So, Hkv, D))
        _need(v_blocks[o], f"v_blocks[{o}]", q.dtype, (B, So, Hkv, D))
        _need(kv_positions[o], f"kv_positions[{o}]", torch.int64, (So,))
        _need(dk_blocks[o], f"dk_blocks[{o}]", torch.float32, (B, So, Hkv, D))
        _need(dv_blocks[o], f"dv_blocks[{o}]", torch.float32, (B, So, Hkv, D))
    arr = lambda ts: (ctypes.c_void_p * n)(*[t.data_ptr() for t in ts])  # noqa: E731
    sq = (ctypes.c_int64 * n)(*[t.shape[1] for t in k_blocks])
    dt = CPATTN_BF16 if q.dtype == torch.bfloat16 else CPATTN_F32
    _check(L.cpattn_ring_share_bwd(_ptr(q), _ptr(dout), arr(k_blocks), arr(v_blocks), arr(kv_positions), sq, n, dt, B,
                                   Sq, Hq, Hkv, D, _ptr(q_pos), float(scale), _ptr(lse), _ptr(delta), _ptr(dq),
                                   arr(dk_blocks), arr(dv_blocks), _stream(q.device)))
    return dq, dk_blocks, dv_blocks


def ring_share_bwd(q, k_blocks, v_blocks, positions, rank: int, scale: float, out, lse, dout,
                   dq=None, dk_blocks=None, dv_blocks=None, mode: str = "single"):
    """Rank ``rank``'s share of the ring backward ("On Context Parallelism", Peer-to-peer /
    Backward): delta once, then for each step the block backward against owner
    (rank - step) mod C's K/V; dq adds up over the steps, and owner o's dk and dv
    contributions go into ``dk_blocks[o]``, ``dv_blocks[o]`` (the buffers that travel with
    its K/V on a ring).  Step 0 writes dq and each owner's dk, dv are written by its one step,
    so nothing needs clearing first.  ``mode``: "single" (cpattn_ring_share_bwd: the dq
    launches per step and one dk/dv launch over all blocks) or "steps" (cpattn_block_bwd per
    step); both give the same bits.  Returns (dq, dk_blocks, dv_blocks)."""
    C = len(k_blocks)
    B, s, Hq, D = q.shape
    if dq is None:
        dq = torch.empty((B, s, Hq, D), dtype=torch.float32, device=q.device)
    if dk_blocks is None:
        dk_blocks = [torch.empty(k.shape, dtype=torch.float32, device=q.device) for k in k_blocks]
    if dv_blocks is None:
        dv_blocks = [torch.empty(v.shape, dtype=torch.float32, device=q.device) for v in v_blocks]
    delta = attn_bwd_delta(out, dout)
    order = [(rank - step) % C for step in range(C)]
    if mode == "single":
        ring_blocks_bwd(q, dout, [k_blocks[o] for o in order], [v_blocks[o] for o in order],
                        [positions[o] for o in order], positions[rank], scale, lse, delta, dq,
                        [dk_blocks[o] for o in order], [dv_blocks[o] for o in order])
        return dq, dk_blocks, dv_blocks
    if mode != "steps":
        raise ValueError(f"unknown mode {mode!r}")
    for step, owner in enumerate(order):
        flags = BWD_WRITE_DKV | (BWD_WRITE_DQ if step == 0 else 0)
        block_bwd(q, k_blocks[owner], v_blocks[owner], dout, positions[rank], positions[owner], scale, lse,
                  delta, dq, dk_blocks[owner], dv_blocks[owner], flags)
    return dq, dk_blocks, dv_blocks

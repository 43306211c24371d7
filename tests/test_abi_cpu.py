"""The C ABI without a GPU: the library loads, exports exactly what include/cpattn.h
declares, and rejects every malformed call on the host before any HIP call."""
from __future__ import annotations

import ctypes
import subprocess

import pytest

import context_causal_attention_amd as cp
from context_causal_attention_amd._binding import STATUS

OK, INVALID, SHAPE, UNSUPPORTED = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    return cp.load_library()


def test_exports_match_header(lib):
    declared = cp.header_entry_points()
    out = subprocess.run(["nm", "-D", "--defined-only", str(cp.library_path())], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted({line.split()[-1] for line in out.splitlines() if line.split()[-2:-1] == ["T"]
                       and line.split()[-1].startswith("cpattn_")})
    assert exported == declared
    for name in declared:
        assert hasattr(lib, name)


def test_status_strings(lib):
    for code, name in STATUS.items():
        assert lib.cpattn_status_string(code).decode() == name
    assert lib.cpattn_abi_version() == 1


def _err(lib):
    return lib.cpattn_last_error().decode()


def test_zigzag_validation(lib):
    f = lib.cpattn_zigzag_index
    assert f(30, 4, 0, FAKE, NULL) == SHAPE and "divisible" in _err(lib)
    assert f(32, 4, 4, FAKE, NULL) == INVALID
    assert f(32, 4, -1, FAKE, NULL) == INVALID
    assert f(32, 0, 0, FAKE, NULL) == INVALID
    assert f(0, 4, 0, FAKE, NULL) == INVALID
    assert f(32, 4, 0, NULL, NULL) == INVALID
    g = lib.cpattn_zigzag_index_all
    assert g(30, 4, FAKE, NULL) == SHAPE and "divisible" in _err(lib)
    assert g(32, 0, FAKE, NULL) == INVALID
    assert g(0, 4, FAKE, NULL) == INVALID
    assert g(32, 4, NULL, NULL) == INVALID
    assert g(1 << 20, 65536, FAKE, NULL) == UNSUPPORTED  # one grid row per rank


def _bf(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, batch=1, seq_q=64, seq_kv=64, hq=4, hkv=2, d=128,
             qpos=FAKE, kvpos=FAKE, scale=0.1, out=FAKE, lse=FAKE)
    a.update(kw)
    return lib.cpattn_block_fwd(a["q"], a["k"], a["v"], a["dtype"], a["batch"], a["seq_q"], a["seq_kv"],
                                a["hq"], a["hkv"], a["d"], a["qpos"], a["kvpos"], a["scale"], a["out"],
                                a["lse"], NULL)


def test_block_fwd_validation(lib):
    assert _bf(lib, dtype=7) == INVALID
    assert _bf(lib, batch=0) == INVALID
    assert _bf(lib, hq=0) == INVALID
    assert _bf(lib, seq_q=-1) == INVALID
    assert _bf(lib, scale=0.0) == INVALID
    assert _bf(lib, scale=-1.0) == INVALID
    assert _bf(lib, scale=float("inf")) == INVALID
    assert _bf(lib, scale=float("nan")) == INVALID
    assert _bf(lib, hq=6, hkv=4) == SHAPE and "multiple" in _err(lib)
    assert _bf(lib, d=96) == UNSUPPORTED
    # bf16 takes D = 64 as well as 128: such a call gets past the head-dim check to the
    # pointer checks
    assert _bf(lib, d=64, dtype=1, q=NULL) == INVALID
    # the bf16 kernels form tile offsets in 32 bits: a K/V row of more than 2^24 elements is
    # refused, whatever the head dim
    assert _bf(lib, hq=(1 << 17) + 1, hkv=(1 << 17) + 1, d=128) == UNSUPPORTED and "2^24" in _err(lib)
    assert _bf(lib, hq=(1 << 18) + 1, hkv=(1 << 18) + 1, d=64) == UNSUPPORTED and "2^24" in _err(lib)
    assert _bf(lib, hq=(1 << 18), hkv=(1 << 18), d=64, q=NULL) == INVALID  # 2^24 exactly is allowed
    # the fp32 path has no such bound
    assert _bf(lib, hq=(1 << 17) + 1, hkv=(1 << 17) + 1, d=128, dtype=0, q=NULL) == INVALID
    assert _bf(lib, q=NULL) == INVALID
    assert _bf(lib, out=NULL) == INVALID
    assert _bf(lib, kvpos=NULL) == INVALID
    assert _bf(lib, q=ctypes.c_void_p(0x1002)) == UNSUPPORTED  # misaligned for 16-byte loads
    # the grid counts query heads: 2^27 query tiles of 32 rows times 16 query heads is past the
    # grid limit even though the one K/V head alone would fit
    assert _bf(lib, seq_q=1 << 32, seq_kv=64, hq=16, hkv=1) == UNSUPPORTED and "grid" in _err(lib)
    # an empty query set is a valid no-op that never touches the GPU
    assert _bf(lib, seq_q=0, q=NULL, out=NULL, lse=NULL, qpos=NULL) == OK


def test_merge_validation(lib):
    f = lib.cpattn_lse_merge
    assert f(FAKE, FAKE, FAKE, FAKE, 0, 8, 2, 128, NULL) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 1, -1, 2, 128, NULL) == INVALID
    assert f(FAKE, FAKE, FAKE, FAKE, 1, 8, 2, 126, NULL) == SHAPE
    assert f(NULL, FAKE, FAKE, FAKE, 1, 8, 2, 128, NULL) == INVALID
    assert f(FAKE, FAKE, FAKE, ctypes.c_void_p(0x2000), 1, 8, 2, 128, NULL) == INVALID  # out aliases tile
    assert f(NULL, NULL, NULL, NULL, 1, 0, 2, 128, NULL) == OK  # empty: no-op


def test_reorder_validation(lib):
    f = lib.cpattn_reorder_gathered
    other = ctypes.c_void_p(0x2000)
    assert f(FAKE, other, 1, 30, 256, 4, 0, NULL) == SHAPE
    assert f(FAKE, other, 1, 32, 0, 4, 0, NULL) == INVALID
    assert f(FAKE, other, 1, 32, 256, 4, 2, NULL) == INVALID
    assert f(FAKE, FAKE, 1, 32, 256, 4, 0, NULL) == INVALID  # in place is not supported
    assert f(NULL, other, 1, 32, 256, 4, 0, NULL) == INVALID


def test_ulysses_validation(lib):
    f = lib.cpattn_ulysses_permute
    other = ctypes.c_void_p(0x2000)
    assert f(FAKE, other, 2, 1, 32, 6, 16, 4, 0, 0, NULL) == SHAPE and "heads" in _err(lib)
    assert f(FAKE, other, 2, 1, 30, 8, 16, 4, 0, 0, NULL) == SHAPE
    assert f(FAKE, other, 2, 1, 32, 8, 16, 4, 4, 0, NULL) == INVALID
    assert f(FAKE, other, 2, 1, 32, 8, 16, 4, 0, 5, NULL) == INVALID
    assert f(FAKE, other, 0, 1, 32, 8, 16, 4, 0, 0, NULL) == INVALID
    assert f(FAKE, FAKE, 2, 1, 32, 8, 16, 4, 0, 0, NULL) == INVALID


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 8, 2, 128, dtype=torch.bfloat16)
    pos = torch.arange(8)
    with pytest.raises(ValueError, match="GPU tensor"):
        cp.block_fwd(x, x, x, pos, pos, 0.1)


def test_block_fwd_merge_validation(lib):
    """The merging entry point validates exactly like cpattn_block_fwd."""
    def bfm(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, dtype=1, batch=1, seq_q=64, seq_kv=64, hq=4, hkv=2, d=128,
                 qpos=FAKE, kvpos=FAKE, scale=0.1, out=FAKE, lse=FAKE)
        a.update(kw)
        return lib.cpattn_block_fwd_merge(a["q"], a["k"], a["v"], a["dtype"], a["batch"], a["seq_q"],
                                          a["seq_kv"], a["hq"], a["hkv"], a["d"], a["qpos"], a["kvpos"],
                                          a["scale"], a["out"], a["lse"], NULL)
    assert bfm(dtype=7) == INVALID and _err(lib).startswith("block_fwd_merge:")
    assert bfm(batch=0) == INVALID
    assert bfm(scale=float("nan")) == INVALID
    assert bfm(hq=6, hkv=4) == SHAPE
    assert bfm(d=96, dtype=1) == UNSUPPORTED
    assert bfm(d=64, dtype=1, q=NULL) == INVALID  # D = 64 gets past the head-dim check
    assert bfm(hq=(1 << 17) + 1, hkv=(1 << 17) + 1) == UNSUPPORTED and "2^24" in _err(lib)
    assert bfm(lse=NULL) == INVALID
    assert bfm(out=ctypes.c_void_p(0x1004)) == UNSUPPORTED
    assert bfm(seq_q=0, q=NULL, out=NULL, lse=NULL, qpos=NULL) == OK


def test_ulysses_zigzag_validation(lib):
    f = lib.cpattn_ulysses_permute_zigzag
    other = ctypes.c_void_p(0x2000)
    # seq_len must split into 2C chunks
    assert f(FAKE, other, 2, 1, 36, 8, 16, 4, 0, 0, NULL) == SHAPE and "2*cp_size" in _err(lib)
    assert f(FAKE, other, 2, 1, 32, 6, 16, 4, 0, 0, NULL) == SHAPE
    assert f(FAKE, other, 2, 1, 32, 8, 16, 4, 4, 0, NULL) == INVALID
    assert f(FAKE, FAKE, 2, 1, 32, 8, 16, 4, 0, 0, NULL) == INVALID
    assert f(FAKE, other, 2, 1, 32, 8, 16, 4, 0, 7, NULL) == INVALID


def _delta(lib, **kw):
    a = dict(out=FAKE, dout=FAKE, dtype=1, batch=1, seq=64, heads=4, d=128, delta=FAKE)
    a.update(kw)
    return lib.cpattn_attn_bwd_delta(a["out"], a["dout"], a["dtype"], a["batch"], a["seq"], a["heads"], a["d"],
                                     a["delta"], NULL)


def test_attn_bwd_delta_validation(lib):
    assert _delta(lib, dtype=7) == INVALID
    assert _delta(lib, batch=0) == INVALID
    assert _delta(lib, heads=-1) == INVALID
    assert _delta(lib, d=0) == INVALID
    assert _delta(lib, seq=-1) == INVALID
    assert _delta(lib, delta=NULL) == INVALID
    assert _delta(lib, dout=NULL) == INVALID
    assert _delta(lib, d=126) == SHAPE and "multiple of 4" in _err(lib)
    assert _delta(lib, out=ctypes.c_void_p(0x1008)) == UNSUPPORTED
    # dout is read four elements at a time: 8 bytes for bf16, 16 for fp32
    # (an 8-byte aligned bf16 dout passes: the call then stops at the grid bound, before any launch)
    assert _delta(lib, dout=ctypes.c_void_p(0x1008), dtype=1, seq=1 << 40) == UNSUPPORTED and "grid" in _err(lib)
    assert _delta(lib, dout=ctypes.c_void_p(0x1004), dtype=1) == UNSUPPORTED and "8-byte" in _err(lib)
    assert _delta(lib, dout=ctypes.c_void_p(0x1008), dtype=0) == UNSUPPORTED and "16-byte" in _err(lib)
    assert _delta(lib, seq=0, out=NULL, dout=NULL, delta=NULL) == OK


def _bb(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dout=FAKE, dtype=1, batch=1, seq_q=64, seq_kv=64, hq=4, hkv=2, d=128,
             qpos=FAKE, kvpos=FAKE, scale=0.1, lse=FAKE, delta=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, flags=0)
    a.update(kw)
    return lib.cpattn_block_bwd(a["q"], a["k"], a["v"], a["dout"], a["dtype"], a["batch"], a["seq_q"],
                                a["seq_kv"], a["hq"], a["hkv"], a["d"], a["qpos"], a["kvpos"], a["scale"],
                                a["lse"], a["delta"], a["dq"], a["dk"], a["dv"], a["flags"], NULL)


def test_block_bwd_validation(lib):
    assert _bb(lib, flags=4) == INVALID and "flags" in _err(lib)
    assert _bb(lib, dtype=7) == INVALID
    assert _bb(lib, batch=0) == INVALID
    assert _bb(lib, hkv=0) == INVALID
    assert _bb(lib, seq_q=-1) == INVALID
    assert _bb(lib, seq_kv=-5) == INVALID
    assert _bb(lib, scale=0.0) == INVALID
    assert _bb(lib, scale=float("nan")) == INVALID
    assert _bb(lib, hq=6, hkv=4) == SHAPE and "multiple" in _err(lib)
    assert _bb(lib, d=96, dtype=0) == UNSUPPORTED
    # bf16 with head_dim 64 passes the head-dim check (refused here only for the misaligned q)
    assert _bb(lib, d=64, dtype=1, q=ctypes.c_void_p(0x1004)) == UNSUPPORTED and "aligned" in _err(lib)
    # bf16 rows of Q (heads_q * head_dim) above 2^24 elements are refused
    assert _bb(lib, hq=(1 << 17) + 2, hkv=2) == UNSUPPORTED and "2^24" in _err(lib)
    for name in ("q", "k", "v", "dout", "qpos", "kvpos", "lse", "delta", "dq", "dk", "dv"):
        assert _bb(lib, **{name: NULL}) == INVALID, name
    for name in ("q", "k", "v", "dout", "dq", "dk", "dv"):
        assert _bb(lib, **{name: ctypes.c_void_p(0x1004)}) == UNSUPPORTED, name
    # no pair and nothing to overwrite: a no-op that never touches the GPU
    assert _bb(lib, seq_q=0, q=NULL, dq=NULL, dk=NULL, dv=NULL) == OK
    assert _bb(lib, seq_kv=0, k=NULL, v=NULL, dq=NULL, dk=NULL, dv=NULL) == OK
    # overwriting an accumulator that exists needs its pointer
    assert _bb(lib, seq_kv=0, flags=1, dq=NULL) == INVALID
    assert _bb(lib, seq_q=0, flags=2, dv=NULL) == INVALID


def _rb(lib, n=4, seqs=None, ks=None, vs=None, ps=None, dks=None, dvs=None, arrays=True, **kw):
    seqs = seqs if seqs is not None else [64] * n
    ks, vs, ps, dks, dvs = ([0x1000] * n if x is None else x for x in (ks, vs, ps, dks, dvs))
    a = dict(q=FAKE, dout=FAKE, dtype=1, batch=1, seq_q=64, hq=4, hkv=2, d=128, qpos=FAKE, scale=0.1, lse=FAKE,
             delta=FAKE, dq=FAKE, n_blocks=n)
    a.update(kw)
    arr = ctypes.c_void_p * max(n, 1)
    blk = (lambda x: arr(*x)) if arrays else (lambda x: None)
    return lib.cpattn_ring_share_bwd(a["q"], a["dout"], blk(ks), blk(vs), blk(ps), (ctypes.c_int64 * max(n, 1))(*seqs),
                                     a["n_blocks"], a["dtype"], a["batch"], a["seq_q"], a["hq"], a["hkv"], a["d"],
                                     a["qpos"], a["scale"], a["lse"], a["delta"], a["dq"], blk(dks), blk(dvs), NULL)


def test_ring_share_bwd_validation(lib):
    assert _rb(lib, n_blocks=0) == INVALID
    assert _rb(lib, n=17) == INVALID and "n_blocks" in _err(lib)
    assert _rb(lib, arrays=False) == INVALID and "NULL block array" in _err(lib)
    assert _rb(lib, seqs=[64, -1, 64, 64]) == INVALID
    assert _rb(lib, dtype=7) == INVALID
    assert _rb(lib, batch=0) == INVALID
    assert _rb(lib, scale=float("nan")) == INVALID
    assert _rb(lib, hq=6, hkv=4) == SHAPE
    assert _rb(lib, d=96) == UNSUPPORTED
    assert _rb(lib, hq=(1 << 17) + 2, hkv=2) == UNSUPPORTED and "2^24" in _err(lib)
    for name in ("q", "dout", "qpos", "lse", "delta", "dq"):
        assert _rb(lib, **{name: NULL}) == INVALID, name
    # each block as a single-block call: its pointers, their alignment
    assert _rb(lib, ks=[0x1000, 0, 0x1000, 0x1000]) == INVALID
    assert _rb(lib, ps=[0x1000, 0x1000, 0, 0x1000]) == INVALID
    assert _rb(lib, dks=[0x1000, 0x1000, 0x1000, 0]) == INVALID
    assert _rb(lib, dvs=[0x1000, 0x1004, 0x1000, 0x1000]) == UNSUPPORTED and "aligned" in _err(lib)
    # a block without keys may hold NULL pointers; no pair anywhere and nothing to overwrite: a no-op
    z = [0] * 4
    assert _rb(lib, seq_q=0, seqs=z, ks=z, vs=z, ps=z, dks=z, dvs=z, q=NULL, dout=NULL, qpos=NULL, dq=NULL) == OK
    # every block is checked before anything is enqueued, for either dtype (without a GPU, a
    # launch would have returned CPATTN_ERR_HIP instead)
    assert _rb(lib, dtype=0, ps=[0x1000, 0x1000, 0x1000, 0]) == INVALID
    assert _rb(lib, dtype=1, dvs=[0x1000, 0x1000, 0x1000, 0]) == INVALID


def _rs(lib, n=4, seqs=None, ks=None, vs=None, ps=None, **kw):
    seqs = seqs if seqs is not None else [64] * n
    ks = ks if ks is not None else [0x1000] * n
    vs = vs if vs is not None else [0x1000] * n
    ps = ps if ps is not None else [0x1000] * n
    a = dict(q=FAKE, dtype=1, batch=1, seq_q=64, hq=4, hkv=2, d=128, qpos=FAKE, scale=0.1, out=FAKE, lse=FAKE,
             n_blocks=n)
    a.update(kw)
    arr = ctypes.c_void_p * max(n, 1)
    return lib.cpattn_ring_share_fwd(a["q"], arr(*ks), arr(*vs), arr(*ps), (ctypes.c_int64 * max(n, 1))(*seqs),
                                     a["n_blocks"], a["dtype"], a["batch"], a["seq_q"], a["hq"], a["hkv"], a["d"],
                                     a["qpos"], a["scale"], a["out"], a["lse"], NULL)


def test_ring_share_fwd_validation(lib):
    assert _rs(lib, n_blocks=0) == INVALID
    assert _rs(lib, n=17) == INVALID and "n_blocks" in _err(lib)
    assert _rs(lib, seqs=[64, -1, 64, 64]) == INVALID
    assert _rs(lib, ks=[0x1000, 0, 0x1000, 0x1000]) == INVALID and "block 1" in _err(lib)
    assert _rs(lib, ps=[0x1000, 0x1000, 0x1000, 0]) == INVALID
    assert _rs(lib, vs=[0x1000, 0x1000, 0x1008, 0x1000]) == UNSUPPORTED and "block 2" in _err(lib)
    # a block without keys may hold NULL pointers
    assert _rs(lib, seqs=[64, 0, 64, 64], ks=[0x1000, 0, 0x1000, 0x1000], q=NULL, seq_q=0) == OK
    assert _rs(lib, batch=0) == INVALID
    assert _rs(lib, hq=0) == INVALID
    assert _rs(lib, seq_q=-1) == INVALID
    assert _rs(lib, scale=float("inf")) == INVALID
    assert _rs(lib, hq=6, hkv=4) == SHAPE
    assert _rs(lib, d=96) == UNSUPPORTED
    assert _rs(lib, d=64, q=NULL) == INVALID  # bf16 D = 64 gets past the head-dim check
    assert _rs(lib, hq=(1 << 17) + 1, hkv=(1 << 17) + 1) == UNSUPPORTED and "2^24" in _err(lib)
    for name in ("q", "qpos", "out", "lse"):
        assert _rs(lib, **{name: NULL}) == INVALID, name
    assert _rs(lib, q=ctypes.c_void_p(0x1004)) == UNSUPPORTED
    assert _rs(lib, out=ctypes.c_void_p(0x1004)) == UNSUPPORTED
    assert _rs(lib, seq_q=0, q=NULL, out=NULL, lse=NULL, qpos=NULL) == OK
    # the fp32 path checks each block as a single-block call does
    assert _rs(lib, dtype=0, d=96) == UNSUPPORTED
    assert _rs(lib, dtype=0, hq=6, hkv=4) == SHAPE
    # ... and every block before the first launch: a bad later block fails the call with
    # nothing enqueued (without a GPU, a launch would have returned CPATTN_ERR_HIP instead)
    assert _rs(lib, dtype=0, ks=[0x1000, 0, 0x1000, 0x1000]) == INVALID
    assert _rs(lib, dtype=0, ps=[0x1000, 0x1000, 0x1000, 0]) == INVALID


def _rows(lib, **kw):
    a = dict(q=FAKE, qs=512, k=FAKE, v=FAKE, ks=128, sq=64, skv=64, hq=4, hkv=1, d=128, qpos=FAKE, kvpos=FAKE,
             scale=0.1, out=FAKE, os=512, lse=FAKE)
    a.update(kw)
    return lib.cpattn_block_fwd_rows(a["q"], a["qs"], a["k"], a["v"], a["ks"], a["sq"], a["skv"], a["hq"], a["hkv"],
                                     a["d"], a["qpos"], a["kvpos"], a["scale"], a["out"], a["os"], a["lse"], NULL)


def test_block_fwd_rows_validation(lib):
    assert _rows(lib, hq=0) == INVALID
    assert _rows(lib, sq=-1) == INVALID
    assert _rows(lib, scale=float("nan")) == INVALID
    assert _rows(lib, hq=6, hkv=4, qs=768, ks=512, os=768) == SHAPE
    assert _rows(lib, d=96) == UNSUPPORTED
    assert _rows(lib, d=64, qs=256, ks=64, os=256, q=NULL) == INVALID  # D = 64 gets past the head-dim check
    # row strides: at least a row, multiples of 8 (q, k/v) or 4 (out), q and k/v at most 2^24
    assert _rows(lib, qs=504) == UNSUPPORTED and "row strides" in _err(lib)
    assert _rows(lib, ks=120) == UNSUPPORTED
    assert _rows(lib, qs=1028) == UNSUPPORTED
    assert _rows(lib, ks=(1 << 24) + 8) == UNSUPPORTED
    assert _rows(lib, os=510) == UNSUPPORTED
    assert _rows(lib, q=NULL) == INVALID
    assert _rows(lib, lse=NULL) == INVALID
    assert _rows(lib, kvpos=NULL) == INVALID
    assert _rows(lib, out=ctypes.c_void_p(0x1004)) == UNSUPPORTED
    assert _rows(lib, k=ctypes.c_void_p(0x1008)) == UNSUPPORTED
    assert _rows(lib, sq=0, q=NULL, out=NULL, lse=NULL, qpos=NULL) == OK
    # (larger strides than the row pass validation: the call would then launch, so a grid
    # bound stands in for it here)
    assert _rows(lib, qs=4096, ks=1024, os=4100, sq=1 << 40) == UNSUPPORTED and "grid" in _err(lib)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libcpattn.so every entry point raises: there is no fallback path."""
    import context_causal_attention_amd._binding as b
    monkeypatch.setattr(b, "_lib", None)
    monkeypatch.setattr(b, "LIB_PATH", tmp_path / "libcpattn.so")
    with pytest.raises(RuntimeError, match="not built"):
        b.load_library()
    import torch
    with pytest.raises(RuntimeError, match="not built"):
        b.zigzag_index(64, 4, 0, out=torch.empty(16, dtype=torch.int64))

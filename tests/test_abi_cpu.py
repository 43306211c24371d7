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
    assert _bf(lib, d=64, dtype=1) == UNSUPPORTED  # bf16 path is D=128 only
    assert _bf(lib, q=NULL) == INVALID
    assert _bf(lib, out=NULL) == INVALID
    assert _bf(lib, kvpos=NULL) == INVALID
    assert _bf(lib, q=ctypes.c_void_p(0x1002)) == UNSUPPORTED  # misaligned for 16-byte loads
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
    assert bfm(d=64, dtype=1) == UNSUPPORTED
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

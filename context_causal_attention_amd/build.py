"""Build libcpattn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m context_causal_attention_amd.build [--verbose]

Each csrc/*.hip file is compiled to an object under _build/ (in parallel), then linked
into context_causal_attention_amd/libcpattn.so.  Only the cpattn_* entry points of
include/cpattn.h are exported (-fvisibility=hidden elsewhere).
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
INCLUDE = ROOT / "include"
BUILD = ROOT / "_build"
LIB = PKG / "libcpattn.so"
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}",
]


# Per-file flags.  Kernels allowed more than 256 registers per lane (one wave per SIMD, as the
# backward's 4-wave dq kernel) otherwise get accumulator-register (AGPR) destinations for
# their matrix products, and every score is copied out of them for the vector math
# (v_accvgpr_read/write around each product).  The vector-register form keeps the products'
# results where the vector instructions read them; AGPRs then serve only as spill space.
# (Kernels with two or three waves per SIMD, as every forward variant, compile to the same
# code either way.)
_VGPR_FORM = ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]
FILE_FLAGS = {
    "block_bwd_bf16.hip": _VGPR_FORM,
    "block_fwd_bf16.hip": _VGPR_FORM,
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and Path(c).exists():
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libcpattn.so)")


def sources() -> list[Path]:
    return sorted(CSRC.glob("*.hip"))


def _compile(src: Path, verbose: bool, extra: list[str]) -> Path:
    obj = BUILD / (src.stem + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *FILE_FLAGS.get(src.name, []), *extra, "-c", str(src), "-o", str(obj)]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 target feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{msg}")
    if msg.strip() and verbose:
        print(msg)
    return obj


def build(verbose: bool = False, extra: list[str] | None = None) -> Path:
    BUILD.mkdir(exist_ok=True)
    extra = list(extra or [])
    srcs = sources()
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, extra), srcs))
    tmp = LIB.with_suffix(".so.tmp")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(verbose=args.verbose))
    return 0


if __name__ == "__main__":
    sys.exit(main())

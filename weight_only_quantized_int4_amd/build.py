"""Build libqgemv.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Each source is compiled to an object under ``_build/`` (in parallel), then the
objects are linked into ``weight_only_quantized_int4_amd/libqgemv.so``.  The
bench's streaming-read probe (``read_probe.hip``) is linked into a library of
its own, ``libqgemv_readprobe.so``, so the product library never holds it.
hipcc cross-compiles for gfx950 without a GPU.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libqgemv.so")
PROBE_LIB = os.path.join(PKG, "libqgemv_readprobe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["qgemv_api.cpp", "int4_gemv.hip", "int4_packed.hip", "q4k_gemv.hip", "bf16_gemv.hip",
           "q4k_mmq.hip"]
PROBE_SOURCES = ["read_probe.hip"]

# -packed-fp32-ops: never emit v_pk_{add,mul,fma}_f32 (kept off on this target).
# Correctly rounded binary32 division: the 8-bit activation codes are decided
# by a quotient.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
    "-Wno-unused-parameter", "-ffp-contract=fast", "-fvisibility=hidden",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


# Per-source flags.  q4k_mmq.hip: keep matrix-core results in VGPRs (its
# vector ALUs consume every result; the AGPR form adds a read per element).
SOURCE_FLAGS = {"q4k_mmq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, "-x", "hip", *FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(extra_flags=(), out: str = LIB, verbose: bool = False, probe: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + (PROBE_SOURCES if probe else [])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, list(extra_flags)), srcs)))
    _link([objs[s] for s in SOURCES], out)
    _write_build_info(out)
    if verbose:
        print(f"built {out}")
    if probe:
        _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
        if verbose:
            print(f"built {PROBE_LIB}")
    return out


def _write_build_info(lib: str) -> None:
    """Record what the library was built from next to it (the GPU runs see the
    tree without its git metadata): commit, whether the tree was dirty, and
    the library's sha256."""
    import hashlib
    import json

    def git(*args):
        r = subprocess.run(["git", "-C", ROOT, *args], capture_output=True, text=True)
        return r.stdout.strip() if r.returncode == 0 else None

    with open(lib, "rb") as f:
        digest = hashlib.sha256(f.read()).hexdigest()
    info = {"git_commit": git("rev-parse", "HEAD"),
            "git_dirty": bool(git("status", "--porcelain", "--untracked-files=no")),
            "library_sha256": digest, "hipcc_flags": FLAGS[:-4]}
    with open(os.path.join(PKG, "build_info.json"), "w") as f:
        json.dump(info, f, indent=1)


if __name__ == "__main__":
    build(sys.argv[1:], verbose=True)

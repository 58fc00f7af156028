"""Build libqgemv.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Each source is compiled to an object under ``_build/`` (in parallel), then the
objects are linked into ``weight_only_quantized_int4_amd/libqgemv.so``.  The
bench's streaming-read probe (``read_probe.hip``) is linked into a library of
its own, ``libqgemv_readprobe.so``, and ``libqgemv_wavetimes.so`` is the product
library rebuilt with ``QG_WAVE_TIMES`` (the int4 span kernel records per-wave
timestamps, read by ``bench.py --wave-times``), so the product library never
holds either.
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
WAVE_TIMES_LIB = os.path.join(PKG, "libqgemv_wavetimes.so")
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


def _compile(src: str, extra, tag: str = "") -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + tag + ".o")
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
    jobs = [(s, "", list(extra_flags)) for s in SOURCES]
    if probe:
        jobs += [(s, "", list(extra_flags)) for s in PROBE_SOURCES]
        jobs.append(("int4_gemv.hip", "_wt", list(extra_flags) + ["-DQG_WAVE_TIMES"]))
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        done = list(ex.map(lambda j: _compile(j[0], j[2], j[1]), jobs))
    objs = {(s, t): o for (s, t, _), o in zip(jobs, done)}
    _link([objs[(s, "")] for s in SOURCES], out)
    _write_build_info(out)
    if verbose:
        print(f"built {out}")
    if probe:
        _link([objs[(s, "")] for s in PROBE_SOURCES], PROBE_LIB)
        _link([objs[(s, "_wt" if s == "int4_gemv.hip" else "")] for s in SOURCES], WAVE_TIMES_LIB)
        if verbose:
            print(f"built {PROBE_LIB}")
            print(f"built {WAVE_TIMES_LIB}")
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

"""Shared helpers of the GPU parity tests (not a test module).

Inputs come from ``datagen`` (seeded, no method arithmetic); expected values
come from ``oracle`` only.  The HIP path is called through the C ABI via the
package binding.
"""
from __future__ import annotations

import concurrent.futures
import functools
import os
import sys

import numpy as np
import torch

import datagen
import oracle

DEV = "cuda:0"
OUT_NAME = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a hard failure still shows it)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(DEV)


def f16_dev(bits: np.ndarray) -> torch.Tensor:
    return to_dev(bits.view(np.int16), torch.float16)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return to_dev(bits.view(np.int16), torch.bfloat16)


def y_host(y: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def assert_accept(y: np.ndarray, y_ref: np.ndarray, S: np.ndarray, out: str, what: str):
    ok, worst = oracle.accept(y, y_ref, S, out)
    assert ok, f"{what}: max |err|/(2e-3*S+ulp) = {worst:.3g}"
    return worst


# ---------------------------------------------------------------------------
# cached problems and oracle results (one per configuration)
# ---------------------------------------------------------------------------

@functools.lru_cache(maxsize=None)
def int4_case(N, K, bs, asym, seed):
    return datagen.int4_problem(N, K, bs, asym, seed)


@functools.lru_cache(maxsize=None)
def int4_ref(N, K, bs, asym, seed, cols=None):
    p = int4_case(N, K, bs, asym, seed)
    return oracle.int4_gemv(p.x, p.w, p.scales, p.zp, datagen.X_ROWS, N, K, bs,
                            cols=None if cols is None else list(cols))


@functools.lru_cache(maxsize=None)
def q4k_case(N, K, seed):
    return datagen.q4k_problem(N, K, seed)


@functools.lru_cache(maxsize=None)
def q4k_ref(N, K, seed, M=datagen.X_ROWS, cols=None):
    p = q4k_case(N, K, seed)
    return oracle.q4k_gemv(p.x, p.w, M, N, K, cols=None if cols is None else list(cols))


@functools.lru_cache(maxsize=None)
def bf16_case(N, K, seed):
    return datagen.bf16_problem(N, K, seed)


def oracle_threads() -> int:
    """Host threads for the oracle: the cores this process may use, at most
    16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_all_columns(fn, N, *args, **kw):
    """(y_ref, S) of every column of an oracle GEMV ``fn(*args, cols=...)``,
    computed over column ranges on host threads (the oracle's C calls release
    the GIL; columns are independent, so the result is the same as one call)."""
    t = oracle_threads()
    bounds = [(i * N) // t for i in range(t + 1)]
    ranges = [np.arange(bounds[i], bounds[i + 1]) for i in range(t) if bounds[i + 1] > bounds[i]]
    with concurrent.futures.ThreadPoolExecutor(len(ranges)) as ex:
        parts = list(ex.map(lambda c: fn(*args, cols=c, **kw), ranges))
    return (np.concatenate([p[0] for p in parts], axis=1),
            np.concatenate([p[1] for p in parts], axis=1))


@functools.lru_cache(maxsize=None)
def int4_ref_all(N, K, bs, asym, seed):
    """All X_ROWS rows of x against every column, on host threads."""
    p = int4_case(N, K, bs, asym, seed)
    return oracle_all_columns(oracle.int4_gemv, N, p.x, p.w, p.scales, p.zp, datagen.X_ROWS, N,
                              K, bs)

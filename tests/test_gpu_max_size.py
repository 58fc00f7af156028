"""GPU parity at the largest encoded weights the C ABI accepts: just under
4 GiB (the limit that keeps every weight byte offset within 32 bits).  The
kernels' offsets reach their top here; sampled output columns, most of them in
the last sixteenth of the rows and the last two rows included, are checked
against the oracle."""
import gc

import numpy as np
import pytest
import torch

import datagen
import oracle
import weight_only_quantized_int4_amd as q
from gpu_cases import DEV, assert_accept, f16_dev, say, to_dev, y_host

pytestmark = pytest.mark.gpu


def _cols(N, seed):
    rng = np.random.default_rng(seed)
    top = rng.integers(N - N // 16, N, 48).tolist()
    rest = rng.integers(0, N, 16).tolist()
    return sorted(set(top) | set(rest) | {0, N - 2, N - 1})


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def test_int4_just_under_4_gib():
    N, K, bs = 131071, 65536, 32
    say(f"int4 max size N={N} K={K}: generating {N * K // 2 / 2**30:.3f} GiB")
    p = datagen.int4_problem(N, K, bs, True, 1600)
    assert 2**32 - 2**20 < p.w.nbytes < 2**32
    wd, sd, zd = to_dev(p.w), f16_dev(p.scales), to_dev(p.zp)
    cols = _cols(N, 1601)
    for M in (1, 4):
        say(f"int4 max size M={M}")
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        q.qgemv_int4_blockwise(f16_dev(p.x[:M]), wd, sd, zd, y, bs)
        got = y_host(y)[:, cols]
        yr, S = oracle.int4_gemv(p.x, p.w, p.scales, p.zp, M, N, K, bs, cols=cols)
        assert_accept(got, yr, S, "f32", f"int4 max size M={M}")
    del wd, sd, zd, y, p
    _free()


def test_q4k_just_under_4_gib():
    N, K = 116508, 65536
    say(f"q4k max size N={N} K={K}: generating {N * K // 256 * 144 / 2**30:.3f} GiB")
    p = datagen.q4k_problem(N, K, 1700)
    assert 2**32 - 2**20 < p.w.nbytes < 2**32
    wd = to_dev(p.w)
    cols = _cols(N, 1701)
    for M in (1, 3):
        say(f"q4k max size M={M}")
        y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
        q.qgemv_q4k(to_dev(p.x[:M]), wd, y)
        got = y_host(y)[:, cols]
        yr, S = oracle.q4k_gemv(p.x, p.w, M, N, K, cols=cols)
        assert_accept(got, yr, S, "f32", f"q4k max size M={M}")
    # the prefill product over the same weights, through the plane
    say("q4k max size: plane and prefill product, T=16")
    dsc = torch.empty((q.q4k_dsc_plane_bytes(N, K) // 8, 2), dtype=torch.float32, device=DEV)
    q.q4k_build_dsc_plane(wd, dsc, N, K)
    T = 16
    x = datagen.prefill_x(T, K, 1702)
    ws = torch.empty(q.q4k_mmq_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    y = torch.full((T, N), float("nan"), dtype=torch.float32, device=DEV)
    q.qgemm_q4k_mmq(to_dev(x), wd, dsc, y, ws)
    got = y_host(y)[:, cols]
    yr, S = oracle.q4k_mmq(x, p.w, T, N, K, cols=cols)
    ok, worst = oracle.accept(got, yr, S, "f32", rtol=oracle.RTOL_MMQ)
    assert ok, f"q4k max size prefill: max |err|/(RTOL_MMQ*S+ulp) = {worst:.3g}"
    del wd, dsc, ws, y, p
    _free()

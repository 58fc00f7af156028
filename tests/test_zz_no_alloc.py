"""GPU check of qgemm_q4k_mmq_noalloc, the prefill entry point that allocates
nothing (its workspace is the library's static device array).

Through the C ABI (package binding), two calls in a row -- the second with a
smaller problem, so it runs on the array the first one left behind -- must
each give exactly what qgemm_q4k_mmq gives with a caller-owned workspace (the
same kernels; the result is bitwise the same) and meet the oracle's bound for
the prefill product.  A problem whose workspace exceeds the array is refused
with nothing enqueued, and the array's contents do not leak into a later call.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import weight_only_quantized_int4_amd as q
from gpu_cases import DEV, q4k_case, say, to_dev, y_host

pytestmark = pytest.mark.gpu


def _plane(wd, N, K):
    dsc = torch.empty((q.q4k_dsc_plane_bytes(N, K) // 8, 2), dtype=torch.float32, device=DEV)
    q.q4k_build_dsc_plane(wd, dsc, N, K)
    return dsc


def _with_workspace(xd, wd, dsc, T, N, K):
    ws = torch.empty(q.q4k_mmq_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    y = torch.full((T, N), float("nan"), dtype=torch.float32, device=DEV)
    q.qgemm_q4k_mmq(xd, wd, dsc, y, ws)
    return y_host(y)


@pytest.mark.parametrize("calls", [[(300, 1000, 4096), (37, 500, 4096)],
                                   [(512, 256, 2048), (65, 130, 1024)]])
def test_noalloc_matches_workspace_entry_point(calls):
    for i, (T, N, K) in enumerate(calls):
        p = q4k_case(N, K, 6600 + N)
        x = datagen.prefill_x(T, K, 6700 + T)
        xd, wd = to_dev(x), to_dev(p.w)
        dsc = _plane(wd, N, K)
        say(f"mmq noalloc call {i}: T={T} N={N} K={K}")
        y = torch.full((T, N), float("nan"), dtype=torch.float32, device=DEV)
        q.qgemm_q4k_mmq_noalloc(xd, wd, dsc, y)
        got = y_host(y)
        assert "q8_quantize" in q.last_launch() and "q4k_mmq" in q.last_launch()
        want = _with_workspace(xd, wd, dsc, T, N, K)
        assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), (T, N, K)
        yr, S = oracle.q4k_mmq(x, p.w, T, N, K)
        ok, worst = oracle.accept(got, yr, S, "f32", rtol=oracle.RTOL_MMQ)
        assert ok, f"noalloc T={T} N={N} K={K}: max |err|/(RTOL_MMQ*S+ulp) = {worst:.3g}"


def test_noalloc_refuses_a_problem_larger_than_its_array():
    T, N, K = 8192, 16, 4096
    assert q.q4k_mmq_workspace_bytes(T, K) > q.MMQ_NOALLOC_SCRATCH_BYTES
    p = q4k_case(N, K, 6601)
    wd = to_dev(p.w)
    dsc = _plane(wd, N, K)
    xd = torch.zeros((T, K), dtype=torch.float32, device=DEV)
    y = torch.full((T, N), 7.0, dtype=torch.float32, device=DEV)
    say("mmq noalloc over the limit")
    with pytest.raises(q.QgemvError) as ei:
        q.qgemm_q4k_mmq_noalloc(xd, wd, dsc, y)
    assert ei.value.status_name == "QG_ERR_UNSUPPORTED"
    assert q.last_launch() == ""
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)

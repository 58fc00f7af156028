"""GPU parity at the degenerate shapes of each format: one output column
(N = 1), the shortest row each format allows (int4: one scale block; q4_K: one
super-block; bf16: K = 1), and both ends of M.  Every kernel meets the
tolerance against the oracle on every output."""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_int4_amd as q
from gpu_cases import (DEV, assert_accept, bf16_case, bf16_dev, f16_dev, int4_case, int4_ref,
                       q4k_case, q4k_ref, say, to_dev, y_host)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,K,bs", [(1, 32, 32), (1, 4096, 32), (3, 128, 128), (1, 8192, 64),
                                    (17, 64, 64)])
@pytest.mark.parametrize("M", [1, 2, 8])
def test_int4(N, K, bs, M):
    say(f"int4 degenerate N={N} K={K} bs={bs} M={M}")
    p = int4_case(N, K, bs, True, 1300 + N + K)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.qgemv_int4_blockwise(f16_dev(p.x[:M]), to_dev(p.w), f16_dev(p.scales), to_dev(p.zp), y, bs)
    yr, S = int4_ref(N, K, bs, True, 1300 + N + K)
    assert_accept(y_host(y), yr[:M], S[:M], "f32", f"int4 {N}x{K} bs={bs} M={M}")


@pytest.mark.parametrize("N,K", [(1, 256), (1, 11008), (5, 256)])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_q4k(N, K, M):
    say(f"q4k degenerate N={N} K={K} M={M}")
    p = q4k_case(N, K, 1400 + N)
    wd = to_dev(p.w)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.qgemv_q4k(to_dev(p.x[:M]), wd, y)
    yr, S = q4k_ref(N, K, 1400 + N)
    assert_accept(y_host(y), yr[:M], S[:M], "f32", f"q4k {N}x{K} M={M}")
    dsc = torch.empty((q.q4k_dsc_plane_bytes(N, K) // 8, 2), dtype=torch.float32, device=DEV)
    q.q4k_build_dsc_plane(wd, dsc, N, K)
    yp = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.qgemv_q4k_dsc(to_dev(p.x[:M]), wd, dsc, yp)
    assert np.array_equal(y_host(yp), y_host(y))


@pytest.mark.parametrize("N,K", [(1, 1), (1, 8), (2, 3), (1, 6912), (9, 1)])
@pytest.mark.parametrize("M", [1, 2, 8])
def test_bf16(N, K, M):
    say(f"bf16 degenerate N={N} K={K} M={M}")
    p = bf16_case(N, K, 1500 + N + K)
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_bf16(bf16_dev(p.x[:M]), bf16_dev(p.w), y)
    yr, S = oracle.bf16_gemv(np.ascontiguousarray(p.x[:M]), np.ascontiguousarray(p.w), M, N, K, K, K)
    assert_accept(y_host(y), yr, S, "f32", f"bf16 {N}x{K} M={M}")

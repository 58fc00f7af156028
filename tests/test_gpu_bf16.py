"""GPU parity of gemv_bf16 (MI355X).

Workloads: (1536 x 1536), (256 x 1536), (1536 x 6912), (6912 x 1536) at
M = 1..8; the unaligned-tail path with K in {7, 12, 100, 1534} at N in
{256, 1536}; 2-byte base offsets on x and W; every output type; the current
stream; invariants; seeded random shapes, offsets and row strides.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_int4_amd as q
from gpu_cases import DEV, OUT_NAME, assert_accept, bf16_case, bf16_dev, say, y_host

pytestmark = pytest.mark.gpu


def _ref(p, M, cols=None, ldw=None, wbuf=None, xbuf=None, ldx=None):
    xb = p.x[:M] if xbuf is None else xbuf
    wb = p.w if wbuf is None else wbuf
    return oracle.bf16_gemv(np.ascontiguousarray(xb), np.ascontiguousarray(wb), M, p.N, p.K,
                            p.K if ldx is None else ldx, p.K if ldw is None else ldw, cols=cols)


@pytest.mark.parametrize("N,K,seed", [(1536, 1536, 301), (256, 1536, 302), (1536, 6912, 303),
                                      (6912, 1536, 304)])
@pytest.mark.parametrize("M", list(range(1, 9)))
def test_decode_shapes(N, K, seed, M):
    p = bf16_case(N, K, seed)
    say(f"bf16 N={N} K={K} M={M}")
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    q.gemv_bf16(bf16_dev(p.x[:M]), bf16_dev(p.w), y)
    launch = q.last_launch()
    # aligned x and W: the v_dot2 kernel at M = 1, the matrix cores from M = 2
    assert ("bf16_aligned" if M == 1 else "bf16_mfma_") in launch, launch
    yr, S = _ref(p, M)
    assert_accept(y_host(y), yr, S, "bf16", f"bf16 {N}x{K} M={M} ({launch})")


@pytest.mark.parametrize("N", [256, 1536])
@pytest.mark.parametrize("K", [7, 12, 100, 1534])
@pytest.mark.parametrize("M", [1, 3, 8])
def test_unaligned_k(N, K, M):
    p = bf16_case(N, K, 310 + K + N)
    say(f"bf16 unaligned K={K} N={N} M={M}")
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_bf16(bf16_dev(p.x[:M]), bf16_dev(p.w), y)
    yr, S = _ref(p, M)
    assert_accept(y_host(y), yr, S, "f32", f"bf16 unaligned K={K}")


@pytest.mark.parametrize("K", [12, 1534, 4096])
@pytest.mark.parametrize("off", [1, 3, 7])
def test_storage_offsets(K, off):
    N, M = 300, 4
    p = bf16_case(N, K, 320 + K)
    # W and x both start `off` elements into their buffers
    wbuf = np.zeros(off + N * K, dtype=np.uint16)
    wbuf[off:] = p.w.ravel()
    xbuf = np.zeros(off + M * K, dtype=np.uint16)
    xbuf[off:] = p.x[:M].ravel()
    wd = bf16_dev(wbuf)[off:].view(N, K)
    xd = bf16_dev(xbuf)[off:].view(M, K)
    say(f"bf16 offset={off} K={K}")
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_bf16(xd, wd, y)
    yr, S = _ref(p, M)
    assert_accept(y_host(y), yr, S, "f32", f"bf16 offset {off}")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_output_types(out_dtype):
    p = bf16_case(512, 2048, 330)
    say(f"bf16 out={out_dtype}")
    y = torch.full((2, 512), float("nan"), dtype=out_dtype, device=DEV)
    q.gemv_bf16(bf16_dev(p.x[:2]), bf16_dev(p.w), y)
    yr, S = _ref(p, 2)
    assert_accept(y_host(y), yr, S, OUT_NAME[out_dtype], "bf16 out types")


def test_long_unaligned_k_multi_chunk():
    # M = 8 stages 1776 elements per pass in the general path: K = 6911 -> 4 passes;
    # x rows start at odd element offsets (ldx = 6911), each row its own alignment
    N, K, M = 200, 6911, 8
    p = bf16_case(N, K, 340)
    say("bf16 general path multi-chunk")
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_bf16(bf16_dev(p.x[:M]), bf16_dev(p.w), y)
    yr, S = _ref(p, M)
    assert_accept(y_host(y), yr, S, "f32", "bf16 general multi-chunk")


@pytest.mark.parametrize("K", [1024, 512])
def test_one_hot_probe_matrix_core_path_is_bit_exact(K):
    """M = 4 (v_mfma path; K = 1024 splits each tile over a workgroup's waves,
    K = 512 gives whole tiles): row r of x is one-hot at k_r, so y[r, n] must
    equal w[n, k_r] (bf16 -> fp32 is exact) bitwise."""
    N = 48
    p = bf16_case(N, K, 350 + K)
    wd = bf16_dev(p.w)
    want_all = (p.w.astype(np.uint32) << 16).view(np.float32)
    ks = list(range(0, K, 3))
    say(f"bf16 mfma one-hot probe K={K}: {len(ks)} positions")
    for i0 in range(0, len(ks), 4):
        kk = ks[i0:i0 + 4]
        M = len(kk)
        x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
        for r, k in enumerate(kk):
            x[r, k] = 1.0
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        q.gemv_bf16(x, wd, y)
        got = y.cpu().numpy()
        want = want_all[:, kk].T
        assert np.array_equal(got, want), kk
        nz = want != 0
        assert np.array_equal(got.view(np.uint32)[nz], want.view(np.uint32)[nz]), kk


def _one_hot_expected(p, ks, xbuf_rows=None):
    """The oracle's y for one-hot rows of x (row i one-hot at ks[i]), as
    float32: each is a bf16 weight, exactly representable."""
    K = p.K
    x = np.zeros((len(ks), K), dtype=np.uint16)
    for i, k in enumerate(ks):
        x[i, k] = 0x3F80  # bf16 1.0
    yr, _ = oracle.bf16_gemv(x, p.w, len(ks), p.N, K, K, K)
    assert np.array_equal(yr.astype(np.float32).astype(np.float64), yr)
    return x, yr.astype(np.float32)


@pytest.mark.parametrize("N,K,path", [(300, 1024, "bf16_aligned"), (64, 1536, "bf16_aligned"),
                                      (300, 1534, "bf16_general"), (48, 100, "bf16_general")])
def test_one_hot_probe_single_row_is_bit_exact(N, K, path):
    """M = 1, fp32 out: y[n] must equal w[n, k] bitwise, the expected value
    coming from the oracle (x = e_k).  K = 1024 / 1536 with aligned rows take
    the v_dot2 kernel; K = 1534 / 100 (rows not 16-byte multiples) the
    anchored general kernel."""
    p = bf16_case(N, K, 370 + K)
    wd = bf16_dev(p.w)
    ks = sorted(set(list(range(0, K, max(1, K // 97))) + [1, 7, 8, K - 2, K - 1]))
    x, want = _one_hot_expected(p, ks)
    xd = bf16_dev(x)
    say(f"bf16 one-hot M=1 N={N} K={K} ({path}): {len(ks)} positions")
    got = np.empty((len(ks), N), dtype=np.float32)
    for i in range(len(ks)):
        y = torch.empty((1, N), dtype=torch.float32, device=DEV)
        q.gemv_bf16(xd[i:i + 1], wd, y)
        assert path in q.last_launch(), q.last_launch()
        got[i] = y.cpu().numpy()[0]
    assert np.array_equal(got, want)
    nz = want != 0
    assert np.array_equal(got.view(np.uint32)[nz], want.view(np.uint32)[nz])


@pytest.mark.parametrize("off", [1, 3])
def test_one_hot_probe_general_path_offsets_is_bit_exact(off):
    """The anchored general kernel with W and x at odd 2-byte offsets (every
    row its own alignment), M = 3: row r of x one-hot at k_r."""
    N, K, M = 200, 1000, 3
    p = bf16_case(N, K, 380 + off)
    wbuf = np.zeros(off + N * K, dtype=np.uint16)
    wbuf[off:] = p.w.ravel()
    wd = bf16_dev(wbuf)[off:].view(N, K)
    ks = list(range(0, K, 11)) + [K - 1]
    x_all, want_all = _one_hot_expected(p, ks)
    say(f"bf16 one-hot general path offset={off}: {len(ks)} positions")
    for i0 in range(0, len(ks), M):
        rows = x_all[i0:i0 + M]
        MM = rows.shape[0]
        xbuf = np.zeros(off + MM * K, dtype=np.uint16)
        xbuf[off:] = rows.ravel()
        xd = bf16_dev(xbuf)[off:].view(MM, K)
        y = torch.empty((MM, N), dtype=torch.float32, device=DEV)
        q.gemv_bf16(xd, wd, y)
        assert "bf16_general" in q.last_launch(), q.last_launch()
        got = y.cpu().numpy()
        assert np.array_equal(got, want_all[i0:i0 + MM]), ks[i0:i0 + MM]


@pytest.mark.parametrize("M", [2, 5])
def test_wide_matrix_sampled(M):
    # 40000 rows = 2500 tiles of 16: every wave owns whole tiles
    N, K = 40000, 1536
    p = bf16_case(N, K, 360)
    say(f"bf16 wide N={N} K={K} M={M}")
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_bf16(bf16_dev(p.x[:M]), bf16_dev(p.w), y)
    cols = sorted(set(np.random.default_rng(6).integers(0, N, 500).tolist()) | {0, 15, 16, N - 1})
    yr, S = _ref(p, M, cols=cols)
    assert_accept(y_host(y)[:, cols], yr, S, "f32", f"bf16 wide M={M}")


def test_invariants_and_stream():
    p = bf16_case(1536, 1536, 301)
    xd, wd = bf16_dev(p.x[:4]), bf16_dev(p.w)
    say("bf16 invariants")
    y = torch.empty((4, 1536), dtype=torch.float32, device=DEV)
    q.gemv_bf16(xd, wd, y)
    base = y_host(y)
    q.gemv_bf16(xd, wd, y)
    assert np.array_equal(base, y_host(y))
    # y(-x) = -y(x) is checked to the tolerance, not bitwise: v_dot2_f32_bf16
    # (M = 1) is not sign-symmetric in its rounding on gfx950 (a probe of the
    # instruction against exact arithmetic shows ~1% of random cases off
    # round-to-nearest).
    q.gemv_bf16(-xd, wd, y)
    yr, S = _ref(p, 4)
    assert_accept(-y_host(y), yr, S, "f32", "bf16 y(-x)")
    assert np.max(np.abs(y_host(y) + base)) <= 1e-5 * np.max(np.abs(base))
    # the call is enqueued on the caller's current stream
    s = torch.cuda.Stream()
    y2 = torch.zeros((4, 1536), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        torch.cuda._sleep(50_000_000)
        q.gemv_bf16(xd, wd, y2)
        ev = torch.cuda.Event()
        ev.record(s)
    assert not ev.query()
    assert torch.cuda.default_stream().query()
    s.synchronize()
    assert np.array_equal(y_host(y2), base)


@pytest.mark.parametrize("case", range(12))
def test_random_shapes_offsets_and_strides(case):
    """Seeded random N, K, M, 2-byte base offsets and row strides (padded,
    odd): mostly the unaligned path, where x rows are staged from aligned
    16-byte words and every row of x and W has its own alignment."""
    rng = np.random.default_rng(5000 + case)
    N, K, M = int(rng.integers(1, 700)), int(rng.integers(1, 3000)), int(rng.integers(1, 9))
    ldx, ldw = K + int(rng.integers(0, 9)), K + int(rng.integers(0, 9))
    offx, offw = int(rng.integers(0, 8)), int(rng.integers(0, 8))
    p = bf16_case(N, K, 6000 + case)
    xrows = np.zeros((M, ldx), dtype=np.uint16)
    xrows[:, :K] = p.x[:M]
    wrows = np.zeros((N, ldw), dtype=np.uint16)
    wrows[:, :K] = p.w
    xbuf = np.concatenate([np.zeros(offx, dtype=np.uint16), xrows.ravel()])
    wbuf = np.concatenate([np.zeros(offw, dtype=np.uint16), wrows.ravel()])
    xd = bf16_dev(xbuf)[offx:].as_strided((M, K), (ldx, 1))
    wd = bf16_dev(wbuf)[offw:].as_strided((N, K), (ldw, 1))
    say(f"bf16 random N={N} K={K} M={M} ldx={ldx} ldw={ldw} offx={offx} offw={offw}")
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_bf16(xd, wd, y)
    yr, S = _ref(p, M, ldw=ldw, wbuf=wrows, xbuf=xrows, ldx=ldx)
    assert_accept(y_host(y), yr, S, "f32", f"bf16 random case {case}")


# k parts of the split matrix-core kernel: where 16-row tiles leave CUs idle,
# the MFMA columns carry 8 rows in 2 parts of their k range (M <= 8) or 4
# rows in 4 parts (M <= 4); one workgroup per tile of 16 / ks rows (rows of
# 12 items: 4 wavefronts per workgroup).
@pytest.mark.parametrize("N,K,M,ks", [(1536, 6912, 3, 2), (1003, 4096, 4, 4), (777, 2048, 6, 2),
                                      (1001, 2048, 8, 2), (203, 4096, 2, 4), (250, 8192, 5, 2),
                                      (1536, 1536, 3, 2), (256, 1536, 8, 2)])
def test_matrix_core_k_parts(N, K, M, ks):
    p = bf16_case(N, K, 390 + M)
    say(f"bf16 k parts N={N} K={K} M={M} ks={ks}")
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.gemv_bf16(bf16_dev(p.x[:M]), bf16_dev(p.w), y)
    tr = 16 // ks
    assert f"bf16_mfma_split M={M} grid={(N + tr - 1) // tr} " in q.last_launch(), q.last_launch()
    yr, S = _ref(p, M)
    assert_accept(y_host(y), yr, S, "f32", f"bf16 k parts {N}x{K} M={M}")


@pytest.mark.parametrize("K,M,ks", [(4096, 4, 4), (4096, 3, 4), (2048, 8, 2), (8192, 5, 2),
                                     (1536, 3, 2), (1536, 6, 2)])
def test_one_hot_probe_k_parts_is_bit_exact(K, M, ks):
    """Row r of x one-hot at k_r (every 128-wide item and its seams probed, so
    every part of every step): y[r, n] must equal the oracle's y, which is
    w[n, k_r] exactly (fp32 out)."""
    N = 203
    p = bf16_case(N, K, 395 + M)
    wd = bf16_dev(p.w)
    kpos = sorted(set(list(range(0, K, 29)) + [128 * i - 1 for i in range(1, K // 128)] +
                      [128 * i for i in range(K // 128)] + [K - 1]))
    x_all, want_all = _one_hot_expected(p, kpos)
    say(f"bf16 k-parts one-hot K={K} M={M}: {len(kpos)} positions")
    tr = 16 // ks
    for i0 in range(0, len(kpos), M):
        rows = list(range(i0, min(i0 + M, len(kpos))))
        rows = rows + [rows[-1]] * (M - len(rows))
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        q.gemv_bf16(bf16_dev(x_all[rows]), wd, y)
        assert f"bf16_mfma_split M={M} grid={(N + tr - 1) // tr} " in q.last_launch(), q.last_launch()
        got = y.cpu().numpy()
        want = want_all[rows]
        assert np.array_equal(got, want), rows
        nz = want != 0
        assert np.array_equal(got.view(np.uint32)[nz], want.view(np.uint32)[nz]), rows

"""GPU parity of qgemv_q4k, q4k_build_dsc_plane and qgemv_q4k_dsc (MI355X).

Workloads: the 7B-decoder q4_K layer shapes (4096 x 4096), (11008 x 4096),
(4096 x 11008) at M = 1, direct decode and through the W_dsc plane; M = 1..8
on smaller shapes; the plane byte-exact against the oracle's plane over a
matrix of shapes (the page's host-mirror-vs-device test); direct and plane
paths bitwise equal; a one-hot dequant probe (bit-exact); invariants; seeded
random shapes and strides.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_int4_amd as q
from gpu_cases import DEV, assert_accept, q4k_case, q4k_ref, say, to_dev, y_host

pytestmark = pytest.mark.gpu


def _plane(wd, N, K):
    dsc = torch.empty((q.q4k_dsc_plane_bytes(N, K) // 8, 2), dtype=torch.float32, device=DEV)
    q.q4k_build_dsc_plane(wd, dsc, N, K)
    return dsc


@pytest.mark.parametrize("N,K,seed", [(4096, 4096, 401), (11008, 4096, 402), (4096, 11008, 403)])
def test_decoder_layer_shapes_direct_and_plane(N, K, seed):
    p = q4k_case(N, K, seed)
    xd, wd = to_dev(p.x[:1]), to_dev(p.w)
    yr, S = q4k_ref(N, K, seed, 1)
    say(f"q4k direct N={N} K={K}")
    y1 = torch.full((1, N), float("nan"), device=DEV)
    q.qgemv_q4k(xd, wd, y1)
    yd = y_host(y1)
    assert_accept(yd, yr, S, "f32", f"q4k direct {N}x{K}")
    say(f"q4k plane build + dsc N={N} K={K}")
    dsc = _plane(wd, N, K)
    y2 = torch.full((1, N), float("nan"), device=DEV)
    q.qgemv_q4k_dsc(xd, wd, dsc, y2)
    yp = y_host(y2)
    assert_accept(yp, yr, S, "f32", f"q4k dsc {N}x{K}")
    # one kernel, one summation order: the two paths agree bitwise
    assert np.array_equal(yd.view(np.uint64), yp.view(np.uint64))


@pytest.mark.parametrize("N,K", [(2, 256), (6, 512), (4096, 256), (2, 4096), (6, 11008),
                                 (4096, 4096), (11008, 4096), (4096, 11008), (37, 768)])
def test_plane_byte_exact(N, K):
    p = q4k_case(N, K, 1000 + N + K)
    say(f"q4k plane byte-exact N={N} K={K}")
    got = _plane(to_dev(p.w), N, K).cpu().numpy()
    want = oracle.q4k_build_plane(p.w, N, K)
    assert got.tobytes() == want.tobytes()


def test_plane_signed_zero_mins():
    """m == 0 must give -0.0 (bits 0x80000000) in the plane."""
    N, K = 64, 512
    p = q4k_case(N, K, 5)
    w = p.w.reshape(N, 2, 144).copy()
    w[:, :, 8:12] = 0        # mins of chunks 0..3 and top bits of chunks 4..7
    w[:, :, 12:16] &= 0x0F   # low bits of the mins of chunks 4..7
    w = w.reshape(N, 288)
    say("q4k plane signed zero")
    got = _plane(to_dev(w), N, K).cpu().numpy()
    assert np.all(got[:, 1].view(np.uint32) == 0x80000000)
    assert got.tobytes() == oracle.q4k_build_plane(w, N, K).tobytes()


@pytest.mark.parametrize("M", list(range(1, 9)))
def test_m_sweep(M):
    N, K = 1000, 4096
    p = q4k_case(N, K, 420)
    yr, S = q4k_ref(N, K, 420)
    xd, wd = to_dev(p.x[:M]), to_dev(p.w)
    say(f"q4k M={M} N={N} K={K}")
    y = torch.full((M, N), float("nan"), device=DEV)
    q.qgemv_q4k(xd, wd, y)
    yd = y_host(y)
    assert_accept(yd, yr[:M], S[:M], "f32", f"q4k M={M}")
    y2 = torch.full((M, N), float("nan"), device=DEV)
    q.qgemv_q4k_dsc(xd, wd, _plane(wd, N, K), y2)
    assert np.array_equal(yd, y_host(y2))


@pytest.mark.parametrize("N,K", [(9001, 4096), (1003, 11008), (300, 8192)])
def test_m1_rows_and_pieces_per_lane(N, K):
    # M = 1: rows past one resident round of wavefronts (9001 x 4096), and 3
    # (K = 11008) or 2 (K = 8192) pieces of a row per lane, with ragged row
    # counts and last strides
    p = q4k_case(N, K, 424)
    yr, S = q4k_ref(N, K, 424)
    xd, wd = to_dev(p.x[:1]), to_dev(p.w)
    say(f"q4k M=1 N={N} K={K}")
    y = torch.full((1, N), float("nan"), device=DEV)
    q.qgemv_q4k(xd, wd, y)
    yd = y_host(y)
    assert_accept(yd, yr[:1], S[:1], "f32", f"q4k M=1 {N}x{K}")
    y2 = torch.full((1, N), float("nan"), device=DEV)
    q.qgemv_q4k_dsc(xd, wd, _plane(wd, N, K), y2)
    assert np.array_equal(yd, y_host(y2))


@pytest.mark.parametrize("M", [2, 3])
def test_long_rows_x_resident(M):
    # K = 11008: x takes 94 KB (M = 2) and 140 KB (M = 3) of LDS, so the
    # whole of x stays resident in one workgroup
    N, K = 700, 11008
    p = q4k_case(N, K, 422)
    yr, S = q4k_ref(N, K, 422)
    xd, wd = to_dev(p.x[:M]), to_dev(p.w)
    say(f"q4k long rows M={M} N={N} K={K}")
    y = torch.full((M, N), float("nan"), device=DEV)
    q.qgemv_q4k(xd, wd, y)
    yd = y_host(y)
    assert_accept(yd, yr[:M], S[:M], "f32", f"q4k K={K} M={M}")
    y2 = torch.full((M, N), float("nan"), device=DEV)
    q.qgemv_q4k_dsc(xd, wd, _plane(wd, N, K), y2)
    assert np.array_equal(yd, y_host(y2))


def test_row_groups_and_strided_x():
    # K = 11008, M = 8: x does not fit in LDS, 3 rows do; three row groups
    N, K, M = 300, 11008, 8
    p = q4k_case(N, K, 421)
    yr, S = q4k_ref(N, K, 421)
    buf = np.zeros((M, K + 3), dtype=np.float32)
    buf[:, 1:K + 1] = p.x[:M]
    xt = to_dev(buf)[:, 1:K + 1]  # ldx = K + 3, 4-byte (not 16-byte) aligned
    say("q4k row groups, strided x")
    y = torch.full((M, N + 2), float("nan"), device=DEV)[:, :N]
    q.qgemv_q4k(xt, to_dev(p.w), y)
    assert_accept(y_host(y), yr, S, "f32", "q4k row groups")


@pytest.mark.parametrize("M", [1, 2, 8])
def test_multi_chunk_k(M):
    # K = 40960: one row of x exceeds 160 KB of LDS, so x is staged
    # in LDS one K chunk (a whole number of super-blocks) at a time, for at
    # most 4 rows of x per launch
    N, K = 64, 40960
    p = q4k_case(N, K, 423)
    yr, S = q4k_ref(N, K, 423)
    xd, wd = to_dev(p.x[:M]), to_dev(p.w)
    say(f"q4k multi-chunk K={K} M={M}")
    y = torch.full((M, N), float("nan"), device=DEV)
    q.qgemv_q4k(xd, wd, y)
    yd = y_host(y)
    assert_accept(yd, yr[:M], S[:M], "f32", f"q4k multi-chunk M={M}")
    y2 = torch.full((M, N), float("nan"), device=DEV)
    q.qgemv_q4k_dsc(xd, wd, _plane(wd, N, K), y2)
    assert np.array_equal(yd, y_host(y2))


def test_one_hot_probe_is_bit_exact():
    N, K = 96, 512
    p = q4k_case(N, K, 77)
    wdq = oracle.q4k_dequant(p.w, N, K).astype(np.float32)
    wd = to_dev(p.w)
    dsc = _plane(wd, N, K)
    ks = list(range(0, 256, 3)) + list(range(256, K, 5)) + [K - 1]
    say(f"q4k one-hot probe {len(ks)} columns")
    for use_plane in (False, True):
        got = np.empty((len(ks), N), dtype=np.float32)
        for i, k in enumerate(ks):
            x = torch.zeros((1, K), device=DEV)
            x[0, k] = 1.0
            y = torch.empty((1, N), device=DEV)
            if use_plane:
                q.qgemv_q4k_dsc(x, wd, dsc, y)
            else:
                q.qgemv_q4k(x, wd, y)
            got[i] = y.cpu().numpy()[0]
        assert np.array_equal(got.view(np.uint32), wdq[:, ks].T.copy().view(np.uint32)), use_plane


@pytest.mark.parametrize("K", [2048, 4096])
def test_one_hot_probe_multi_row_is_bit_exact(K):
    """M = 8: row r of x is one-hot at k_r; y must equal the oracle's
    dequantized weight bitwise, through the header and the plane."""
    N = 40
    p = q4k_case(N, K, 78)
    wdq = oracle.q4k_dequant(p.w, N, K).astype(np.float32)
    wd = to_dev(p.w)
    dsc = _plane(wd, N, K)
    ks = list(range(0, K, 7)) + [K - 1]
    say(f"q4k multi-row one-hot probe K={K}: {len(ks)} columns")
    for use_plane in (False, True):
        for i0 in range(0, len(ks), 8):
            kk = ks[i0:i0 + 8]
            M = len(kk)
            x = torch.zeros((M, K), device=DEV)
            for r, k in enumerate(kk):
                x[r, k] = 1.0
            y = torch.empty((M, N), device=DEV)
            if use_plane:
                q.qgemv_q4k_dsc(x, wd, dsc, y)
            else:
                q.qgemv_q4k(x, wd, y)
            got = y.cpu().numpy()
            assert np.array_equal(got.view(np.uint32), wdq[:, kk].T.copy().view(np.uint32)), (use_plane, kk)


@pytest.mark.parametrize("N,K,M", [(4096, 4096, 2), (4096, 4096, 8), (11008, 4096, 5),
                                   (4096, 11008, 3), (4096, 11008, 8), (1000, 2048, 4)])
def test_multi_row_layer_shapes_sampled(N, K, M):
    p = q4k_case(N, K, 990 + M)
    say(f"q4k multi-row N={N} K={K} M={M}")
    xd, wd = to_dev(p.x[:M]), to_dev(p.w)
    dsc = _plane(wd, N, K)
    cols = sorted(set(np.random.default_rng(8).integers(0, N, 300).tolist()) | {0, 15, 16, N - 1})
    yr, S = oracle.q4k_gemv(p.x, p.w, M, N, K, cols=cols)
    outs = []
    for use_plane in (False, True):
        y = torch.full((M, N), float("nan"), device=DEV)
        if use_plane:
            q.qgemv_q4k_dsc(xd, wd, dsc, y)
        else:
            q.qgemv_q4k(xd, wd, y)
        outs.append(y_host(y))
        assert_accept(outs[-1][:, cols], yr, S, "f32", f"q4k {N}x{K} M={M} plane={use_plane}")
    # one kernel template, one summation order: header and plane agree bitwise
    assert np.array_equal(outs[0].view(np.uint64), outs[1].view(np.uint64))


def test_row_magnitudes_and_unaligned_x():
    """Rows of x at magnitudes from 1e-6 to 1e6 (and one 6e7 outlier), x at a
    4-byte offset with a padded stride."""
    N, K, M = 700, 4096, 6
    p = q4k_case(N, K, 991)
    x = p.x[:M].astype(np.float64)
    x *= np.array([1e-6, 1e-2, 1.0, 3e2, 1e4, 1e6])[:, None]
    x = x.astype(np.float32)
    x[5, 100] = 6.0e7  # one large outlier in the last row
    ldx = K + 3
    buf = torch.zeros(1 + M * ldx, device=DEV)
    for r in range(M):
        buf[1 + r * ldx:1 + r * ldx + K] = torch.from_numpy(x[r]).to(DEV)
    xd = buf[1:].as_strided((M, K), (ldx, 1))
    wd = to_dev(p.w)
    say(f"q4k scaled rows N={N} K={K} M={M}")
    y = torch.full((M, N), float("nan"), device=DEV)
    q.qgemv_q4k(xd, wd, y)
    yr, S = oracle.q4k_gemv(x, p.w, M, N, K)
    assert_accept(y_host(y), yr, S, "f32", "q4k scaled rows")


def test_invariants():
    N, K, M = 512, 1024, 8
    p = q4k_case(N, K, 99)
    xd, wd = to_dev(p.x[:M]), to_dev(p.w)
    say("q4k invariants")
    y = torch.empty((M, N), device=DEV)
    q.qgemv_q4k(xd, wd, y)
    base = y_host(y)
    q.qgemv_q4k(xd, wd, y)
    assert np.array_equal(base, y_host(y))
    q.qgemv_q4k(-xd, wd, y)
    assert np.array_equal(y_host(y), -base)
    q.qgemv_q4k(xd * 0.25, wd, y)
    assert np.array_equal(y_host(y), 0.25 * base)
    # all quants 0 and all mins 0 -> y == 0
    w0 = p.w.reshape(N, 4, 144).copy()
    w0[:, :, 16:] = 0
    w0[:, :, 8:12] = 0
    w0[:, :, 12:16] &= 0x0F
    q.qgemv_q4k(xd, to_dev(w0.reshape(N, 576)), y)
    assert np.all(y_host(y) == 0.0)


def test_host_tensor_is_refused_before_the_call():
    # a host tensor's address must never reach a kernel: the binding refuses it
    p = q4k_case(16, 256, 1)
    say("q4k host tensor refused")
    with pytest.raises(ValueError, match="x must be a GPU tensor"):
        q.qgemv_q4k(torch.from_numpy(p.x[:1]), to_dev(p.w), torch.empty((1, 16), device=DEV))
    with pytest.raises(ValueError, match="y must be a GPU tensor"):
        q.qgemv_q4k(to_dev(p.x[:1]), to_dev(p.w), torch.empty((1, 16)))


def test_null_plane_is_rejected_on_device():
    p = q4k_case(16, 256, 1)
    say("q4k null plane")
    with pytest.raises(q.QgemvError) as ei:
        q.qgemv_q4k_dsc(to_dev(p.x[:1]), to_dev(p.w), None, torch.empty((1, 16), device=DEV))
    assert ei.value.status_name == "QG_ERR_NULL_POINTER"


@pytest.mark.parametrize("case", range(12))
def test_random_shapes_and_strides(case):
    """Seeded random N, K, M, x row stride and base offset, y row stride:
    direct decode and the plane (bitwise the same), against the oracle; long
    rows with many rows of x take row groups."""
    rng = np.random.default_rng(8000 + case)
    N, M = int(rng.integers(1, 1500)), int(rng.integers(1, 9))
    K = 256 * int(rng.integers(1, 49))
    ldx, offx = K + int(rng.integers(0, 9)), int(rng.integers(0, 4))
    ldy = N + int(rng.integers(0, 5))
    p = q4k_case(N, K, 8100 + case)
    xrows = np.zeros((M, ldx), dtype=np.float32)
    xrows[:, :K] = p.x[:M]
    xbuf = np.concatenate([np.zeros(offx, dtype=np.float32), xrows.ravel()])
    xd = to_dev(xbuf)[offx:].as_strided((M, K), (ldx, 1))
    wd = to_dev(p.w)
    say(f"q4k random N={N} K={K} M={M} ldx={ldx} offx={offx} ldy={ldy}")
    y = torch.full((M, ldy), float("nan"), device=DEV)[:, :N]
    q.qgemv_q4k(xd, wd, y)
    what = f"q4k random case {case} ({q.last_launch()})"
    y2 = torch.full((M, ldy), float("nan"), device=DEV)[:, :N]
    q.qgemv_q4k_dsc(xd, wd, _plane(wd, N, K), y2)
    yd = y_host(y)
    assert np.array_equal(yd, y_host(y2)), what
    yr, S = oracle.q4k_gemv(xrows, p.w, M, N, K, ldx=ldx)
    assert_accept(yd, yr, S, "f32", what)


@pytest.mark.parametrize("N,K", [(64, 2048), (300, 11008)])
@pytest.mark.parametrize("M", [1, 8])
def test_exactly_zero_weight_rows(N, K, M):
    """Rows whose weights are all exactly zero although no chunk's (dv, mv)
    is: y must be exactly 0 there (the bound is 1 subnormal ulp), through the
    header and through the plane.  The second half of the rows mixes such
    chunks with random ones and is held to the usual bound.  K = 11008 at
    M = 8 runs as row groups of x."""
    from q4k_cases import zero_weight_rows

    half = N // 2
    w = zero_weight_rows(N, K, seed=4000 + K, zero_frac=[1.0] * half + [0.5] * (N - half))
    x = np.random.default_rng(4100 + M).standard_normal((M, K)).astype(np.float32)
    yr, S = oracle.q4k_gemv(x, w, M, N, K)
    assert np.all(S[:, :half] == 0.0) and np.all(S[:, half:] > 0.0)
    xd, wd = to_dev(x), to_dev(w)
    dsc = _plane(wd, N, K)
    outs = []
    for use_plane in (False, True):
        say(f"q4k zero-weight rows N={N} K={K} M={M} plane={use_plane}")
        y = torch.full((M, N), float("nan"), device=DEV)
        if use_plane:
            q.qgemv_q4k_dsc(xd, wd, dsc, y)
        else:
            q.qgemv_q4k(xd, wd, y)
        got = y_host(y)
        outs.append(got)
        assert np.all(got[:, :half] == 0.0), (use_plane, np.abs(got[:, :half]).max())
        assert_accept(got, yr, S, "f32", f"q4k zero rows {N}x{K} M={M} plane={use_plane}")
    assert np.array_equal(outs[0].view(np.uint64), outs[1].view(np.uint64))

"""GPU parity of qgemv_int4_blockwise against the fp64 oracle (MI355X).

Workloads: the int4 decode shapes -- (256 x 1536, block 32, asymmetric, M=1),
(1536 x 1536) and (1536 x 6912) with block 128 and the implicit zero point 8,
M = 1..8, and the lm_head shape (151936 x 4096, block 32, asymmetric) at M = 1
and 8 on every column -- plus block sizes 64/256, every output type, ragged
N, strided and unaligned x, multi-chunk K, a one-hot dequant probe (bit-exact),
invariants, and seeded random shapes, block sizes, strides and output types.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import weight_only_quantized_int4_amd as q
from gpu_cases import (DEV, OUT_NAME, assert_accept, f16_dev, int4_case, int4_ref,
                       int4_ref_all, oracle_threads, say, to_dev, y_host)

pytestmark = pytest.mark.gpu


def _run(p, M, out_dtype=torch.float16, x=None, ldy=None):
    xd = f16_dev(p.x[:M]) if x is None else x
    wd = to_dev(p.w)
    sd = f16_dev(p.scales)
    zd = None if p.zp is None else to_dev(p.zp)
    if ldy is None:
        y = torch.full((M, p.N), float("nan"), dtype=out_dtype, device=DEV)
    else:
        y = torch.full((M, ldy), float("nan"), dtype=out_dtype, device=DEV)[:, :p.N]
    q.qgemv_int4_blockwise(xd, wd, sd, zd, y, p.block_size)
    return y


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_small_decode_shape_block32_asym(M):
    # 256 x 1536, block 32, asymmetric zero points, fp16 out
    say(f"int4 N=256 K=1536 bs=32 asym M={M}")
    p = int4_case(256, 1536, 32, True, 101)
    y = y_host(_run(p, M))
    yr, S = int4_ref(256, 1536, 32, True, 101)
    assert_accept(y, yr[:M], S[:M], "f16", f"int4 256x1536 M={M}")


@pytest.mark.parametrize("K,seed", [(1536, 201), (6912, 202)])
@pytest.mark.parametrize("M", list(range(1, 9)))
def test_symmetric_block128_sweep(K, seed, M):
    say(f"int4 N=1536 K={K} bs=128 sym M={M}")
    p = int4_case(1536, K, 128, False, seed)
    y = y_host(_run(p, M))
    yr, S = int4_ref(1536, K, 128, False, seed)
    assert_accept(y, yr[:M], S[:M], "f16", f"int4 1536x{K} M={M}")


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16, torch.float32])
@pytest.mark.parametrize("bs", [32, 64, 128, 256])
def test_block_sizes_and_output_types(bs, out_dtype):
    N, K = 1000, 2048  # ragged N (not a multiple of any row tile)
    say(f"int4 N={N} K={K} bs={bs} asym M=3 out={out_dtype}")
    p = int4_case(N, K, bs, True, 7 + bs)
    y = y_host(_run(p, 3, out_dtype))
    yr, S = int4_ref(N, K, bs, True, 7 + bs)
    assert_accept(y, yr[:3], S[:3], OUT_NAME[out_dtype], f"int4 bs={bs}")


def test_odd_block_count_and_tiny_shapes():
    for (N, K, bs) in [(1, 32, 32), (3, 96, 32), (17, 160, 32), (5, 128, 32), (5, 384, 128)]:
        say(f"int4 tiny N={N} K={K} bs={bs}")
        p = int4_case(N, K, bs, True, N * K)
        for M in (1, 8):
            y = y_host(_run(p, M, torch.float32))
            yr, S = int4_ref(N, K, bs, True, N * K)
            assert_accept(y, yr[:M], S[:M], "f32", f"int4 tiny {N}x{K} M={M}")


def test_strided_and_unaligned_x_and_strided_y():
    N, K, bs, M = 300, 1024, 32, 5
    say("int4 strided/unaligned x, strided y")
    p = int4_case(N, K, bs, True, 55)
    yr, S = int4_ref(N, K, bs, True, 55)
    # x rows with ldx = K + 3 and a 2-byte base offset
    buf = np.zeros(1 + M * (K + 3), dtype=np.uint16)
    for m in range(M):
        buf[1 + m * (K + 3):1 + m * (K + 3) + K] = p.x[m]
    xt = f16_dev(buf)[1:].view(M, K + 3)[:, :K]
    assert xt.data_ptr() % 16 == 2
    y = y_host(_run(p, M, torch.float16, x=xt, ldy=N + 5))
    assert_accept(y, yr[:M], S[:M], "f16", "int4 strided")


def test_multi_chunk_k():
    # K = 8224 (not a multiple of 128: v_dot2 kernel); M = 8 puts at most 3200
    # elements of x in LDS per pass, so K takes 3 passes
    N, K = 512, 8224
    say(f"int4 multi-chunk N={N} K={K} M=8")
    p = int4_case(N, K, 32, True, 77)
    y = y_host(_run(p, 8, torch.float32))
    yr, S = int4_ref(N, K, 32, True, 77)
    assert_accept(y, yr, S, "f32", "int4 multi-chunk")


@pytest.mark.parametrize("N", [512, 40000])
def test_matrix_core_x_above_64k(N):
    # M = 8, K = 8192: x takes 128 KB of LDS (one workgroup per CU); N = 512
    # splits tiles over the waves of a workgroup, N = 40000 gives whole tiles
    K, M = 8192, 8
    say(f"int4 matrix-core large x N={N} K={K} M={M}")
    p = int4_case(N, K, 32, True, 78)
    y = y_host(_run(p, M, torch.float32))
    cols = None if N == 512 else tuple(sorted(set(np.random.default_rng(4).integers(0, N, 400).tolist()) | {N - 1}))
    yr, S = int4_ref(N, K, 32, True, 78, cols)
    got = y if cols is None else y[:, list(cols)]
    assert_accept(got, yr[:M], S[:M], "f32", f"int4 large x N={N}")


@pytest.mark.parametrize("N,K,bs,asym,M,sampled", [(4096, 11008, 32, False, 8, True),
                                                  (4100, 11008, 64, True, 8, True),
                                                  (1000, 16384, 128, True, 5, False),
                                                  (520, 9856, 32, True, 8, False)])
def test_matrix_core_x_in_chunks(N, K, bs, asym, M, sampled):
    # x beyond the LDS left beside the split partials: the split kernel stages
    # x in chunks (two here), one tile per workgroup.  9856 = 77 items: x fits
    # whole (154 KB) but not with the partials.
    say(f"int4 matrix-core chunked x N={N} K={K} bs={bs} asym={asym} M={M}")
    p = int4_case(N, K, bs, asym, 80 + M)
    y = y_host(_run(p, M, torch.float32))
    assert "int4_mfma_phased" in q.last_launch(), q.last_launch()
    cols = tuple(sorted(set(np.random.default_rng(6).integers(0, N, 300).tolist()) | {0, 15, 16, N - 1})) \
        if sampled else None
    yr, S = int4_ref(N, K, bs, asym, 80 + M, cols)
    got = y if cols is None else y[:, list(cols)]
    assert_accept(got, yr[:M], S[:M], "f32", f"int4 chunked x {N}x{K} M={M}")


def test_one_hot_probe_chunked_x_is_bit_exact():
    """M = 8, K = 11008 (x staged in two chunks): row r of x is one-hot at k_r,
    positions spread over both chunks and their seams; y must equal the
    oracle's dequantized weights bitwise."""
    N, K, bs = 48, 11008, 64
    p = int4_case(N, K, bs, True, 34)
    wdq = oracle.int4_dequant(p.w, p.scales, p.zp, N, K, bs)
    wd, sd, zd = to_dev(p.w), f16_dev(p.scales), to_dev(p.zp)
    seam = 43 * 128  # first k of the second chunk
    ks = sorted(set(list(range(0, K, 97)) + [seam - 2, seam - 1, seam, seam + 1, K - 1]))
    say(f"int4 chunked one-hot probe K={K}: {len(ks)} positions")
    for i0 in range(0, len(ks), 8):
        kk = ks[i0:i0 + 8]
        M = len(kk)
        x = torch.zeros((M, K), dtype=torch.float16, device=DEV)
        for r, k in enumerate(kk):
            x[r, k] = 1.0
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        q.qgemv_int4_blockwise(x, wd, sd, zd, y, bs)
        if M == 8:
            assert "int4_mfma_phased" in q.last_launch(), q.last_launch()
        got = y.cpu().numpy()
        want = wdq[:, kk].T.astype(np.float32)
        assert np.array_equal(got, want), kk
        nz = want != 0
        assert np.array_equal(got.view(np.uint32)[nz], want.view(np.uint32)[nz]), kk


@pytest.mark.parametrize("M", [1, 8])
def test_lm_head_shape_every_column(M):
    """The lm_head shape, every one of the 151936 columns against the oracle
    (computed on host threads over column ranges)."""
    N, K = 151936, 4096
    say(f"int4 lm_head N={N} K={K} bs=32 asym M={M}")
    p = int4_case(N, K, 32, True, 501)
    y = y_host(_run(p, M))
    say(f"int4 lm_head oracle, {oracle_threads()} host threads")
    yr, S = int4_ref_all(N, K, 32, True, 501)
    assert_accept(y, yr[:M], S[:M], "f16", f"int4 lm_head M={M} ({q.last_launch()})")


def test_one_hot_probe_is_bit_exact():
    """x = e_k, fp32 out: y[n] must equal the oracle's dequantized w[n,k] bitwise."""
    N, K, bs = 64, 512, 32
    p = int4_case(N, K, bs, True, 31)
    wdq = oracle.int4_dequant(p.w, p.scales, p.zp, N, K, bs)
    wd, sd, zd = to_dev(p.w), f16_dev(p.scales), to_dev(p.zp)
    ks = list(range(0, 64)) + list(range(64, K, 7)) + [K - 1]
    say(f"int4 one-hot probe {len(ks)} columns of x")
    xs = torch.zeros((len(ks), K), dtype=torch.float16, device=DEV)
    for i, k in enumerate(ks):
        xs[i, k] = 1.0
    ys = torch.empty((len(ks), N), dtype=torch.float32, device=DEV)
    for i in range(len(ks)):
        q.qgemv_int4_blockwise(xs[i:i + 1], wd, sd, zd, ys[i:i + 1], bs)
    got = ys.cpu().numpy()
    want = wdq[:, ks].T.astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_lm_head_one_hot_sampled():
    N, K, bs = 151936, 4096, 32
    p = int4_case(N, K, bs, True, 501)
    wd, sd, zd = to_dev(p.w), f16_dev(p.scales), to_dev(p.zp)
    rng = np.random.default_rng(2)
    rows = sorted(set(rng.integers(0, N, 300).tolist()) | {N - 1})
    for k in [0, 31, 32, 2047, 4095]:
        say(f"int4 lm_head one-hot k={k}")
        x = torch.zeros((1, K), dtype=torch.float16, device=DEV)
        x[0, k] = 1.0
        y = torch.empty((1, N), dtype=torch.float32, device=DEV)
        q.qgemv_int4_blockwise(x, wd, sd, zd, y, bs)
        got = y.cpu().numpy()[0, rows]
        want = oracle.int4_dequant(p.w, p.scales, p.zp, N, K, bs, rows=rows)[:, k].astype(np.float32)
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), k


def test_invariants():
    N, K, bs, M = 512, 1024, 32, 8
    say("int4 invariants")
    p = int4_case(N, K, bs, True, 91)
    base = y_host(_run(p, M, torch.float32))
    # determinism
    again = y_host(_run(p, M, torch.float32))
    assert np.array_equal(base, again)
    # y(-x) == -y(x) and y(4x) == 4 y(x), bitwise
    neg = p.x[:M] ^ np.uint16(0x8000)
    yn = y_host(_run(p, M, torch.float32, x=f16_dev(neg)))
    assert np.array_equal(yn, -base)
    x4 = (f16_dev(p.x[:M]).float() * 4).half()
    y4 = y_host(_run(p, M, torch.float32, x=x4))
    assert np.array_equal(y4, 4 * base)
    # every code equal to its zero point -> y == 0 exactly
    zp_nib = np.empty((N, K // bs), dtype=np.uint8)
    zp_nib[:, 0::2] = p.zp & 15
    zp_nib[:, 1::2] = p.zp >> 4
    per_k = np.repeat(zp_nib, bs, axis=1)
    wz = (per_k[:, 0::2] | (per_k[:, 1::2] << 4)).astype(np.uint8)
    y0 = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.qgemv_int4_blockwise(f16_dev(p.x[:M]), to_dev(wz), f16_dev(p.scales), to_dev(p.zp), y0, bs)
    assert np.all(y_host(y0) == 0.0)
    # column permutation of (w, scales, zp) permutes y bitwise
    perm = np.random.default_rng(5).permutation(N)
    yp = torch.empty((M, N), dtype=torch.float32, device=DEV)
    q.qgemv_int4_blockwise(f16_dev(p.x[:M]), to_dev(p.w[perm]), f16_dev(p.scales[perm]),
                           to_dev(p.zp[perm]), yp, bs)
    assert np.array_equal(y_host(yp), base[:, perm])
    # row independence: M >= 3 here runs on the matrix cores (v_mfma), M = 1
    # and 2 on v_dot2; rows 0..2 of an M = 3 call equal those of an M = 4 call
    # bitwise (same kernel, rows of the MFMA A operand are independent), and
    # the v_dot2 calls agree to the tolerance
    yr, S = int4_ref(N, K, bs, True, 91)
    outs = {}
    for MM in (1, 2, 3, 4):
        yy = torch.empty((MM, N), dtype=torch.float32, device=DEV)
        q.qgemv_int4_blockwise(f16_dev(p.x[4:4 + MM]), to_dev(p.w), f16_dev(p.scales),
                               to_dev(p.zp), yy, bs)
        assert ("int4_mfma_" in q.last_launch()) == (MM >= 3), q.last_launch()
        outs[MM] = y_host(yy)
    assert np.array_equal(outs[3], outs[4][:3])
    assert_accept(outs[1], yr[4:5], S[4:5], "f32", "row 4, M=1")
    assert_accept(outs[2], yr[4:6], S[4:6], "f32", "rows 4..5, M=2")
    assert_accept(outs[4], yr[4:8], S[4:8], "f32", "rows 4..7, M=4")
    assert_accept(base, yr[:M], S[:M], "f32", "M=8")


# (K, block): K >= 1024 splits each 16-row tile over a workgroup's waves, K <
# 1024 gives each wave whole tiles; blocks 32 / 64 / >= 128 take the three
# scale layouts of the matrix-core kernel.
@pytest.mark.parametrize("K,bs", [(1024, 32), (1024, 64), (1024, 128), (512, 32), (512, 256)])
def test_one_hot_probe_matrix_core_path_is_bit_exact(K, bs):
    """M = 4 (v_mfma path): row r of x is one-hot at k_r; y[r, n] must equal the
    oracle's dequantized w[n, k_r] bitwise (fp32 out)."""
    N = 48
    p = int4_case(N, K, bs, True, 33)
    wdq = oracle.int4_dequant(p.w, p.scales, p.zp, N, K, bs)
    wd, sd, zd = to_dev(p.w), f16_dev(p.scales), to_dev(p.zp)
    ks = list(range(0, K, 3))
    say(f"int4 mfma one-hot probe K={K} bs={bs}: {len(ks)} positions")
    for i0 in range(0, len(ks), 4):
        kk = ks[i0:i0 + 4]
        M = len(kk)
        x = torch.zeros((M, K), dtype=torch.float16, device=DEV)
        for r, k in enumerate(kk):
            x[r, k] = 1.0
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        q.qgemv_int4_blockwise(x, wd, sd, zd, y, bs)
        got = y.cpu().numpy()
        want = wdq[:, kk].T.astype(np.float32)
        assert np.array_equal(got, want), kk
        nz = want != 0
        assert np.array_equal(got.view(np.uint32)[nz], want.view(np.uint32)[nz]), kk


@pytest.mark.parametrize("bs,asym,M", [(64, True, 4), (128, False, 5), (256, True, 8), (32, True, 2),
                                       (32, True, 3)])
def test_wide_matrix_sampled(bs, asym, M):
    # 65576 rows = 4099 tiles of 16: enough for every wave to own whole tiles
    N, K = 65576, 1024
    say(f"int4 wide N={N} K={K} bs={bs} asym={asym} M={M}")
    p = int4_case(N, K, bs, asym, 600 + bs)
    y = y_host(_run(p, M, torch.float32))
    rng = np.random.default_rng(3)
    cols = tuple(sorted(set(rng.integers(0, N, 500).tolist()) | {0, 15, 16, N - 1}))
    yr, S = int4_ref(N, K, bs, asym, 600 + bs, cols)
    assert_accept(y[:, list(cols)], yr[:M], S[:M], "f32", f"int4 wide bs={bs} M={M}")


@pytest.mark.parametrize("N,K,bs,mfma", [(4096, 4096, 128, True), (4100, 11008, 32, True),
                                         (2064, 4096, 64, True), (4096, 4096, 32, False),
                                         (1536, 6912, 128, True), (2048, 1536, 64, True),
                                         (1536, 4096, 32, False)])
def test_two_rows_kernel_choice(N, K, bs, mfma):
    """M = 2 runs on the matrix cores except with blocks of 32 along rows of at
    most 4096 weights (v_dot2); both kernels meet the tolerance on every
    column."""
    say(f"int4 M=2 N={N} K={K} bs={bs} mfma={mfma}")
    p = int4_case(N, K, bs, True, 740 + bs)
    y = y_host(_run(p, 2, torch.float32))
    assert ("int4_mfma_" in q.last_launch()) == mfma, q.last_launch()
    yr, S = int4_ref(N, K, bs, True, 740 + bs)
    assert_accept(y, yr[:2], S[:2], "f32", f"int4 M=2 {N}x{K} bs={bs}")


@pytest.mark.parametrize("N,K,bs,asym", [(4096, 11008, 32, False), (4100, 14336, 32, True),
                                         (4096, 4096, 128, True), (11008, 4096, 128, False),
                                         (6912, 1536, 64, True)])
def test_layer_shapes_single_row_sampled(N, K, bs, asym):
    # The single-row launch shapes of 7B-class layers: 512-thread workgroups
    # for rows of 8192 weights or more, lanes per row widened for short N, and
    # a ragged last tile (4100 rows).
    say(f"int4 layer N={N} K={K} bs={bs} asym={asym} M=1")
    p = int4_case(N, K, bs, asym, 700 + bs)
    y = y_host(_run(p, 1, torch.float32))
    rng = np.random.default_rng(5)
    cols = tuple(sorted(set(rng.integers(0, N, 400).tolist()) | {0, 1, 63, 64, N - 2, N - 1}))
    yr, S = int4_ref(N, K, bs, asym, 700 + bs, cols)
    assert_accept(y[:, list(cols)], yr[:1], S[:1], "f32", f"int4 layer {N}x{K} bs={bs}")


# At M = 1, rows of 2048, 4096 or 8192 weights, and the rows of matrices too
# short for the persistent kernel with P = K/32 pieces, 128 < P <= 512, take
# the span kernel (runs of 4, 2 or 1 whole rows per wavefront): ragged last
# spans (N not a multiple of the rows per span, down to N = 1), rows that end
# inside a wavefront's last piece (K = 4864, 6912, 8960, 11008, 13824), every
# U from 1 to 8, every block size, both zero-point modes and every output
# type, on every column.
@pytest.mark.parametrize("N,K,bs,asym,out_dtype", [
    (1, 2048, 32, True, torch.float32), (3, 4096, 64, False, torch.float16),
    (4099, 2048, 32, True, torch.bfloat16), (1001, 4096, 256, True, torch.float32),
    (517, 8192, 128, False, torch.float16), (2, 8192, 32, True, torch.float32),
    (9000, 4096, 32, True, torch.float16), (301, 6144, 64, True, torch.float32),
    (77, 8960, 128, True, torch.float32), (130, 10240, 256, False, torch.bfloat16),
    (513, 11008, 128, True, torch.float16), (5, 11008, 64, False, torch.float32),
    (260, 13824, 32, True, torch.float32), (97, 14336, 128, True, torch.float16),
    (33, 16384, 32, False, torch.float32), (896, 4864, 32, True, torch.float16),
    (1536, 6912, 128, False, torch.float32)])
def test_span_kernel_every_column(N, K, bs, asym, out_dtype):
    say(f"int4 span N={N} K={K} bs={bs} asym={asym} out={out_dtype}")
    p = int4_case(N, K, bs, asym, 900 + N % 97)
    y = y_host(_run(p, 1, out_dtype))
    assert q.last_launch().startswith("int4_span M=1 "), q.last_launch()
    yr, S = int4_ref(N, K, bs, asym, 900 + N % 97)
    assert_accept(y, yr[:1], S[:1], OUT_NAME[out_dtype], f"int4 span {N}x{K} bs={bs}")


def test_span_kernel_strided_unaligned_x_and_strided_y():
    N, K, bs = 777, 4096, 32
    say("int4 span strided/unaligned x, strided y")
    p = int4_case(N, K, bs, True, 56)
    buf = np.zeros(1 + (K + 3), dtype=np.uint16)
    buf[1:1 + K] = p.x[0]
    xt = f16_dev(buf)[1:].view(1, K + 3)[:, :K]
    assert xt.data_ptr() % 16 == 2
    y = y_host(_run(p, 1, torch.float16, x=xt, ldy=N + 3))
    assert q.last_launch().startswith("int4_span M=1 "), q.last_launch()
    yr, S = int4_ref(N, K, bs, True, 56)
    assert_accept(y, yr[:1], S[:1], "f16", "int4 span strided")


@pytest.mark.parametrize("K", [2048, 4096, 8192, 11008, 14336])
def test_span_kernel_one_hot_is_bit_exact(K):
    """x = e_k through the span kernel, fp32 out: y[n] equals the oracle's
    dequantized w[n,k] bitwise, for k at the edges of each lane's pieces."""
    N, bs = 70, 32
    p = int4_case(N, K, bs, True, 33)
    wdq = oracle.int4_dequant(p.w, p.scales, p.zp, N, K, bs)
    wd, sd, zd = to_dev(p.w), f16_dev(p.scales), to_dev(p.zp)
    ks = sorted({0, 1, 31, 32, 33, 2047, 2048 % K, 2049 % K, K // 2, K - 32, K - 1})
    say(f"int4 span one-hot K={K}, {len(ks)} columns of x")
    ys = torch.empty((len(ks), N), dtype=torch.float32, device=DEV)
    for i, k in enumerate(ks):
        x = torch.zeros((1, K), dtype=torch.float16, device=DEV)
        x[0, k] = 1.0
        q.qgemv_int4_blockwise(x, wd, sd, zd, ys[i:i + 1], bs)
        assert q.last_launch().startswith("int4_span M=1 "), q.last_launch()
    got = ys.cpu().numpy()
    want = wdq[:, ks].T.astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_misaligned_scales_and_zero_points():
    # scales 2 bytes past an 8-byte boundary and zero points at an odd address
    N, K, bs, M = 300, 1024, 32, 4
    say("int4 misaligned scales / zero points")
    p = int4_case(N, K, bs, True, 57)
    nb, zrow = K // bs, p.zp.shape[1]
    sbuf = f16_dev(np.concatenate([np.zeros(1, np.uint16), p.scales.reshape(-1)]))
    zbuf = to_dev(np.concatenate([np.zeros(1, np.uint8), p.zp.reshape(-1)]))
    sd, zd = sbuf[1:].view(N, nb), zbuf[1:].view(N, zrow)
    assert sd.data_ptr() % 8 == 2 and zd.data_ptr() % 2 == 1
    y = torch.full((M, N), float("nan"), dtype=torch.float32, device=DEV)
    q.qgemv_int4_blockwise(f16_dev(p.x[:M]), to_dev(p.w), sd, zd, y, bs)
    yr, S = int4_ref(N, K, bs, True, 57)
    assert_accept(y_host(y), yr[:M], S[:M], "f32", "int4 misaligned scales")


def test_empty_and_rejected_calls_on_device():
    p = int4_case(16, 64, 32, True, 3)
    say("int4 N=0 and M=9 on device")
    xd, wd, sd, zd = f16_dev(p.x[:1]), to_dev(p.w), f16_dev(p.scales), to_dev(p.zp)
    y = torch.full((1, 16), 7.0, dtype=torch.float16, device=DEV)
    L = q.load_library()
    st = torch.cuda.current_stream().cuda_stream
    assert L.qgemv_int4_blockwise(xd.data_ptr(), 64, 0, wd.data_ptr(), sd.data_ptr(),
                                  zd.data_ptr(), y.data_ptr(), 16, 0, 1, 0, 64, 32, st) == 0
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    with pytest.raises(q.QgemvError):
        x9 = torch.zeros((9, 64), dtype=torch.float16, device=DEV)
        y9 = torch.zeros((9, 16), dtype=torch.float16, device=DEV)
        q.qgemv_int4_blockwise(x9, wd, sd, zd, y9, 32)


def test_uses_current_stream():
    p = int4_case(256, 1536, 32, True, 101)
    xd, wd, sd, zd = f16_dev(p.x[:1]), to_dev(p.w), f16_dev(p.scales), to_dev(p.zp)
    y = torch.zeros((1, 256), dtype=torch.float16, device=DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    say("int4 current-stream")
    with torch.cuda.stream(s):
        torch.cuda._sleep(50_000_000)
        q.qgemv_int4_blockwise(xd, wd, sd, zd, y, 32)
        ev = torch.cuda.Event()
        ev.record(s)
    assert not ev.query(), "work did not go to the caller's stream"
    assert torch.cuda.default_stream().query()
    s.synchronize()
    yr, S = int4_ref(256, 1536, 32, True, 101)
    assert_accept(y_host(y), yr[:1], S[:1], "f16", "int4 stream")


@pytest.mark.parametrize("case", range(16))
def test_random_shapes_and_strides(case):
    """Seeded random block size, zero points, N, K, M, x row stride and base
    offset, y row stride and output type: the kernel choices (v_dot2 or
    matrix cores; whole, split, chunked or phased x) follow from the shape."""
    rng = np.random.default_rng(7000 + case)
    bs = [32, 64, 128][int(rng.integers(0, 3))]
    asym = bool(rng.integers(0, 2))
    N, M = int(rng.integers(1, 1500)), int(rng.integers(1, 9))
    K = bs * int(rng.integers(1, 6144 // bs + 1))
    ldx, offx = K + int(rng.integers(0, 12)), int(rng.integers(0, 3))
    ldy = N + int(rng.integers(0, 5))
    out_dtype = [torch.float16, torch.bfloat16, torch.float32][int(rng.integers(0, 3))]
    p = int4_case(N, K, bs, asym, 7100 + case)
    xrows = np.zeros((M, ldx), dtype=np.uint16)
    xrows[:, :K] = p.x[:M]
    xbuf = np.concatenate([np.zeros(offx, dtype=np.uint16), xrows.ravel()])
    xd = f16_dev(xbuf)[offx:].as_strided((M, K), (ldx, 1))
    say(f"int4 random N={N} K={K} bs={bs} asym={asym} M={M} ldx={ldx} offx={offx} ldy={ldy} "
        f"out={out_dtype}")
    y = _run(p, M, out_dtype, x=xd, ldy=ldy)
    yr, S = oracle.int4_gemv(xrows, p.w, p.scales, p.zp, M, N, K, bs, ldx=ldx)
    assert_accept(y_host(y), yr, S, OUT_NAME[out_dtype], f"int4 random case {case} ({q.last_launch()})")


# k parts of the split matrix-core kernel: where 16-row tiles leave CUs idle,
# the MFMA columns carry 8 rows in 2 parts of their k range (M <= 8) or 4 rows
# in 4 parts (M <= 4); the grid is one workgroup per tile of 16 / ks rows
# (rows of 12 items: 4 wavefronts per workgroup).
@pytest.mark.parametrize("N,K,bs,asym,M,ks", [(1000, 4096, 32, True, 3, 4),
                                              (1003, 4096, 64, True, 4, 4),
                                              (1003, 4096, 128, False, 4, 4),
                                              (777, 2048, 256, True, 6, 2),
                                              (250, 8192, 32, True, 5, 2),
                                              (1001, 2048, 64, True, 8, 2),
                                              (1536, 6912, 128, False, 7, 2),
                                              (1536, 1536, 128, False, 5, 2),
                                              (300, 1536, 32, True, 3, 2)])
def test_matrix_core_k_parts(N, K, bs, asym, M, ks):
    say(f"int4 matrix-core k parts N={N} K={K} bs={bs} asym={asym} M={M} ks={ks}")
    p = int4_case(N, K, bs, asym, 1500 + M)
    y = y_host(_run(p, M, torch.float32))
    tr = 16 // ks
    assert f"int4_mfma_split M={M} grid={(N + tr - 1) // tr} " in q.last_launch(), q.last_launch()
    yr, S = int4_ref(N, K, bs, asym, 1500 + M)
    assert_accept(y, yr[:M], S[:M], "f32", f"int4 k parts {N}x{K} M={M}")


@pytest.mark.parametrize("K,bs,M,ks", [(4096, 32, 4, 4), (4096, 64, 3, 4), (4096, 256, 4, 4),
                                       (2048, 32, 8, 2), (2048, 128, 5, 2), (8192, 64, 4, 4),
                                       (8192, 32, 6, 2), (1536, 64, 4, 2), (1536, 32, 7, 2)])
def test_one_hot_probe_k_parts_is_bit_exact(K, bs, M, ks):
    """Row r of x is one-hot at k_r (positions across every item and at item
    seams, so every part of every step is probed); y[r, n] must equal the
    oracle's dequantized w[n, k_r] bitwise (fp32 out)."""
    N = 203
    p = int4_case(N, K, bs, True, 35)
    wdq = oracle.int4_dequant(p.w, p.scales, p.zp, N, K, bs)
    wd, sd, zd = to_dev(p.w), f16_dev(p.scales), to_dev(p.zp)
    kpos = sorted(set(list(range(0, K, 29)) + [128 * i - 1 for i in range(1, K // 128)] +
                      [128 * i for i in range(K // 128)] + [K - 1]))
    say(f"int4 k-parts one-hot probe K={K} bs={bs} M={M}: {len(kpos)} positions")
    tr = 16 // ks
    for i0 in range(0, len(kpos), M):
        kk = kpos[i0:i0 + M]
        kk = kk + [kk[-1]] * (M - len(kk))
        x = torch.zeros((M, K), dtype=torch.float16, device=DEV)
        for r, k in enumerate(kk):
            x[r, k] = 1.0
        y = torch.empty((M, N), dtype=torch.float32, device=DEV)
        q.qgemv_int4_blockwise(x, wd, sd, zd, y, bs)
        assert f"int4_mfma_split M={M} grid={(N + tr - 1) // tr} " in q.last_launch(), q.last_launch()
        got = y.cpu().numpy()
        want = wdq[:, kk].T.astype(np.float32)
        assert np.array_equal(got, want), kk
        nz = want != 0
        assert np.array_equal(got.view(np.uint32)[nz], want.view(np.uint32)[nz]), kk


def test_k_parts_strided_unaligned_x_and_strided_y():
    """The k-part split kernel (4 parts: 1003 rows, M = 4) with x rows at a
    2-byte offset and ldx = K + 3 (x staged element-wise) and y rows of
    stride N + 5."""
    N, K, bs, M = 1003, 4096, 64, 4
    say("int4 k parts, unaligned strided x, strided y")
    p = int4_case(N, K, bs, True, 1590)
    yr, S = int4_ref(N, K, bs, True, 1590)
    buf = np.zeros(1 + M * (K + 3), dtype=np.uint16)
    for m in range(M):
        buf[1 + m * (K + 3):1 + m * (K + 3) + K] = p.x[m]
    xt = f16_dev(buf)[1:].view(M, K + 3)[:, :K]
    assert xt.data_ptr() % 16 == 2
    y = y_host(_run(p, M, torch.float32, x=xt, ldy=N + 5))
    assert f"int4_mfma_split M={M} grid={(N + 3) // 4} " in q.last_launch(), q.last_launch()
    assert_accept(y, yr[:M], S[:M], "f32", "int4 k parts strided")

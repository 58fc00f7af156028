"""GPU checks of the load-time packed int4 layout (int4_repack,
qgemv_int4_packed) on MI355X.

The repack is compared byte for byte with the layout's definition (restated
here with NumPy index arithmetic from include/qgemv.h, independent of the
kernel); the GEMV on packed weights is compared with the fp64 oracle on the
original layout -- every column, every block size, M = 1..8, ragged tiles,
rows shorter than 8 items (fewer wavefronts per tile), strided x and y, every
output type -- and with one-hot x it must reproduce the oracle's dequantized
weights bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import weight_only_quantized_int4_amd as q
from gpu_cases import (DEV, OUT_NAME, assert_accept, f16_dev, int4_case, int4_ref,
                       int4_ref_all, say, to_dev, y_host)

pytestmark = pytest.mark.gpu


def _packed_expected(p, N, K, bs):
    """The QG_INT4_LAYOUT_TILE16_V1 bytes of (p.w, p.scales, p.zp)."""
    nbi = max(1, 128 // bs)
    T, C = (N + 15) // 16, K // 128
    zb = 32 if nbi == 4 else 16
    rb = 1024 + 32 * nbi + zb
    nb = K // bs
    out = np.zeros((T, C, rb), np.uint8)
    wpad = np.zeros((T * 16, K // 2), np.uint8)
    wpad[:N] = p.w
    # word index of row byte 64c + 16j + 4g is 16c + 4j + g
    words = wpad.view("<u4").reshape(T, 16, C, 4, 4)          # (t, n, c, j, g)
    lanes = words.transpose(0, 2, 4, 1, 3)                      # (t, c, g, n, j): lane 16g + n
    out[:, :, :1024] = np.ascontiguousarray(lanes).view(np.uint8).reshape(T, C, 1024)
    spad = np.zeros((T * 16, nb), np.uint16)
    spad[:N] = p.scales
    zpad = np.full((T * 16, nb), 8, np.uint8)
    if p.zp is not None:
        blk = np.arange(nb)
        zpad[:N] = (p.zp[:, blk // 2] >> (4 * (blk % 2))) & 15
    zpad[N:] = 0
    first = (128 * np.arange(C)) // bs                          # first block of item c
    idx = first[:, None] + np.arange(nbi)[None, :]              # (c, b)
    sc = spad[:, idx].reshape(T, 16, C, nbi).transpose(0, 2, 1, 3)   # (t, c, n, b)
    out[:, :, 1024:1024 + 32 * nbi] = np.ascontiguousarray(sc).view(np.uint8).reshape(T, C, -1)
    zz = zpad[:, idx].reshape(T, 16, C, nbi).transpose(0, 2, 1, 3).astype(np.uint32)
    bits = np.zeros((T, C, 16), np.uint32)
    for b in range(nbi):
        bits |= zz[..., b] << (4 * b)
    zrow = 2 if nbi == 4 else 1
    zbytes = np.zeros((T, C, 16, zrow), np.uint8)
    zbytes[..., 0] = bits & 0xFF
    if zrow == 2:
        zbytes[..., 1] = bits >> 8
    out[:, :, 1024 + 32 * nbi:1024 + 32 * nbi + 16 * zrow] = zbytes.reshape(T, C, 16 * zrow)
    return out.reshape(-1)


def _pack(p, N, K, bs):
    nbytes = q.int4_packed_bytes(N, K, bs)
    assert nbytes > 0
    packed = torch.full((nbytes,), 0xA5, dtype=torch.uint8, device=DEV)
    zd = None if p.zp is None else to_dev(p.zp)
    q.int4_repack(to_dev(p.w), f16_dev(p.scales), zd, packed, bs)
    return packed


def _run(packed, p, M, bs, out_dtype=torch.float16, x=None, ldy=None):
    xd = f16_dev(p.x[:M]) if x is None else x
    if ldy is None:
        y = torch.full((M, p.N), float("nan"), dtype=out_dtype, device=DEV)
    else:
        y = torch.full((M, ldy), float("nan"), dtype=out_dtype, device=DEV)[:, :p.N]
    q.qgemv_int4_packed(xd, packed, y, bs)
    assert q.last_launch().startswith(f"int4_packed M="), q.last_launch()
    return y


@pytest.mark.parametrize("bs,asym", [(32, True), (64, True), (128, False), (256, True)])
def test_repack_matches_the_layout_definition(bs, asym):
    N, K = 37, 1024
    say(f"int4 repack layout N={N} K={K} bs={bs} asym={asym}")
    p = int4_case(N, K, bs, asym, 1200 + bs)
    got = _pack(p, N, K, bs).cpu().numpy()
    want = _packed_expected(p, N, K, bs)
    assert got.shape == want.shape
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8]}"


@pytest.mark.parametrize("N,K,bs,asym", [
    (256, 1536, 32, True), (1536, 1536, 128, False), (1536, 6912, 128, False),
    (300, 1024, 64, True), (33, 256, 256, True), (17, 384, 128, True), (1000, 2048, 32, True),
    (50, 128, 32, False)])
@pytest.mark.parametrize("M", list(range(1, 9)))
def test_packed_gemv_every_column(N, K, bs, asym, M):
    say(f"int4 packed N={N} K={K} bs={bs} asym={asym} M={M}")
    p = int4_case(N, K, bs, asym, 1300 + N % 89)
    packed = _pack(p, N, K, bs)
    y = y_host(_run(packed, p, M, bs, torch.float32))
    yr, S = int4_ref(N, K, bs, asym, 1300 + N % 89)
    assert_accept(y, yr[:M], S[:M], "f32", f"int4 packed {N}x{K} bs={bs} M={M}")


@pytest.mark.parametrize("bs", [32, 64, 128, 256])
def test_packed_one_hot_is_bit_exact(bs):
    """x = e_k in one row of x (M = 3), fp32 out: y equals the oracle's
    dequantized w[n, k] bitwise, and the other rows are exactly 0."""
    N, K = 40, 1024
    p = int4_case(N, K, bs, True, 1400 + bs)
    wdq = oracle.int4_dequant(p.w, p.scales, p.zp, N, K, bs)
    packed = _pack(p, N, K, bs)
    ks = sorted({0, 1, 7, 8, 31, 32, 127, 128, 255, 256, 511, 640, K - 1})
    say(f"int4 packed one-hot bs={bs}, {len(ks)} columns")
    for k in ks:
        x = torch.zeros((3, K), dtype=torch.float16, device=DEV)
        x[1, k] = 1.0
        y = torch.empty((3, N), dtype=torch.float32, device=DEV)
        q.qgemv_int4_packed(x, packed, y, bs)
        got = y.cpu().numpy()
        want = wdq[:, k].astype(np.float32)
        assert np.array_equal(got[1].view(np.uint32), want.view(np.uint32)), k
        assert not got[0].any() and not got[2].any(), k


@pytest.mark.parametrize("M", [1, 8])
def test_packed_lm_head_every_column(M):
    N, K = 151936, 4096
    say(f"int4 packed lm_head M={M}")
    p = int4_case(N, K, 32, True, 501)
    packed = _pack(p, N, K, 32)
    y = y_host(_run(packed, p, M, 32))
    yr, S = int4_ref_all(N, K, 32, True, 501)
    assert_accept(y, yr[:M], S[:M], "f16", f"int4 packed lm_head M={M} ({q.last_launch()})")


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.bfloat16, torch.float32])
def test_packed_strided_unaligned_x_and_strided_y(out_dtype):
    N, K, bs, M = 301, 1024, 32, 5
    say(f"int4 packed strided x/y out={out_dtype}")
    p = int4_case(N, K, bs, True, 55)
    buf = np.zeros(1 + M * (K + 3), dtype=np.uint16)
    for m in range(M):
        buf[1 + m * (K + 3):1 + m * (K + 3) + K] = p.x[m]
    xt = f16_dev(buf)[1:].view(M, K + 3)[:, :K]
    assert xt.data_ptr() % 16 == 2
    packed = _pack(p, N, K, bs)
    y = y_host(_run(packed, p, M, bs, out_dtype, x=xt, ldy=N + 5))
    yr, S = int4_ref(N, K, bs, True, 55)
    assert_accept(y, yr[:M], S[:M], OUT_NAME[out_dtype], "int4 packed strided")


def _unaligned_x(p, M, K):
    """x[:M] as a view whose rows start 2 bytes past a 16-byte boundary."""
    buf = np.zeros(1 + M * K, dtype=np.uint16)
    buf[1:] = p.x[:M].reshape(-1)
    xt = f16_dev(buf)[1:].view(M, K)
    assert xt.data_ptr() % 16 == 2
    return xt


def test_packed_rows_of_x_in_groups():
    """K = 16384 at M = 8 with x not 16-byte aligned: x is staged in LDS,
    where it does not fit at once, so the rows run in groups (each a
    launch)."""
    N, K, bs, M = 100, 16384, 128, 8
    say(f"int4 packed row groups N={N} K={K} M={M}")
    p = int4_case(N, K, bs, True, 71)
    packed = _pack(p, N, K, bs)
    y = y_host(_run(packed, p, M, bs, torch.float32, x=_unaligned_x(p, M, K)))
    assert q.last_launch().count("int4_packed") >= 2, q.last_launch()
    yr, S = int4_ref(N, K, bs, True, 71)
    assert_accept(y, yr[:M], S[:M], "f32", "int4 packed row groups")


@pytest.mark.parametrize("N,K,bs,M", [(100, 16384, 128, 8), (4100, 11008, 32, 8),
                                      (300, 32768, 64, 5)])
def test_packed_x_from_global_memory_any_row_length(N, K, bs, M):
    """Aligned x whose rows LDS cannot hold reads the A operands from global
    memory: one launch, no workgroup LDS for x."""
    say(f"int4 packed x from global N={N} K={K} bs={bs} M={M}")
    p = int4_case(N, K, bs, True, 72)
    packed = _pack(p, N, K, bs)
    y = y_host(_run(packed, p, M, bs, torch.float32))
    launch = q.last_launch()
    assert launch.count("int4_packed") == 1, launch
    assert int(launch.split("lds=")[1].split()[0]) <= 16 * 1024, launch
    yr, S = int4_ref(N, K, bs, True, 72)
    assert_accept(y, yr[:M], S[:M], "f32", f"int4 packed x from global {N}x{K}")


@pytest.mark.parametrize("N,K,bs", [(1536, 16384, 128), (37, 12288, 32)])
def test_packed_x_staged_and_x_from_global_agree(N, K, bs):
    """The same problem (M = 8 rows of x, more than LDS holds) with 16-byte
    aligned x (A operands from global memory, one launch) and with unaligned
    x (staged in LDS, groups of rows): both within the bound of the oracle,
    and equal to each other bit for bit (the same MFMA chain per row)."""
    M = 8
    say(f"int4 packed staged vs global x N={N} K={K} bs={bs}")
    p = int4_case(N, K, bs, True, 73)
    packed = _pack(p, N, K, bs)
    ya = _run(packed, p, M, bs, torch.float32)
    la = q.last_launch()
    yb = _run(packed, p, M, bs, torch.float32, x=_unaligned_x(p, M, K))
    lb = q.last_launch()
    assert la != lb, (la, lb)
    yr, S = int4_ref(N, K, bs, True, 73)
    assert_accept(y_host(ya), yr[:M], S[:M], "f32", "int4 packed x from global")
    assert_accept(y_host(yb), yr[:M], S[:M], "f32", "int4 packed staged x")
    assert torch.equal(ya.cpu().view(torch.int32), yb.cpu().view(torch.int32))


def test_packed_is_deterministic():
    """Two calls on the same packed weights give identical bits."""
    N, K, bs, M = 700, 2048, 64, 4
    p = int4_case(N, K, bs, True, 88)
    packed = _pack(p, N, K, bs)
    a = _run(packed, p, M, bs, torch.float32).cpu()
    b = _run(packed, p, M, bs, torch.float32).cpu()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))

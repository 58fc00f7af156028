"""Pins of the fp64 CPU oracle against facts fixed outside the oracle itself.

Each test ties a part of ``oracle/`` to something it could get wrong on its own:
values worked by hand from the pages' formulas (``tests/golden/``), library
routines for the number formats (NumPy's fp16, torch's bfloat16), exact integer
arithmetic on tiny brute-force cases, invariants of the definition, and an
independently written NumPy decoder.  CPU only.
"""
import json
import os

import numpy as np
import pytest
import torch

import datagen
import oracle
from oracle import numpy_cross as npx

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _f32_bits(v):
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_f16_decode_every_pattern(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signed zero survives
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_bf16_decode_every_pattern(oracle_lib):
    bits = np.arange(65536, dtype=np.int64)
    t = torch.from_numpy(bits.astype(np.int32).astype(np.int16)).view(torch.bfloat16)
    want = t.to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(int(b)) for b in bits])
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])


def test_round_f16_matches_numpy(oracle_lib):
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(4000) * 10.0 ** rng.integers(-9, 5, 4000),
        # exact ties between neighbouring fp16 values, and the overflow edge
        (np.arange(1024, 2048, dtype=np.float64) + 0.5) * 2.0 ** -10,
        np.array([65504.0, 65519.999, 65520.0, 2.0 ** -25, 3 * 2.0 ** -26, 1e-9, 0.0, -0.0]),
    ])
    for v in vals:
        want = float(np.float64(v).astype(np.float16))
        got = oracle.round_to(v, "f16")
        assert got == want and np.signbit(got) == np.signbit(want), (v, got, want)


def test_round_bf16_matches_torch(oracle_lib):
    rng = np.random.default_rng(8)
    vals = (rng.standard_normal(4000) * 10.0 ** rng.integers(-30, 30, 4000)).astype(np.float32)
    vals = np.concatenate([vals, np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float32)])
    want = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    for v, w in zip(vals, want):
        assert oracle.round_to(float(v), "bf16") == w, v


def test_round_f32_matches_numpy(oracle_lib):
    """binary32 rounding against NumPy's float64 -> float32 cast (IEEE
    round-to-nearest-even): random values over the whole range, exact ties
    between neighbouring normal and subnormal values (even neighbour wins),
    the subnormal and overflow edges, and signed zeros."""
    rng = np.random.default_rng(9)
    rand = rng.standard_normal(6000) * 10.0 ** rng.integers(-46, 39, 6000)
    i = np.arange(0, 600, dtype=np.float64)
    ties_normal = np.concatenate([(2.0 ** 23 + i + 0.5) * 2.0 ** (e - 23) for e in (-126, -3, 0, 77)])
    ties_sub = (i + 0.5) * 2.0 ** -149
    tiny = np.array([2.0 ** -150, 3 * 2.0 ** -151, 2.0 ** -149, 2.0 ** -126 * (1 - 2.0 ** -25),
                     1e-46, 1e-45])
    maxf = float(np.finfo(np.float32).max)
    big = np.array([maxf, maxf + 2.0 ** 103, maxf + 2.0 ** 103 - 2.0 ** 60, 2.0 ** 128, 1e39,
                    3.4e38])
    vals = np.concatenate([rand, ties_normal, ties_sub, tiny, big, [0.0, -0.0]])
    vals = np.concatenate([vals, -vals])
    with np.errstate(over="ignore"):
        want_all = vals.astype(np.float32).astype(np.float64)
    for v, want in zip(vals, want_all):
        got = oracle.round_to(float(v), "f32")
        assert got == want and np.signbit(got) == np.signbit(want), (v, got, want)


def test_ulp_values(oracle_lib):
    assert oracle.ulp(1.0, "f16") == 2.0 ** -10
    assert oracle.ulp(1.999, "f16") == 2.0 ** -10
    assert oracle.ulp(65504.0, "f16") == 32.0
    assert oracle.ulp(1e-6, "f16") == 2.0 ** -24
    assert oracle.ulp(0.0, "f16") == 2.0 ** -24
    assert oracle.ulp(-3.0, "bf16") == 2.0 ** -6
    assert oracle.ulp(1.0, "f32") == 2.0 ** -23
    assert oracle.ulp(0.0, "f32") == 2.0 ** -149


# ---------------------------------------------------------------------------
# q4_K: get_scale_min_k4, plane values, weights
# ---------------------------------------------------------------------------

def test_q4k_scale_min_worked_example(oracle_lib):
    g = _gold("q4k_worked_example.json")
    sc = bytes(g["scale_bytes"])
    assert sc.hex().upper() == g["scale_bytes_hex"]
    for cc, sm in enumerate(g["scale_min_per_chunk"]):
        assert oracle.q4k_scale_min(sc, cc) == tuple(sm), cc
    for cc in range(8):
        assert oracle.q4k_scale_min(b"\xff" * 12, cc) == tuple(g["all_ff_scale_min"])
        assert oracle.q4k_scale_min(b"\x00" * 12, cc) == tuple(g["all_00_scale_min"])


def _bitmap_expectation():
    """(byte, bit) -> (field, chunk, field_bit), read from the golden rules."""
    rules = _gold("q4k_scale_bitmap.json")["rules"]
    out = {}
    for r in rules:
        for byte in r["bytes"]:
            for bit in range(r["bits"][0], r["bits"][1] + 1):
                chunk = eval(r["chunk"], {}, {"byte": byte})  # noqa: S307 (fixture arithmetic)
                fbit = eval(r["field_bit"], {}, {"bit": bit})  # noqa: S307
                out[(byte, bit)] = (r["field"], chunk, fbit)
    return out


def test_q4k_scale_min_bit_map_is_the_documented_bijection(oracle_lib):
    expect = _bitmap_expectation()
    assert len(expect) == 96
    seen = set()
    for byte in range(12):
        for bit in range(8):
            sc = bytearray(12)
            sc[byte] = 1 << bit
            lit = []
            for cc in range(8):
                s, m = oracle.q4k_scale_min(bytes(sc), cc)
                if s:
                    lit.append(("s", cc, s))
                if m:
                    lit.append(("m", cc, m))
            assert len(lit) == 1, (byte, bit, lit)
            field, cc, value = lit[0]
            assert value & (value - 1) == 0 and value < 64
            got = (field, cc, value.bit_length() - 1)
            assert got == expect[(byte, bit)], (byte, bit, got)
            seen.add(got)
    assert len(seen) == 96  # every bit of the sixteen 6-bit fields is reached once


def _one_block(d_bits, dmin_bits, sc, qs=None):
    qs = bytes(128) if qs is None else qs
    raw = (int(d_bits).to_bytes(2, "little") + int(dmin_bits).to_bytes(2, "little")
           + bytes(sc) + bytes(qs))
    return np.frombuffer(raw, dtype=np.uint8).copy().reshape(1, 144)


def test_q4k_plane_values_worked_example(oracle_lib):
    g = _gold("q4k_worked_example.json")
    w = _one_block(g["d_bits"], g["dmin_bits"], g["scale_bytes"])
    assert oracle.f16_to_f64(g["d_bits"]) == g["d_value"]
    assert oracle.f16_to_f64(g["dmin_bits"]) == g["dmin_value"]
    plane = oracle.q4k_build_plane(w, 1, 256)
    bits = plane.view(np.uint32)
    for cc, (dv_hex, mv_hex) in enumerate(g["plane_f32_bits_per_chunk"]):
        assert oracle.q4k_coeffs(w, 256, 0, cc) == (int(dv_hex, 16), int(mv_hex, 16))
        assert (int(bits[cc, 0]), int(bits[cc, 1])) == (int(dv_hex, 16), int(mv_hex, 16))


def test_q4k_plane_minus_zero(oracle_lib):
    g = _gold("q4k_worked_example.json")
    # all mins zero -> mv is -0.0 (exact negation, not 0 - x)
    w = _one_block(g["d_bits"], g["dmin_bits"], bytes(12))
    plane = oracle.q4k_build_plane(w, 1, 256).view(np.uint32)
    assert all(int(v) == int(g["minus_zero_mv_bits"], 16) for v in plane[:, 1])
    # dmin == 0 with nonzero mins -> -0.0 as well
    w = _one_block(g["d_bits"], 0, b"\xff" * 12)
    plane = oracle.q4k_build_plane(w, 1, 256).view(np.uint32)
    assert all(int(v) == 0x80000000 for v in plane[:, 1])


def test_q4k_weights_worked_example(oracle_lib):
    g = _gold("q4k_worked_example.json")
    for case in g["weights"]:
        cc, q = case["chunk"], case["q"]
        # place code q at element l = 3 of chunk cc (GGUF order: low nibble for
        # even chunks, high nibble for odd chunks, byte 32*(cc//2) + l)
        qs = bytearray(128)
        qs[32 * (cc // 2) + 3] = q if cc % 2 == 0 else (q << 4)
        w = _one_block(g["d_bits"], g["dmin_bits"], g["scale_bytes"], qs)
        k = 32 * cc + 3
        assert oracle.lib().oracle_q4k_weight(w.ctypes.data, 256, 0, k) == case["w"]


def test_q4k_nibble_order_convention(oracle_lib):
    """GGUF order (parity unpinned by the pages; convention): element 64g+l is the
    low nibble of qs[32g+l], element 64g+32+l its high nibble."""
    qs = bytes(range(128))
    w = _one_block(0x3C00, 0, bytes(12), qs)
    L = oracle.lib()
    for e in range(256):
        g, r = divmod(e, 64)
        byte = 32 * g + (r % 32)
        want = (byte & 0x0F) if r < 32 else (byte >> 4)
        assert L.oracle_q4k_code(w.ctypes.data, 256, 0, e) == want, e


# ---------------------------------------------------------------------------
# int4
# ---------------------------------------------------------------------------

def test_int4_worked_example(oracle_lib):
    g = _gold("int4_worked_example.json")
    L = oracle.lib()
    K, bs = 64, 32
    w = np.zeros((1, K // 2), dtype=np.uint8)
    w[0, 0] = g["code_byte"]
    scales = np.array([[g["scale_bits"], 0x3C00]], dtype=np.uint16)
    zp = np.array([[g["zp_byte"]]], dtype=np.uint8)
    assert [L.oracle_int4_code(w.ctypes.data, K, 0, k) for k in (0, 1)] == g["codes_low_first"]
    assert [L.oracle_int4_zero_point(zp.ctypes.data, K, bs, 0, b) for b in (0, 1)] == g["zp_blocks"]
    assert oracle.f16_to_f64(g["scale_bits"]) == g["scale_value"]
    wd = oracle.int4_dequant(w, scales, zp, 1, K, bs)
    assert list(wd[0, :2]) == g["weights_block0"]
    # block 1 uses zero point 3 and scale 1.0; its codes are 0
    assert np.all(wd[0, 32:] == -3.0)
    assert oracle.f16_to_f64(g["f16_0p01_bits"]) == g["f16_0p01_as_f32"]
    assert np.float32(g["f16_0p01_as_f32"]) == g["f16_0p01_as_f32"]


def test_int4_symmetric_default_zero_point(oracle_lib):
    L = oracle.lib()
    assert L.oracle_int4_zero_point(None, 128, 32, 5, 3) == 8


def test_int4_odd_block_count_padding_is_ignored(oracle_lib):
    N, K, bs = 2, 96, 32  # 3 blocks -> 2 zero-point bytes per row, top nibble padding
    rng = np.random.default_rng(3)
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = np.full((N, 3), 0x3C00, dtype=np.uint16)
    zp = rng.integers(0, 256, (N, 2), dtype=np.uint8)
    zp2 = zp.copy()
    zp2[:, 1] ^= 0xF0
    a = oracle.int4_dequant(w, scales, zp, N, K, bs)
    b = oracle.int4_dequant(w, scales, zp2, N, K, bs)
    assert np.array_equal(a, b)
    assert oracle.int4_zp_row_bytes(96, 32) == 2


def test_int4_one_hot_positions(oracle_lib):
    """A single non-neutral nibble moves exactly one weight, at the documented k."""
    N, K, bs = 3, 128, 32
    w = np.full((N, K // 2), 0x88, dtype=np.uint8)       # every code 8
    zp = np.full((N, 2), 0x88, dtype=np.uint8)            # every zero point 8
    scales = np.full((N, 4), 0x3C00, dtype=np.uint16)
    assert np.all(oracle.int4_dequant(w, scales, zp, N, K, bs) == 0.0)
    for (n, byte, hi) in [(0, 0, False), (1, 17, True), (2, 63, True), (2, 40, False)]:
        w2 = w.copy()
        w2[n, byte] = 0x8F if not hi else 0xF8
        d = oracle.int4_dequant(w2, scales, zp, N, K, bs)
        nz = np.argwhere(d != 0)
        assert nz.tolist() == [[n, 2 * byte + int(hi)]]
        assert d[n, 2 * byte + int(hi)] == 7.0
    # zero point of block 3 of row 1 (high nibble of byte 1)
    zp2 = zp.copy()
    zp2[1, 1] = 0x28
    d = oracle.int4_dequant(w, scales, zp2, N, K, bs)
    assert np.array_equal(np.argwhere(d != 0)[:, 1], np.arange(96, 128))
    assert np.all(d[1, 96:] == 6.0)


# ---------------------------------------------------------------------------
# brute force: integer-valued problems against exact Python integers
# ---------------------------------------------------------------------------

def _exact_int_matmul(x_int, w_int):
    M, K = len(x_int), len(x_int[0])
    return [[sum(int(x_int[m][k]) * int(w_int[n][k]) for k in range(K))
             for n in range(len(w_int))] for m in range(M)]


@pytest.mark.parametrize("N,K,bs", [(1, 32, 32), (2, 64, 32), (3, 128, 64), (2, 256, 128)])
def test_int4_bruteforce_integer(oracle_lib, N, K, bs):
    rng = np.random.default_rng(N * 1000 + K)
    w = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    zp = np.zeros((N, (K // bs + 1) // 2), dtype=np.uint8)   # zero point 0 -> w = q
    scales = np.full((N, K // bs), 0x3C00, dtype=np.uint16)  # scale 1.0
    M = 8
    x_int = rng.integers(-4, 5, (M, K))
    x = x_int.astype(np.float16).view(np.uint16).copy()
    codes = [[(int(w[n, k // 2]) >> (4 * (k % 2))) & 15 for k in range(K)] for n in range(N)]
    want = _exact_int_matmul(x_int.tolist(), codes)
    y, S = oracle.int4_gemv(x, w, scales, zp, M, N, K, bs)
    assert y.tolist() == [[float(v) for v in row] for row in want]


@pytest.mark.parametrize("N,K", [(1, 256), (3, 512)])
def test_q4k_bruteforce_integer(oracle_lib, N, K):
    """d = 1, every scale 1, every min 0  =>  w = q exactly."""
    rng = np.random.default_rng(K + N)
    nsb = K // 256
    sc = bytes([1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1])
    blocks = []
    for _ in range(N * nsb):
        blocks.append(_one_block(0x3C00, 0x3C00, sc, rng.integers(0, 256, 128, dtype=np.uint8).tobytes()))
    w = np.concatenate(blocks).reshape(N, nsb * 144)
    M = 8
    x_int = rng.integers(-4, 5, (M, K))
    x = x_int.astype(np.float32)
    codes = []
    for n in range(N):
        row = []
        for k in range(K):
            sb, e = divmod(k, 256)
            g, r = divmod(e, 64)
            byte = int(w[n, sb * 144 + 16 + 32 * g + (r % 32)])
            row.append(byte & 15 if r < 32 else byte >> 4)
        codes.append(row)
    want = _exact_int_matmul(x_int.tolist(), codes)
    y, _ = oracle.q4k_gemv(x, w, M, N, K)
    assert y.tolist() == [[float(v) for v in row] for row in want]


def test_bf16_bruteforce_integer(oracle_lib):
    rng = np.random.default_rng(11)
    N, K, M = 3, 37, 5
    w_int = rng.integers(-8, 9, (N, K))
    x_int = rng.integers(-4, 5, (M, K))
    w = torch.from_numpy(w_int.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    x = torch.from_numpy(x_int.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    y, _ = oracle.bf16_gemv(x, w, M, N, K, K, K)
    assert y.tolist() == [[float(v) for v in row] for row in _exact_int_matmul(x_int.tolist(), w_int.tolist())]


# ---------------------------------------------------------------------------
# invariants of the definition
# ---------------------------------------------------------------------------

def test_invariants_zero_weights(oracle_lib):
    import datagen
    p = datagen.int4_problem(4, 256, 32, True, seed=5)
    # every code equal to its block's zero point -> y == 0 exactly
    zp_nib = np.empty((4, 8), dtype=np.uint8)
    zp_nib[:, 0::2] = p.zp & 15
    zp_nib[:, 1::2] = p.zp >> 4
    per_k = np.repeat(zp_nib, 32, axis=1)
    w = (per_k[:, 0::2] | (per_k[:, 1::2] << 4)).astype(np.uint8)
    y, S = oracle.int4_gemv(p.x, w, p.scales, p.zp, 8, 4, 256, 32)
    assert np.all(y == 0.0) and np.all(S == 0.0)
    # q4_K: every quant 0 and every min 0 -> y == 0
    q = datagen.q4k_problem(3, 512, seed=6)
    wq = q.w.reshape(3, 2, 144).copy()
    wq[:, :, 16:] = 0
    wq[:, :, 8:12] = 0            # mins of chunks 0..3 (and top bits of 4..7)
    wq[:, :, 12:16] &= 0x0F       # mins of chunks 4..7 (low bits)
    wq = wq.reshape(3, 288)
    y, _ = oracle.q4k_gemv(q.x, wq, 8, 3, 512)
    assert np.all(y == 0.0)


def test_q4k_exactly_zero_weights(oracle_lib):
    """q4_K weights that are exactly zero with nonzero coefficients: every
    chunk has quant q, scale sc and min m = sc*q with d = dmin, so
    w = d*sc*q - d*m = 0 exactly.  The definition gives y = 0 and S = 0; with
    some chunks random instead, the zero chunks add nothing."""
    from q4k_cases import pack_scale_min, zero_weight_rows

    rng = np.random.default_rng(11)
    for _ in range(20):
        sc, m = rng.integers(0, 64, 8), rng.integers(0, 64, 8)
        packed = pack_scale_min(sc, m)
        for cc in range(8):
            assert oracle.q4k_scale_min(packed, cc) == (sc[cc], m[cc])
    N, K = 6, 512
    w = zero_weight_rows(N, K, seed=12)
    assert np.all(oracle.q4k_dequant(w, N, K) == 0.0)
    x = rng.standard_normal((3, K)).astype(np.float32)
    y, S = oracle.q4k_gemv(x, w, 3, N, K)
    assert np.all(y == 0.0) and np.all(S == 0.0)
    plane = oracle.q4k_build_plane(w, N, K)
    assert np.all(plane[:, 0] > 0.0) and np.all(plane[:, 1] < 0.0)
    y2, S2 = oracle.q4k_plane_gemv(x, w, plane, 3, N, K)
    assert np.all(y2 == 0.0) and np.all(S2 == 0.0)
    # half of the chunks random: the degenerate ones contribute nothing
    wm = zero_weight_rows(N, K, seed=13, zero_frac=[0.5] * N)
    dq = oracle.q4k_dequant(wm, N, K).reshape(N, K // 32, 32)
    zero_chunks = np.all(dq == 0.0, axis=2)
    assert 0 < zero_chunks.sum() < zero_chunks.size
    ym, Sm = oracle.q4k_gemv(x, wm, 3, N, K)
    keep = np.repeat(~zero_chunks, 32, axis=1)
    assert np.allclose(ym, (x.astype(np.float64) @ (dq.reshape(N, K) * keep).T), rtol=1e-12, atol=0)


def test_invariants_sign_and_scale(oracle_lib):
    import datagen
    p = datagen.int4_problem(5, 128, 32, True, seed=9)
    y, S = oracle.int4_gemv(p.x, p.w, p.scales, p.zp, 8, 5, 128, 32)
    xneg = p.x ^ np.uint16(0x8000)
    y2, S2 = oracle.int4_gemv(xneg, p.w, p.scales, p.zp, 8, 5, 128, 32)
    assert np.array_equal(y2, -y) and np.array_equal(S2, S)
    # doubling every scale doubles y (fp16 exponent +1, no overflow at these values)
    s2 = (p.scales + np.uint16(0x0400)).astype(np.uint16)
    y3, _ = oracle.int4_gemv(p.x, p.w, s2, p.zp, 8, 5, 128, 32)
    assert np.array_equal(y3, 2 * y)


def test_column_subset_matches_full(oracle_lib):
    import datagen
    q = datagen.q4k_problem(7, 512, seed=12)
    y, S = oracle.q4k_gemv(q.x, q.w, 3, 7, 512)
    ys, Ss = oracle.q4k_gemv(q.x, q.w, 3, 7, 512, cols=[6, 0, 3])
    assert np.array_equal(ys, y[:, [6, 0, 3]]) and np.array_equal(Ss, S[:, [6, 0, 3]])


def test_plane_gemv_equals_direct(oracle_lib):
    import datagen
    q = datagen.q4k_problem(6, 768, seed=13)
    plane = oracle.q4k_build_plane(q.w, 6, 768)
    assert plane.shape == (768 // 32 * 6, 2)
    y1, s1 = oracle.q4k_gemv(q.x, q.w, 8, 6, 768)
    y2, s2 = oracle.q4k_plane_gemv(q.x, q.w, plane, 8, 6, 768)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


# ---------------------------------------------------------------------------
# the independently written NumPy decoder
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,K,bs,asym", [(1, 32, 32, True), (3, 96, 32, True), (4, 256, 64, False),
                                         (2, 512, 128, True), (3, 512, 256, False)])
def test_int4_against_numpy_cross_oracle(oracle_lib, N, K, bs, asym):
    import datagen
    p = datagen.int4_problem(N, K, bs, asym, seed=N + K + bs)
    wd_c = oracle.int4_dequant(p.w, p.scales, p.zp, N, K, bs)
    wd_n = npx.int4_weights(p.w, p.scales, p.zp, N, K, bs)
    assert np.array_equal(wd_c, wd_n)
    y, S = oracle.int4_gemv(p.x, p.w, p.scales, p.zp, 8, N, K, bs)
    yn, Sn = npx.gemv(npx.x_f16(p.x), wd_n)
    assert np.allclose(y, yn, rtol=1e-12, atol=1e-12) and np.allclose(S, Sn, rtol=1e-12)


@pytest.mark.parametrize("N,K", [(1, 256), (3, 512), (4, 1024)])
def test_q4k_against_numpy_cross_oracle(oracle_lib, N, K):
    import datagen
    q = datagen.q4k_problem(N, K, seed=N * 7 + K)
    assert np.array_equal(oracle.q4k_dequant(q.w, N, K), npx.q4k_weights(q.w, N, K))
    pc = oracle.q4k_build_plane(q.w, N, K)
    pn = npx.q4k_plane(q.w, N, K)
    assert pc.tobytes() == pn.tobytes()
    y, S = oracle.q4k_gemv(q.x, q.w, 8, N, K)
    yn, Sn = npx.gemv(q.x.astype(np.float64), npx.q4k_weights(q.w, N, K))
    assert np.allclose(y, yn, rtol=1e-12, atol=1e-12) and np.allclose(S, Sn, rtol=1e-12)


def test_bf16_against_numpy_cross_oracle(oracle_lib):
    import datagen
    p = datagen.bf16_problem(5, 100, seed=4)
    # strided W: rows of 103 elements, offset 1
    ldw = 103
    wbuf = np.zeros(5 * ldw + 1, dtype=np.uint16)
    for n in range(5):
        wbuf[1 + n * ldw:1 + n * ldw + 100] = p.w[n]
    wv = wbuf[1:].copy()
    y, S = oracle.bf16_gemv(p.x, wv, 8, 5, 100, 100, ldw)
    yn, Sn = npx.gemv(npx.x_bf16(p.x), npx.bf16_weights(wv, 5, 100, ldw))
    assert np.allclose(y, yn, rtol=1e-12, atol=1e-12) and np.allclose(S, Sn, rtol=1e-12)


# ---------------------------------------------------------------------------
# q4_K x 8-bit activations (prefill)
# ---------------------------------------------------------------------------

def test_q8_worked_example(oracle_lib):
    g = _gold("q8_worked_example.json")
    for blk in g["blocks"]:
        x = np.array(blk["x"], dtype=np.float32).reshape(1, 32)
        q, d = oracle.q8_quantize(x, 1, 32)
        assert float(d[0, 0]) == blk["d"]
        assert q[0].tolist() == blk["q"]


def _q8_blocks(rng, T, K):
    """Rows of varied magnitude, with exact halfway quotients planted."""
    x = (rng.standard_normal((T, K)) * rng.uniform(1e-3, 50.0, (T, 1))).astype(np.float32)
    xb = x.reshape(T, K // 32, 32)
    # block 0 of every row: amax 127/16 (scale exactly 1/16) and halfway codes
    xb[:, 0, :] = (rng.integers(-126, 126, (T, 32)) + 0.5 * rng.integers(0, 2, (T, 32))) / 16.0
    xb[:, 0, 0] = -127 / 16.0
    xb[:, 1, :] = 0.0  # an all-zero block
    return np.ascontiguousarray(xb.reshape(T, K))


def test_q8_invariants(oracle_lib):
    rng = np.random.default_rng(21)
    T, K = 6, 512
    x = _q8_blocks(rng, T, K)
    q, d = oracle.q8_quantize(x, T, K)
    xb = x.reshape(T, K // 32, 32).astype(np.float64)
    qb = q.reshape(T, K // 32, 32).astype(np.int64)
    amax = np.abs(xb).max(axis=2)
    assert np.all(np.abs(qb) <= 127)
    # the scale is the binary32 quotient amax / 127
    assert np.array_equal(d, (amax.astype(np.float32) / np.float32(127.0)).astype(np.float32))
    dd = d.astype(np.float64)[..., None]
    # the largest magnitude maps to +-127, signs agree, error within half a step
    arg = np.abs(xb).argmax(axis=2)
    at = np.take_along_axis(qb, arg[..., None], axis=2)[..., 0]
    xat = np.take_along_axis(xb, arg[..., None], axis=2)[..., 0]
    nz = amax > 0
    assert np.all(at[nz] == np.where(xat[nz] > 0, 127, -127))
    assert np.all((qb == 0) | (np.sign(qb) == np.sign(xb)))
    assert np.all(np.abs(xb - dd * qb) <= dd * (0.5 + 1e-5))
    assert np.all(qb[~nz] == 0) and np.all(d[~nz] == 0)
    # block 0: scale exactly 1/16, halfway quotients rounded away from zero
    assert np.all(d[:, 0] == 0.0625)
    v = xb[:, 0, :] * 16.0
    assert np.array_equal(qb[:, 0, :], (np.sign(v) * np.floor(np.abs(v) + 0.5)).astype(np.int64))


def test_q8_against_numpy_cross_oracle(oracle_lib):
    rng = np.random.default_rng(22)
    T, K = 9, 1024
    x = _q8_blocks(rng, T, K)
    q, d = oracle.q8_quantize(x, T, K)
    qn, dn = npx.q8_quantize(x, K)
    assert np.array_equal(q.astype(np.int64), qn) and np.array_equal(d.view(np.uint32), dn.view(np.uint32))


def test_q4k_mmq_worked_example(oracle_lib):
    g = _gold("q4k_mmq_worked_example.json")
    w = _one_block(g["d_bits"], g["dmin_bits"], g["scale_bytes"], bytes([g["quant_byte"]]) * 128)
    x = np.zeros((2, 256), dtype=np.float32)
    for c in range(8):
        x[0, 32 * c] = 127.0
        x[0, 32 * c + 1] = c + 1
    x[1] = x[0] * 0.5
    y, S = oracle.q4k_mmq(x, w, 2, 1, 256)
    assert y[:, 0].tolist() == g["y"] and S[:, 0].tolist() == g["S"]


@pytest.mark.parametrize("N,K", [(2, 256), (3, 512)])
def test_q4k_mmq_bruteforce_integer(oracle_lib, N, K):
    """d = dmin = 1 and activation blocks with amax 127: d_a = 1, q_a = x and
    w = s*q - m, so y is an exact integer matmul."""
    rng = np.random.default_rng(30 + K + N)
    nsb = K // 256
    blocks = [_one_block(0x3C00, 0x3C00, rng.integers(0, 256, 12, dtype=np.uint8).tobytes(),
                         rng.integers(0, 256, 128, dtype=np.uint8).tobytes()) for _ in range(N * nsb)]
    w = np.concatenate(blocks).reshape(N, nsb * 144)
    T = 4
    x_int = rng.integers(-127, 128, (T, K))
    x_int.reshape(T, K // 32, 32)[:, :, 5] = 127 * rng.choice([-1, 1], (T, K // 32))
    x = x_int.astype(np.float32)
    wint = []
    for n in range(N):
        row = []
        for k in range(K):
            sb, e = divmod(k, 256)
            cc, l = divmod(e, 32)
            sc = [int(v) for v in w[n, sb * 144 + 4:sb * 144 + 16]]
            s_, m_ = oracle.q4k_scale_min(bytes(sc), cc)
            byte = int(w[n, sb * 144 + 16 + 32 * (cc // 2) + l])
            q_ = byte & 15 if cc % 2 == 0 else byte >> 4
            row.append(s_ * q_ - m_)
        wint.append(row)
    want = _exact_int_matmul(x_int.tolist(), wint)
    y, _ = oracle.q4k_mmq(x, w, T, N, K)
    assert y.tolist() == [[float(v) for v in r] for r in want]


def test_q4k_mmq_within_quantization_error_of_exact_gemv(oracle_lib):
    """|y_mmq - x . w| is bounded by sum_k |w_k| * |x_k - d_a q_a,k|, the error
    the 8-bit activations introduce (w exact in these distributions)."""
    import datagen
    N, K, T = 6, 1024, 3
    p = datagen.q4k_problem(N, K, seed=31)
    x = p.x[:T].copy()
    y, S = oracle.q4k_mmq(x, p.w, T, N, K)
    yg, _ = oracle.q4k_gemv(x, p.w, T, N, K)
    q, d = oracle.q8_quantize(x, T, K)
    dx = np.abs(x.astype(np.float64) - q * np.repeat(d.astype(np.float64), 32, axis=1))
    wdq = np.abs(oracle.q4k_dequant(p.w, N, K))
    bound = dx @ wdq.T
    assert np.all(np.abs(y - yg) <= bound * (1 + 1e-9) + 1e-12 * S)
    assert np.all(bound <= 0.02 * np.abs(x.astype(np.float64)) @ wdq.T)  # the bound is small


@pytest.mark.parametrize("N,K,T", [(3, 256, 2), (5, 768, 4)])
def test_q4k_mmq_against_numpy_cross_oracle(oracle_lib, N, K, T):
    import datagen
    p = datagen.q4k_problem(N, K, seed=32 + K)
    x = p.x[:T].copy()
    y, S = oracle.q4k_mmq(x, p.w, T, N, K)
    yn = npx.q4k_mmq(x, p.w, N, K)
    assert np.allclose(y, yn, rtol=1e-12, atol=1e-12 * float(np.abs(S).max()))
    yc, Sc = oracle.q4k_mmq(x, p.w, T, N, K, cols=[N - 1, 0])
    assert np.array_equal(yc, y[:, [N - 1, 0]]) and np.array_equal(Sc, S[:, [N - 1, 0]])


# ---------------------------------------------------------------------------
# the acceptance rule
# ---------------------------------------------------------------------------

def test_accept_rule(oracle_lib):
    y_ref = np.array([[1.0, 0.0, -100.0]])
    S = np.array([[10.0, 0.0, 1000.0]])
    # bound = 2e-3*S + ulp_f16(y_ref) = 0.02 + 2^-10, 2^-24, 2 + 2^-4
    ok, worst = oracle.accept(y_ref + np.array([[0.02, 0.0, 2.0]]), y_ref, S, "f16")
    assert ok and worst <= 1.0
    ok, _ = oracle.accept(y_ref + np.array([[0.03, 0.0, 0.0]]), y_ref, S, "f16")
    assert not ok
    ok, _ = oracle.accept(np.array([[1.0, 2.0 ** -24, -100.0]]), y_ref, S, "f16")
    assert ok
    ok, _ = oracle.accept(np.array([[np.nan, 0.0, -100.0]]), y_ref, S, "f16")
    assert not ok

"""Hand-built q4_K weights for the parity tests (not a test module).

``zero_weight_rows`` lays out q4_K super-blocks whose dequantized weights are
exactly zero although every chunk's coefficients are not: with d = dmin, a
chunk with scale sc, min m = sc*q and every quant equal to q has
w = d*sc*q - d*m = 0.  Only bytes are laid out here (the 6-bit scale/min
packing of the format, "62 . r59 -- q4_K W_dsc plane + riders", section 3.2);
the tests check the decoded (sc, m) with the oracle.
"""
from __future__ import annotations

import numpy as np


def pack_scale_min(sc, m) -> bytes:
    """The twelve packed bytes of eight 6-bit (scale, min) pairs."""
    sc = np.asarray(sc, dtype=np.int64)
    m = np.asarray(m, dtype=np.int64)
    b = np.zeros(12, dtype=np.int64)
    b[0:4] = sc[0:4] | ((sc[4:8] >> 4) << 6)
    b[4:8] = m[0:4] | ((m[4:8] >> 4) << 6)
    b[8:12] = (sc[4:8] & 15) | ((m[4:8] & 15) << 4)
    return bytes(b.astype(np.uint8))


def zero_weight_rows(N: int, K: int, seed: int, zero_frac=None):
    """uint8 [N][K/256*144] q4_K weights.  ``zero_frac`` None: every chunk of
    every row has exactly-zero weights.  Otherwise row n's chunks are
    degenerate with probability zero_frac[n] and random otherwise (6-bit
    scale and min uniform 0..63, quants uniform 0..15).  d = dmin in every
    super-block, drawn from U(1e-3, 4e-3) and rounded to fp16."""
    assert K % 256 == 0
    rng = np.random.default_rng(seed)
    nsb = K // 256
    out = np.empty((N, nsb, 144), dtype=np.uint8)
    for n in range(N):
        for s in range(nsb):
            d = np.float16(rng.uniform(1e-3, 4e-3)).view(np.uint16)
            sc = np.zeros(8, dtype=np.int64)
            m = np.zeros(8, dtype=np.int64)
            quants = np.zeros((8, 32), dtype=np.uint8)
            for cc in range(8):
                if zero_frac is None or rng.uniform() < zero_frac[n]:
                    sc[cc] = rng.integers(1, 12)
                    q = rng.integers(1, min(15, 63 // sc[cc]) + 1)
                    m[cc] = sc[cc] * q
                    quants[cc] = q
                else:
                    sc[cc], m[cc] = rng.integers(0, 64, 2)
                    quants[cc] = rng.integers(0, 16, 32)
            qs = np.zeros(128, dtype=np.uint8)
            for g in range(4):
                qs[32 * g:32 * g + 32] = quants[2 * g] | (quants[2 * g + 1] << 4)
            out[n, s, 0:2] = np.frombuffer(d.tobytes(), np.uint8)
            out[n, s, 2:4] = np.frombuffer(d.tobytes(), np.uint8)
            out[n, s, 4:16] = np.frombuffer(pack_scale_min(sc, m), np.uint8)
            out[n, s, 16:] = qs
    return np.ascontiguousarray(out.reshape(N, nsb * 144))

"""Second, independent oracle in vectorised NumPy (tiny shapes only).

TEST INFRASTRUCTURE ONLY (same rules as the rest of ``oracle/``).  It shares no
code with ``qgemv_oracle.c``: the C oracle walks one weight at a time through
per-element decoders, this module decodes whole tensors at once with array
bit operations and NumPy's own fp16 decoder.  Agreement of the two on random
tiny cases pins the C oracle's indexing (row strides, nibble positions, block
indices) against a differently written program.

Sources as in ``qgemv_oracle.c``: onnx-genai pull request #1000 (int4
MatMulNBits), "62 . r59 -- q4_K W_dsc plane + riders" sections 2.1-3.2 (q4_K and
the plane), the AstrAI backend commit list (bf16).
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def _f16(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _bf16(bits: np.ndarray) -> np.ndarray:
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def int4_weights(w: np.ndarray, scales: np.ndarray, zp: Optional[np.ndarray], N: int,
                 K: int, bs: int) -> np.ndarray:
    w = np.asarray(w, dtype=np.uint8).reshape(N, K // 2)
    codes = np.empty((N, K), dtype=np.int64)
    codes[:, 0::2] = w & 0x0F
    codes[:, 1::2] = w >> 4
    nb = K // bs
    if zp is None:
        zpts = np.full((N, nb), 8, dtype=np.int64)
    else:
        z = np.asarray(zp, dtype=np.uint8).reshape(N, -1)
        both = np.empty((N, 2 * z.shape[1]), dtype=np.int64)
        both[:, 0::2] = z & 0x0F
        both[:, 1::2] = z >> 4
        zpts = both[:, :nb]
    s = _f16(np.asarray(scales).reshape(N, nb))
    return np.repeat(s, bs, axis=1) * (codes - np.repeat(zpts, bs, axis=1))


def q4k_coeffs(w: np.ndarray, N: int, K: int):
    """(dv, mv) as float32 arrays [N][K/32]."""
    nsb = K // 256
    blk = np.asarray(w, dtype=np.uint8).reshape(N, nsb, 144)
    d = _f16(blk[:, :, 0:2].copy().view(np.uint16)[..., 0]).astype(np.float32)
    dmin = _f16(blk[:, :, 2:4].copy().view(np.uint16)[..., 0]).astype(np.float32)
    b = blk[:, :, 4:16].astype(np.int64)
    s = np.empty((N, nsb, 8), dtype=np.int64)
    m = np.empty((N, nsb, 8), dtype=np.int64)
    s[:, :, 0:4] = b[:, :, 0:4] & 63
    m[:, :, 0:4] = b[:, :, 4:8] & 63
    s[:, :, 4:8] = (b[:, :, 8:12] & 0x0F) | ((b[:, :, 0:4] >> 6) << 4)
    m[:, :, 4:8] = (b[:, :, 8:12] >> 4) | ((b[:, :, 4:8] >> 6) << 4)
    dv = (d[..., None] * s.astype(np.float32)).astype(np.float32)
    mv = -(dmin[..., None] * m.astype(np.float32)).astype(np.float32)
    return dv.reshape(N, nsb * 8), mv.reshape(N, nsb * 8)


def q4k_codes(w: np.ndarray, N: int, K: int) -> np.ndarray:
    nsb = K // 256
    qs = np.asarray(w, dtype=np.uint8).reshape(N, nsb, 144)[:, :, 16:].reshape(N, nsb, 4, 32)
    out = np.empty((N, nsb, 4, 2, 32), dtype=np.int64)
    out[:, :, :, 0, :] = qs & 0x0F
    out[:, :, :, 1, :] = qs >> 4
    return out.reshape(N, K)


def q4k_weights(w: np.ndarray, N: int, K: int) -> np.ndarray:
    dv, mv = q4k_coeffs(w, N, K)
    q = q4k_codes(w, N, K).astype(np.float32)
    wv = np.repeat(dv, 32, axis=1) * q + np.repeat(mv, 32, axis=1)  # float32 ops
    return wv.astype(np.float64)


def q4k_plane(w: np.ndarray, N: int, K: int) -> np.ndarray:
    dv, mv = q4k_coeffs(w, N, K)
    return np.ascontiguousarray(np.stack([dv.T, mv.T], axis=-1).reshape(-1, 2))


def bf16_weights(w: np.ndarray, N: int, K: int, ldw: int) -> np.ndarray:
    flat = np.asarray(w, dtype=np.uint16).ravel()
    rows = np.stack([flat[n * ldw:n * ldw + K] for n in range(N)]) if N else np.zeros((0, K))
    return _bf16(rows)


def gemv(x: np.ndarray, wdq: np.ndarray):
    """x: float64 [M][K]; wdq: float64 [N][K] -> (y_ref, S)."""
    return x @ wdq.T, np.abs(x) @ np.abs(wdq).T


def x_f16(bits: np.ndarray) -> np.ndarray:
    return _f16(bits)


def x_bf16(bits: np.ndarray) -> np.ndarray:
    return _bf16(bits)


def q8_quantize(x: np.ndarray, K: int):
    """Per 32-block symmetric 8-bit codes of float32 rows x [T][K]: the scale
    is amax/127 and the code x/scale rounded half away from zero, both
    quotients in float32 (NumPy's float32 division is IEEE)."""
    xb = np.asarray(x, dtype=np.float32).reshape(x.shape[0], K // 32, 32)
    amax = np.abs(xb).max(axis=2)
    d = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(d == 0, np.float32(1.0), d).astype(np.float32)
    v = (xb / safe[..., None]).astype(np.float32).astype(np.float64)
    q = np.sign(v) * np.floor(np.abs(v) + 0.5)
    q = np.where(d[..., None] == 0, 0.0, q)
    return q.reshape(x.shape[0], K).astype(np.int64), d


def q4k_mmq(x: np.ndarray, w: np.ndarray, N: int, K: int):
    """The q4_K x q8 product: the GEMV of the dequantized activations
    d_a * q_a with the exact weights dv * q + mv."""
    q, d = q8_quantize(x, K)
    xa = q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    dv, mv = q4k_coeffs(w, N, K)
    wex = (np.repeat(dv.astype(np.float64), 32, axis=1) * q4k_codes(w, N, K)
           + np.repeat(mv.astype(np.float64), 32, axis=1))
    return xa @ wex.T

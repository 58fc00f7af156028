"""Seeded synthetic inputs for the weight-only quantized GEMV.

Shared by the tests, the smoke check and the bench; it holds none of the
method's arithmetic (no dequantization, no dot products): it only draws random
values with numpy's PCG64 generator and lays the drawn bytes out in the stored
formats, which both the HIP path and the oracle then consume.

Distributions (one per workload, as the decode workloads are specified):

* int4 MatMulNBits: weight bytes uniform 0..255 (= two independent uniform
  nibbles per byte), fp16 scales ~ U(0.005, 0.02) rounded to nearest fp16,
  zero-point bytes uniform 0..255 (two uniform 4-bit zero points per byte; a
  padding nibble, when the block count is odd, is random too), x ~ N(0,1)
  rounded to fp16.
* q4_K: per 144-byte super-block, d and dmin ~ U(1e-3, 4e-3) rounded to fp16,
  twelve scale bytes uniform 0..255 (which makes every 6-bit scale and min
  uniform 0..63: the 96 bits map one-to-one onto the sixteen 6-bit fields),
  128 quant bytes uniform 0..255; x ~ N(0,1) in float32.
* bf16: W ~ N(0, 0.02) and x ~ N(0, 1), float32 draws rounded to nearest-even
  bfloat16.

Draw order within one seed: weights, then scales, then zero points, then x.
x is always drawn as 8 rows so that the M = 1..8 sweeps share a prefix.

Prefill activations (the q4_K x 8-bit path): ``prefill_x`` draws T rows of
x ~ N(0,1) in float32 from a seed of their own, with the row scale varying
by a factor of 100 across rows (prompt tokens differ in magnitude) and one
all-zero 32-block per row so that the zero-scale case is always present.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

X_ROWS = 8  # x is drawn with this many rows; callers slice the first M


def _f16_bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a.astype(np.float16).view(np.uint16))


def _bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite inputs)."""
    import torch  # torch's CPU conversion is the rounding routine used here

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return np.ascontiguousarray(t.view(torch.int16).numpy().view(np.uint16))


@dataclass
class Int4Problem:
    N: int
    K: int
    block_size: int
    w: np.ndarray                 # uint8 [N][K/2]
    scales: np.ndarray            # uint16 (fp16 bits) [N][K/bs]
    zp: Optional[np.ndarray]      # uint8 [N][ceil(K/bs/2)] or None
    x: np.ndarray                 # uint16 (fp16 bits) [8][K]


@dataclass
class Q4KProblem:
    N: int
    K: int
    w: np.ndarray                 # uint8 [N][K/256*144]
    x: np.ndarray                 # float32 [8][K]


@dataclass
class Bf16Problem:
    N: int
    K: int
    w: np.ndarray                 # uint16 (bf16 bits) [N][K]
    x: np.ndarray                 # uint16 (bf16 bits) [8][K]


def int4_problem(N: int, K: int, block_size: int, asym: bool, seed: int,
                 scale_lo: float = 0.005, scale_hi: float = 0.02) -> Int4Problem:
    assert K % block_size == 0 and K % 2 == 0
    rng = np.random.default_rng(seed)
    nb = K // block_size
    w = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = _f16_bits(rng.uniform(scale_lo, scale_hi, size=(N, nb)))
    zp = rng.integers(0, 256, size=(N, (nb + 1) // 2), dtype=np.uint8) if asym else None
    x = _f16_bits(rng.standard_normal((X_ROWS, K)))
    return Int4Problem(N, K, block_size, w, scales, zp, x)


def q4k_problem(N: int, K: int, seed: int) -> Q4KProblem:
    assert K % 256 == 0
    rng = np.random.default_rng(seed)
    nsb = K // 256
    qs = rng.integers(0, 256, size=(N, nsb, 128), dtype=np.uint8)
    d = _f16_bits(rng.uniform(1e-3, 4e-3, size=(N, nsb)))
    dmin = _f16_bits(rng.uniform(1e-3, 4e-3, size=(N, nsb)))
    sc = rng.integers(0, 256, size=(N, nsb, 12), dtype=np.uint8)
    x = rng.standard_normal((X_ROWS, K)).astype(np.float32)
    blocks = np.empty((N, nsb, 144), dtype=np.uint8)
    blocks[:, :, 0:2] = d[..., None].view(np.uint8).reshape(N, nsb, 2)
    blocks[:, :, 2:4] = dmin[..., None].view(np.uint8).reshape(N, nsb, 2)
    blocks[:, :, 4:16] = sc
    blocks[:, :, 16:144] = qs
    return Q4KProblem(N, K, np.ascontiguousarray(blocks.reshape(N, nsb * 144)), x)


def bf16_problem(N: int, K: int, seed: int) -> Bf16Problem:
    rng = np.random.default_rng(seed)
    w = _bf16_bits(rng.normal(0.0, 0.02, size=(N, K)).astype(np.float32))
    x = _bf16_bits(rng.standard_normal((X_ROWS, K)).astype(np.float32))
    return Bf16Problem(N, K, w, x)


def q4k_header(d_bits: int, dmin_bits: int, sc12: bytes, qs128: bytes) -> bytes:
    """Assemble one 144-byte super-block from its fields (for hand-made cases)."""
    assert len(sc12) == 12 and len(qs128) == 128
    return (int(d_bits).to_bytes(2, "little") + int(dmin_bits).to_bytes(2, "little")
            + bytes(sc12) + bytes(qs128))


def prefill_x(T: int, K: int, seed: int) -> np.ndarray:
    """float32 [T][K] prefill activations (see the module docstring)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, K)).astype(np.float32)
    x *= (10.0 ** rng.uniform(-1.0, 1.0, (T, 1))).astype(np.float32)
    if K >= 64:
        z = rng.integers(0, K // 32, T)
        for t in range(T):
            x[t, 32 * z[t]:32 * z[t] + 32] = 0.0
    return np.ascontiguousarray(x)

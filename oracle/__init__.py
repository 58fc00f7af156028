"""fp64 CPU oracle for the weight-only quantized decode GEMV.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``weight_only_quantized_int4_amd``) never imports it, and the two share no code:
this package wraps ``qgemv_oracle.c`` (plain C, built with gcc, no HIP) through
ctypes and adds the acceptance rule used by the parity tests.

What it computes (see the header of ``qgemv_oracle.c`` for the sources):

* ``int4_gemv``  -- MatMulNBits blockwise int4, w = f16(scale) * (q - zp)
  (onnx-genai pull request #1000, "Summary" / "What it does").
* ``q4k_gemv``   -- q4_K super-blocks decoded with get_scale_min_k4
  ("62 . r59 -- q4_K W_dsc plane + riders", sections 2.1 and 3.2).
* ``q4k_build_plane`` / ``q4k_plane_gemv`` -- the chunk-major float2 plane
  (same page, sections 2.2 and 2.3).
* ``bf16_gemv``  -- the dense bf16 GEMV (AstrAI backend commit list).
* ``q8_quantize`` / ``q4k_mmq`` -- q4_K prefill with 8-bit activations: the
  activation prepass and the per-chunk rank-1 rescale of exact integer dot
  products ("62 . r59 -- q4_K W_dsc plane + riders", sections 2.1 and 3.2;
  the activation rule is a reading, stated in ``qgemv_oracle.c``).

Each GEMV returns ``(y_ref, S)`` in float64: ``y_ref = sum_k x*w`` and
``S = sum_k |x*w|``.  ``accept`` applies the rule
``|y - y_ref| <= 2e-3 * S + ulp_out(y_ref)``.

Parity unpinned by the pages: the MatMulNBits tensor layout and the q4_K quant
nibble order are conventions (see ``qgemv_oracle.c``); the arithmetic is pinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qgemv_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the binding at another build of the oracle (used only by the
# mutation check, which compiles deliberately broken copies of the source).
_LIB_OVERRIDE = os.environ.get("QGEMV_ORACLE_LIB")

# Relative tolerance of the acceptance rule (fp32 accumulate, 16-bit output).
RTOL = 2e-3
# Relative tolerance of the q4_K x q8 product against its exact value: the
# integer sums are exact, and fp32 evaluation of d_a*(dv*D + mv*Sa) plus the
# running sum over K/32 chunks rounds at most K/32 + 4 times, each time by at
# most 2^-24 of a partial magnitude bounded by S; (K/32 + 4) * 2^-24 < 1e-4 for
# K <= 52000.
RTOL_MMQ = 1e-4


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no contraction of a*b+c into an FMA)."""
    if force or not os.path.exists(_LIB):
        tmp = f"{_LIB}.{os.getpid()}.tmp"  # concurrent builders never share a file
        subprocess.check_call(
            ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11",
             "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            L = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            L = ctypes.CDLL(_LIB)
        P, I64, D, U16, I = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_double,
                             ctypes.c_uint16, ctypes.c_int)
        sig = {
            "oracle_f16_to_f64": (D, [U16]),
            "oracle_bf16_to_f64": (D, [U16]),
            "oracle_f32bits_to_f64": (D, [ctypes.c_uint32]),
            "oracle_round_f16": (D, [D]),
            "oracle_round_bf16": (D, [D]),
            "oracle_round_f32": (D, [D]),
            "oracle_ulp_f16": (D, [D]),
            "oracle_ulp_bf16": (D, [D]),
            "oracle_ulp_f32": (D, [D]),
            "oracle_int4_zp_row_bytes": (I64, [I64, I64]),
            "oracle_int4_code": (I, [P, I64, I64, I64]),
            "oracle_int4_zero_point": (I, [P, I64, I64, I64, I64]),
            "oracle_int4_weight": (D, [P, P, P, I64, I64, I64, I64]),
            "oracle_int4_dequant_rows": (None, [P, P, P, I64, I64, I64, I64, P]),
            "oracle_q4k_scale_min": (None, [P, I, P, P]),
            "oracle_q4k_coeffs": (None, [P, I64, I64, I64, P, P]),
            "oracle_q4k_code": (I, [P, I64, I64, I64]),
            "oracle_q4k_weight": (D, [P, I64, I64, I64]),
            "oracle_q4k_weight_plane": (D, [P, P, I64, I64, I64, I64]),
            "oracle_q4k_dequant_rows": (None, [P, I64, I64, I64, P]),
            "oracle_q4k_build_plane": (None, [P, I64, I64, P]),
            "oracle_int4_gemv": (None, [P, I64, P, P, P, I64, I64, I64, I64, P, I64, P, P]),
            "oracle_q4k_gemv": (None, [P, I64, P, I64, I64, I64, P, I64, P, P]),
            "oracle_q4k_plane_gemv": (None, [P, I64, P, P, I64, I64, I64, P, I64, P, P]),
            "oracle_bf16_gemv": (None, [P, I64, P, I64, I64, I64, I64, P, I64, P, P]),
            "oracle_q8_quantize_block": (None, [P, P, P]),
            "oracle_q8_quantize_rows": (None, [P, I64, I64, I64, P, P]),
            "oracle_q4k_mmq": (None, [P, I64, P, I64, I64, I64, P, I64, P, P, P, P, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _cols(cols: Optional[Sequence[int]], N: int) -> Tuple[Optional[np.ndarray], int]:
    if cols is None:
        return None, N
    c = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    assert c.ndim == 1 and (c.size == 0 or (c.min() >= 0 and c.max() < N))
    return c, int(c.size)


# ---------------------------------------------------------------------------
# scalar decoders / rounding (exposed for the pins)
# ---------------------------------------------------------------------------

def f16_to_f64(bits: int) -> float:
    return lib().oracle_f16_to_f64(bits)


def bf16_to_f64(bits: int) -> float:
    return lib().oracle_bf16_to_f64(bits)


def round_to(v: float, dtype: str) -> float:
    return {"f16": lib().oracle_round_f16, "bf16": lib().oracle_round_bf16,
            "f32": lib().oracle_round_f32}[dtype](float(v))


def ulp(v: float, dtype: str) -> float:
    return {"f16": lib().oracle_ulp_f16, "bf16": lib().oracle_ulp_bf16,
            "f32": lib().oracle_ulp_f32}[dtype](float(v))


# ---------------------------------------------------------------------------
# int4 MatMulNBits
# ---------------------------------------------------------------------------

def int4_zp_row_bytes(K: int, block_size: int) -> int:
    return lib().oracle_int4_zp_row_bytes(K, block_size)


def int4_dequant(w: np.ndarray, scales: np.ndarray, zp: Optional[np.ndarray],
                 N: int, K: int, block_size: int, rows: Optional[Sequence[int]] = None
                 ) -> np.ndarray:
    """Dequantized weights (float64, each exactly a binary32 value), [len(rows)][K]."""
    rows = list(range(N)) if rows is None else list(rows)
    out = np.empty((len(rows), K), dtype=np.float64)
    for i, n in enumerate(rows):
        lib().oracle_int4_dequant_rows(_ptr(w), _ptr(scales), _ptr(zp), K, block_size,
                                       int(n), 1, out[i].ctypes.data)
    return out


def int4_gemv(x_f16: np.ndarray, w: np.ndarray, scales: np.ndarray,
              zp: Optional[np.ndarray], M: int, N: int, K: int, block_size: int,
              cols: Optional[Sequence[int]] = None, ldx: Optional[int] = None):
    """x_f16: uint16 bits [M][ldx]; w: uint8 [N][K/2]; scales: uint16 [N][K/bs];
    zp: uint8 [N][ceil(K/bs/2)] or None.  Returns (y_ref, S), float64 [M][ncols]."""
    c, nc = _cols(cols, N)
    ldx = K if ldx is None else ldx
    y = np.zeros((M, nc), dtype=np.float64)
    s = np.zeros((M, nc), dtype=np.float64)
    lib().oracle_int4_gemv(_ptr(x_f16), ldx, _ptr(w), _ptr(scales), _ptr(zp), M, N, K,
                           block_size, _ptr(c), nc, y.ctypes.data, s.ctypes.data)
    return y, s


# ---------------------------------------------------------------------------
# q4_K
# ---------------------------------------------------------------------------

def q4k_scale_min(sc12: bytes, cc: int) -> Tuple[int, int]:
    buf = np.frombuffer(bytes(sc12), dtype=np.uint8).copy()
    assert buf.size == 12
    s = ctypes.c_int()
    m = ctypes.c_int()
    lib().oracle_q4k_scale_min(buf.ctypes.data, cc, ctypes.byref(s), ctypes.byref(m))
    return s.value, m.value


def q4k_coeffs(w: np.ndarray, K: int, n: int, c: int) -> Tuple[int, int]:
    """(dv, mv) of chunk c of row n as binary32 bit patterns."""
    dv = ctypes.c_float()
    mv = ctypes.c_float()
    lib().oracle_q4k_coeffs(_ptr(w), K, n, c, ctypes.byref(dv), ctypes.byref(mv))
    as_bits = lambda f: int(np.array([f.value], dtype=np.float32).view(np.uint32)[0])
    return as_bits(dv), as_bits(mv)


def q4k_dequant(w: np.ndarray, N: int, K: int, rows: Optional[Sequence[int]] = None
                ) -> np.ndarray:
    rows = list(range(N)) if rows is None else list(rows)
    out = np.empty((len(rows), K), dtype=np.float64)
    for i, n in enumerate(rows):
        lib().oracle_q4k_dequant_rows(_ptr(w), K, int(n), 1, out[i].ctypes.data)
    return out


def q4k_build_plane(w: np.ndarray, N: int, K: int) -> np.ndarray:
    """The chunk-major W_dsc plane, float32 [(K/32)*N][2]."""
    plane = np.zeros(((K // 32) * N, 2), dtype=np.float32)
    lib().oracle_q4k_build_plane(_ptr(w), N, K, plane.ctypes.data)
    return plane


def q4k_gemv(x: np.ndarray, w: np.ndarray, M: int, N: int, K: int,
             cols: Optional[Sequence[int]] = None, ldx: Optional[int] = None):
    c, nc = _cols(cols, N)
    ldx = K if ldx is None else ldx
    y = np.zeros((M, nc), dtype=np.float64)
    s = np.zeros((M, nc), dtype=np.float64)
    lib().oracle_q4k_gemv(_ptr(x), ldx, _ptr(w), M, N, K, _ptr(c), nc,
                          y.ctypes.data, s.ctypes.data)
    return y, s


def q4k_plane_gemv(x: np.ndarray, w: np.ndarray, plane: np.ndarray, M: int, N: int,
                   K: int, cols: Optional[Sequence[int]] = None,
                   ldx: Optional[int] = None):
    c, nc = _cols(cols, N)
    ldx = K if ldx is None else ldx
    y = np.zeros((M, nc), dtype=np.float64)
    s = np.zeros((M, nc), dtype=np.float64)
    lib().oracle_q4k_plane_gemv(_ptr(x), ldx, _ptr(w), _ptr(plane), M, N, K, _ptr(c),
                                nc, y.ctypes.data, s.ctypes.data)
    return y, s


# ---------------------------------------------------------------------------
# q4_K x 8-bit activations (prefill)
# ---------------------------------------------------------------------------

def q8_quantize(x: np.ndarray, T: int, K: int, ldx: Optional[int] = None):
    """Codes int8 [T][K] and scales float32 [T][K/32] of x float32 [T][ldx]."""
    ldx = K if ldx is None else ldx
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.zeros((T, K), dtype=np.int8)
    d = np.zeros((T, K // 32), dtype=np.float32)
    lib().oracle_q8_quantize_rows(_ptr(x), ldx, T, K, q.ctypes.data, d.ctypes.data)
    return q, d


def q4k_mmq(x: np.ndarray, w: np.ndarray, T: int, N: int, K: int,
            cols: Optional[Sequence[int]] = None, ldx: Optional[int] = None):
    """(y_ref, S) [T][ncols] of the q4_K x q8 product (see qgemv_oracle.c)."""
    c, nc = _cols(cols, N)
    ldx = K if ldx is None else ldx
    x = np.ascontiguousarray(x, dtype=np.float32)
    qa = np.zeros((T, K), dtype=np.int8)
    da = np.zeros((T, K // 32), dtype=np.float32)
    qw = np.zeros(K, dtype=np.intc)
    y = np.zeros((T, nc), dtype=np.float64)
    s = np.zeros((T, nc), dtype=np.float64)
    lib().oracle_q4k_mmq(_ptr(x), ldx, _ptr(w), T, N, K, _ptr(c), nc, qa.ctypes.data,
                         da.ctypes.data, qw.ctypes.data, y.ctypes.data, s.ctypes.data)
    return y, s


# ---------------------------------------------------------------------------
# bf16
# ---------------------------------------------------------------------------

def bf16_gemv(x: np.ndarray, w: np.ndarray, M: int, N: int, K: int, ldx: int,
              ldw: int, cols: Optional[Sequence[int]] = None):
    """x, w: uint16 bf16 bits, flat buffers starting at element (0, 0)."""
    c, nc = _cols(cols, N)
    y = np.zeros((M, nc), dtype=np.float64)
    s = np.zeros((M, nc), dtype=np.float64)
    lib().oracle_bf16_gemv(_ptr(x), ldx, _ptr(w), ldw, M, N, K, _ptr(c), nc,
                           y.ctypes.data, s.ctypes.data)
    return y, s


# ---------------------------------------------------------------------------
# acceptance rule
# ---------------------------------------------------------------------------

def ulp_array(v: np.ndarray, dtype: str) -> np.ndarray:
    f = {"f16": lib().oracle_ulp_f16, "bf16": lib().oracle_ulp_bf16,
         "f32": lib().oracle_ulp_f32}[dtype]
    flat = np.asarray(v, dtype=np.float64).ravel()
    return np.array([f(float(t)) for t in flat], dtype=np.float64).reshape(np.shape(v))


def accept(y: np.ndarray, y_ref: np.ndarray, S: np.ndarray, out_dtype: str,
           rtol: float = RTOL):
    """Apply |y - y_ref| <= rtol*S + ulp_out(y_ref) elementwise.

    Returns (ok, worst) where worst is max |y - y_ref| / (rtol*S + ulp).  NaN in
    y counts as a failure."""
    y = np.asarray(y, dtype=np.float64)
    bound = rtol * np.asarray(S, dtype=np.float64) + ulp_array(y_ref, out_dtype)
    err = np.abs(y - y_ref)
    ratio = np.where(np.isfinite(err), err / bound, np.inf)
    worst = float(ratio.max()) if ratio.size else 0.0
    return bool(np.all(ratio <= 1.0)), worst

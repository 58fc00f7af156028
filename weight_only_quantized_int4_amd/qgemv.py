"""ctypes binding of libqgemv.so -- argument marshalling only.

Every function takes torch tensors and checks what the C library cannot see
through a raw pointer: each tensor's dtype, that it lives in GPU memory (on a
machine with a GPU, a host tensor's address would otherwise reach a kernel),
and that every tensor's shape and layout agree with the sizes taken from x and
w (a y, scale, zero-point, plane or workspace tensor shorter than the problem
would otherwise be read or written past its end).  It turns shapes into sizes
and strides into leading dimensions,
passes ``data_ptr()`` and the current HIP stream, and raises ``QgemvError``
with the library's own message on a non-OK status.  All compute happens in the HIP kernels; if the library is missing the
import of a function fails loudly -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqgemv.so")

QG_F16, QG_BF16, QG_F32 = 0, 1, 2
_OUT_TYPES = {torch.float16: QG_F16, torch.bfloat16: QG_BF16, torch.float32: QG_F32}
_X_TYPES = {torch.float16: QG_F16, torch.bfloat16: QG_BF16}
# Size of the static device workspace of qgemm_q4k_mmq_noalloc
# (QG_MMQ_NOALLOC_SCRATCH_BYTES in include/qgemv.h).
MMQ_NOALLOC_SCRATCH_BYTES = 32 << 20
# Layout flag of the packed int4 weights (QG_INT4_LAYOUT_TILE16_V1).
INT4_LAYOUT_TILE16_V1 = 1


class QgemvError(RuntimeError):
    """A libqgemv entry point returned a non-OK status."""

    def __init__(self, fn: str, status: int, name: str, detail: str):
        super().__init__(f"{fn}: {name} ({status}): {detail}")
        self.status = status
        self.status_name = name
        self.detail = detail


_lib: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libqgemv.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(_LIB_PATH)
    P, I64, I32, St = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    sigs = {
        "qgemv_int4_blockwise": (St, [P, I64, I32, P, P, P, P, I64, I32, I64, I64, I64, I32, P]),
        "qgemv_q4k": (St, [P, I64, P, P, I64, I64, I64, I64, P]),
        "qgemv_q4k_dsc": (St, [P, I64, P, P, P, I64, I64, I64, I64, P]),
        "gemv_bf16": (St, [P, I64, P, I64, P, I64, I32, I64, I64, I64, P]),
        "q4k_dsc_plane_bytes": (ctypes.c_size_t, [I64, I64]),
        "q4k_build_dsc_plane": (St, [P, P, I64, I64, P]),
        "qg_status_string": (ctypes.c_char_p, [St]),
        "qg_last_error": (ctypes.c_char_p, []),
        "qg_last_launch": (ctypes.c_char_p, []),
        "qg_path_count": (I32, []),
        "qg_path_name": (ctypes.c_char_p, [I32]),
        "qg_path_launches": (ctypes.c_uint64, [I32]),
        "q4k_mmq_workspace_bytes": (ctypes.c_size_t, [I64, I64]),
        "q8_quantize_rows": (St, [P, I64, P, P, I64, I64, P]),
        "qgemm_q4k_mmq": (St, [P, I64, P, P, P, I64, I64, I64, I64, P, ctypes.c_size_t, P]),
        "qgemm_q4k_mmq_noalloc": (St, [P, I64, P, P, P, I64, I64, I64, I64, P]),
        "int4_packed_bytes": (ctypes.c_size_t, [I64, I64, I32, I32]),
        "int4_repack": (St, [P, P, P, P, ctypes.c_size_t, I64, I64, I32, I32, P]),
        "qgemv_int4_packed": (St, [P, I64, I32, P, ctypes.c_size_t, I32, P, I64, I32, I64, I64,
                                   I64, I32, P]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status != 0:
        L = load_library()
        raise QgemvError(fn, status, L.qg_status_string(status).decode(),
                         L.qg_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_F16, _BF16, _F32, _U8, _I8 = (torch.float16,), (torch.bfloat16,), (torch.float32,), (torch.uint8,), \
    (torch.int8,)
_OUT = tuple(_OUT_TYPES)
_gpu_present: Optional[bool] = None


def _arg(t: Optional[torch.Tensor], name: str, dtypes) -> None:
    """Refuse a tensor of another dtype, or one in host memory on a machine
    with a GPU.  None passes through: the library reports a missing required
    pointer itself."""
    global _gpu_present
    if t is None:
        return
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name}: expected {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if t.device.type != "cuda":
        if _gpu_present is None:
            _gpu_present = torch.cuda.is_available()
        if _gpu_present:
            raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")


def _dims(t: torch.Tensor, name: str, shape) -> None:
    """Refuse a tensor whose shape is not ``shape``."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _dense(t: Optional[torch.Tensor], name: str, shape) -> None:
    """Refuse a tensor that is not a dense row-major array of ``shape`` (the
    library reads it as one without a stride)."""
    if t is None:
        return
    _dims(t, name, shape)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (dense row-major)")


def _xy(x: torch.Tensor, y: torch.Tensor, N: int):
    """(M, K) of x [M, K], checking y [M, N]."""
    if x.dim() != 2:
        raise ValueError(f"x: expected a 2-D tensor [M, K], got shape {tuple(x.shape)}")
    M, K = x.shape
    _dims(y, "y", (M, N))
    return M, K


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ld(t: torch.Tensor) -> int:
    """Leading dimension of a row-major 2-D tensor (unit stride in the last dim)."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D tensor with unit stride in its last dimension")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


def qgemv_int4_blockwise(x: torch.Tensor, w: torch.Tensor, scales: torch.Tensor,
                         zero_points: Optional[torch.Tensor], y: torch.Tensor,
                         block_size: int, stream=None) -> torch.Tensor:
    """y[M,N] = x[M,K] . dequant(w)^T.  x fp16 [M,K] (the library refuses bf16
    activations with QG_ERR_UNSUPPORTED); w uint8 [N,K/2]; scales fp16
    [N,K/bs]; zero_points uint8 [N,ceil(K/bs/2)] or None; y fp16/bf16/fp32 [M,N]."""
    for t, n, d in ((x, "x", tuple(_X_TYPES)), (w, "w", _U8), (scales, "scales", _F16),
                    (zero_points, "zero_points", _U8), (y, "y", _OUT)):
        _arg(t, n, d)
    if w.dim() != 2:
        raise ValueError(f"w: expected a 2-D tensor [N, K/2], got shape {tuple(w.shape)}")
    N = w.shape[0]
    M, K = _xy(x, y, N)
    _dense(w, "w", (N, K // 2))
    if block_size > 0 and K % block_size == 0:  # otherwise the library rejects the call
        nb = K // block_size
        _dense(scales, "scales", (N, nb))
        _dense(zero_points, "zero_points", (N, (nb + 1) // 2))
    _check("qgemv_int4_blockwise", load_library().qgemv_int4_blockwise(
        _ptr(x), _ld(x), _X_TYPES[x.dtype], _ptr(w), _ptr(scales), _ptr(zero_points), _ptr(y), _ld(y),
        _OUT_TYPES[y.dtype], M, N, K, block_size, _stream(stream)))
    return y


def int4_packed_bytes(N: int, K: int, block_size: int, layout: int = INT4_LAYOUT_TILE16_V1) -> int:
    """Bytes of the packed form (0 when the layout or shape is not provided)."""
    return int(load_library().int4_packed_bytes(N, K, block_size, layout))


def int4_repack(w: torch.Tensor, scales: torch.Tensor, zero_points: Optional[torch.Tensor],
                packed: torch.Tensor, block_size: int, layout: int = INT4_LAYOUT_TILE16_V1,
                stream=None) -> torch.Tensor:
    """Write the packed layout of (w, scales, zero_points) -- as taken by
    qgemv_int4_blockwise -- into ``packed`` (uint8, int4_packed_bytes bytes)."""
    for t, n, d in ((w, "w", _U8), (scales, "scales", _F16), (zero_points, "zero_points", _U8),
                    (packed, "packed", _U8)):
        _arg(t, n, d)
    if w.dim() != 2:
        raise ValueError(f"w: expected a 2-D tensor [N, K/2], got shape {tuple(w.shape)}")
    N, K = w.shape[0], 2 * w.shape[1]
    _dense(w, "w", (N, K // 2))
    if block_size > 0 and K % block_size == 0:  # otherwise the library rejects the call
        nb = K // block_size
        _dense(scales, "scales", (N, nb))
        _dense(zero_points, "zero_points", (N, (nb + 1) // 2))
    if not packed.is_contiguous():
        raise ValueError("packed must be contiguous")
    _check("int4_repack", load_library().int4_repack(
        _ptr(w), _ptr(scales), _ptr(zero_points), _ptr(packed), packed.numel(), N, K, block_size,
        layout, _stream(stream)))
    return packed


def qgemv_int4_packed(x: torch.Tensor, packed: torch.Tensor, y: torch.Tensor, block_size: int,
                      layout: int = INT4_LAYOUT_TILE16_V1, stream=None) -> torch.Tensor:
    """y[M,N] = x[M,K] . dequant(W)^T with W packed by int4_repack (N from y,
    K from x).  x fp16 [M,K]; y fp16/bf16/fp32 [M,N]."""
    for t, n, d in ((x, "x", tuple(_X_TYPES)), (packed, "packed", _U8), (y, "y", _OUT)):
        _arg(t, n, d)
    if y.dim() != 2:
        raise ValueError(f"y: expected a 2-D tensor [M, N], got shape {tuple(y.shape)}")
    N = y.shape[1]
    M, K = _xy(x, y, N)
    if not packed.is_contiguous():
        raise ValueError("packed must be contiguous")
    _check("qgemv_int4_packed", load_library().qgemv_int4_packed(
        _ptr(x), _ld(x), _X_TYPES[x.dtype], _ptr(packed), packed.numel(), layout, _ptr(y), _ld(y),
        _OUT_TYPES[y.dtype], M, N, K, block_size, _stream(stream)))
    return y


def _q4k_rows(w: torch.Tensor) -> int:
    if w.dim() != 2:
        raise ValueError(f"w: expected a 2-D uint8 tensor [N, K/256*144], got shape {tuple(w.shape)}")
    return w.shape[0]


def qgemv_q4k(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """q4_K GEMV.  x fp32 [M,K]; w uint8 [N, K/256*144]; y fp32 [M,N]."""
    for t, n, d in ((x, "x", _F32), (w, "w", _U8), (y, "y", _F32)):
        _arg(t, n, d)
    N = _q4k_rows(w)
    M, K = _xy(x, y, N)
    if K % 256 == 0:  # otherwise the library rejects the call
        _dense(w, "w", (N, K // 256 * 144))
    _check("qgemv_q4k", load_library().qgemv_q4k(
        _ptr(x), _ld(x), _ptr(w), _ptr(y), _ld(y), M, N, K, _stream(stream)))
    return y


def qgemv_q4k_dsc(x: torch.Tensor, w: torch.Tensor, dsc: Optional[torch.Tensor],
                  y: torch.Tensor, stream=None) -> torch.Tensor:
    """q4_K GEMV with (dv, mv) read from the W_dsc plane (fp32 [(K/32)*N, 2])."""
    for t, n, d in ((x, "x", _F32), (w, "w", _U8), (dsc, "dsc", _F32), (y, "y", _F32)):
        _arg(t, n, d)
    N = _q4k_rows(w)
    M, K = _xy(x, y, N)
    if K % 256 == 0:  # otherwise the library rejects the call
        _dense(w, "w", (N, K // 256 * 144))
        _dense(dsc, "dsc", (K // 32 * N, 2))
    _check("qgemv_q4k_dsc", load_library().qgemv_q4k_dsc(
        _ptr(x), _ld(x), _ptr(w), _ptr(dsc), _ptr(y), _ld(y), M, N, K, _stream(stream)))
    return y


def gemv_bf16(x: torch.Tensor, w: torch.Tensor, y: torch.Tensor, stream=None) -> torch.Tensor:
    """y[M,N] = x[M,K] . w[N,K]^T in bf16 (any K, any 2-byte offset)."""
    for t, n, d in ((x, "x", _BF16), (w, "w", _BF16), (y, "y", _OUT)):
        _arg(t, n, d)
    if w.dim() != 2:
        raise ValueError(f"w: expected a 2-D tensor [N, K], got shape {tuple(w.shape)}")
    N = w.shape[0]
    M, K = _xy(x, y, N)
    _dims(w, "w", (N, K))
    _check("gemv_bf16", load_library().gemv_bf16(
        _ptr(x), _ld(x), _ptr(w), _ld(w), _ptr(y), _ld(y), _OUT_TYPES[y.dtype], M, N, K,
        _stream(stream)))
    return y


def q4k_dsc_plane_bytes(N: int, K: int) -> int:
    return int(load_library().q4k_dsc_plane_bytes(N, K))


def q4k_build_dsc_plane(w: torch.Tensor, dsc_out: torch.Tensor, N: int, K: int,
                        stream=None) -> torch.Tensor:
    """Load-time repack of raw q4_K weights into the chunk-major W_dsc plane."""
    _arg(w, "w", _U8)
    _arg(dsc_out, "dsc_out", _F32)
    if N >= 0 and K >= 256 and K % 256 == 0:  # otherwise the library rejects the call
        _dense(w, "w", (N, K // 256 * 144))
        _dense(dsc_out, "dsc_out", (K // 32 * N, 2))
    _check("q4k_build_dsc_plane", load_library().q4k_build_dsc_plane(
        _ptr(w), _ptr(dsc_out), N, K, _stream(stream)))
    return dsc_out


def q4k_mmq_workspace_bytes(T: int, K: int) -> int:
    return int(load_library().q4k_mmq_workspace_bytes(T, K))


def q8_quantize_rows(x: torch.Tensor, qa: torch.Tensor, sda: torch.Tensor, stream=None):
    """8-bit activation prepass.  x fp32 [T,K]; qa int8 [T,K]; sda fp32 [T,K/32,2]."""
    for t, n, d in ((x, "x", _F32), (qa, "qa", _I8), (sda, "sda", _F32)):
        _arg(t, n, d)
    if x.dim() != 2:
        raise ValueError(f"x: expected a 2-D tensor [T, K], got shape {tuple(x.shape)}")
    T, K = x.shape
    _dense(qa, "qa", (T, K))
    if K % 32 == 0:  # otherwise the library rejects the call
        _dense(sda, "sda", (T, K // 32, 2))
    _check("q8_quantize_rows", load_library().q8_quantize_rows(
        _ptr(x), _ld(x), _ptr(qa), _ptr(sda), T, K, _stream(stream)))
    return qa, sda


def qgemm_q4k_mmq(x: torch.Tensor, w: torch.Tensor, dsc: Optional[torch.Tensor], y: torch.Tensor,
                  workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """q4_K prefill: y[T,N] fp32 from x fp32 [T,K], raw q4_K w, its W_dsc plane
    and a caller-owned workspace (uint8, >= q4k_mmq_workspace_bytes(T, K))."""
    for t, n, d in ((x, "x", _F32), (w, "w", _U8), (dsc, "dsc", _F32), (y, "y", _F32),
                    (workspace, "workspace", None)):
        _arg(t, n, d)
    N = _q4k_rows(w)
    T, K = _xy(x, y, N)
    if K % 256 == 0:  # otherwise the library rejects the call
        _dense(w, "w", (N, K // 256 * 144))
        _dense(dsc, "dsc", (K // 32 * N, 2))
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _check("qgemm_q4k_mmq", load_library().qgemm_q4k_mmq(
        _ptr(x), _ld(x), _ptr(w), _ptr(dsc), _ptr(y), _ld(y), T, N, K, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream)))
    return y


def qgemm_q4k_mmq_noalloc(x: torch.Tensor, w: torch.Tensor, dsc: Optional[torch.Tensor],
                          y: torch.Tensor, stream=None) -> torch.Tensor:
    """The q4_K prefill product with the workspace in the library's static
    device array (no allocation anywhere; at most MMQ_NOALLOC_SCRATCH_BYTES of
    workspace, see q4k_mmq_workspace_bytes).  Calls that overlap on one GPU
    share that array and race."""
    for t, n, d in ((x, "x", _F32), (w, "w", _U8), (dsc, "dsc", _F32), (y, "y", _F32)):
        _arg(t, n, d)
    N = _q4k_rows(w)
    T, K = _xy(x, y, N)
    if K % 256 == 0:  # otherwise the library rejects the call
        _dense(w, "w", (N, K // 256 * 144))
        _dense(dsc, "dsc", (K // 32 * N, 2))
    _check("qgemm_q4k_mmq_noalloc", load_library().qgemm_q4k_mmq_noalloc(
        _ptr(x), _ld(x), _ptr(w), _ptr(dsc), _ptr(y), _ld(y), T, N, K, _stream(stream)))
    return y


def last_launch() -> str:
    """Kernels enqueued by this thread's last library call ("" if none)."""
    return load_library().qg_last_launch().decode()


def path_names() -> list:
    L = load_library()
    return [L.qg_path_name(i).decode() for i in range(L.qg_path_count())]


def path_launches() -> dict:
    """Launches per kernel path since the library was loaded (all threads)."""
    L = load_library()
    return {L.qg_path_name(i).decode(): int(L.qg_path_launches(i)) for i in range(L.qg_path_count())}

"""Decode-time dispatch on top of the C ABI: q4_K plane registration with
liveness labels, and row groups for any number of rows of x.

q4_K plane ("62 . r59 -- q4_K W_dsc plane + riders", section 3.1): the plane of
a weight is built once at load time and kept in a map keyed by the weight's
device pointer and shape (N, K); the entry is dropped when the weight tensor
is freed, so a later tensor at a reused address never meets a stale plane.
A call takes the plane when one is registered.  When a registration failed,
the call degrades to in-kernel decode, with a warning once per process and a
label that says so: which path ran cannot be told from the result, so a
silent degradation would go unnoticed.  Labels (counted by ``liveness()``):

    dsc-plane             the plane was used
    in-kernel(dsc=off)    no plane registered for this weight, or the plane
                          path is switched off (QGEMV_Q4K_DSC=0, or
                          use_plane=False) -- the page's contrast switch
    in-kernel(fallback!)  a registration was attempted and failed
    mmq(q8 activations)   the prefill product (8-bit activations, the plane)

Rows (the AstrAI backend commit list: decode-time linear layers go to the GEMV
for small M): the kernels take M = 1..8; these wrappers take any M >= 1 and
run row groups of at most 8 rows of x (each group reads the weights again).

Prefill arm (the same page, section 3.2: the dispatch arm that quantizes the
activations): with a plane registered, a q4_K call with at least
``prefill_min_rows`` rows of x (argument, else QGEMV_Q4K_MMQ_MIN_ROWS; 0 =
never, the default) goes to the prefill product instead of row groups.  It is
opt-in because its result is a different computation (activations rounded to 8
bits per block of 32).  Measured on the 7B layer shapes with cold weights, the
product overtakes the row groups from about 16-32 rows of x.  Its workspace is
kept per (device, stream) and grows on demand.

int4 packed copy (the onnx-genai pull request #1000, "Roadmap recommendation":
an offline repack with a versioned layout flag): ``register_int4_packed`` writes
the packed layout of a MatMulNBits weight once, kept like a plane (keyed by the
weight's device pointer, shape and block size, dropped with the weight).
``int4_linear`` then takes it for row groups of at least 2 rows of x on
matrices of at least as many 16-row tiles as the GPU has CUs, where it measured
faster than the original layout (lm_head M = 2: 64 against 75 us; 4096 x 11008
M = 8: 13.9 against 17.3); on shorter matrices and at M = 1 the original
layout's kernels are faster and run.  ``int4_liveness()`` counts row groups per
layout.

Everything here is argument handling; every output element is computed by the
library's HIP kernels.  ``explain()`` returns the library's description of the
kernels the calling thread's last call enqueued.
"""
from __future__ import annotations

import os
import threading
import warnings
import weakref
from typing import Optional, Tuple

import torch

from . import qgemv as _q

MAX_ROWS = 8
LABEL_PLANE = "dsc-plane"
LABEL_OFF = "in-kernel(dsc=off)"
LABEL_FALLBACK = "in-kernel(fallback!)"
LABEL_MMQ = "mmq(q8 activations)"

_lock = threading.Lock()
_planes = {}   # (weight device pointer, N, K) -> plane tensor
_failed = {}   # (weight device pointer, N, K) -> reason the registration failed
_finalizers = {}  # (weight device pointer, N, K) -> weakref.finalize on the weight tensor
_warned = False
_liveness = {LABEL_PLANE: 0, LABEL_OFF: 0, LABEL_FALLBACK: 0, LABEL_MMQ: 0}
_workspaces = {}  # (device index, stream handle) -> uint8 workspace of the prefill product
LABEL_INT4 = "int4"
LABEL_INT4_PACKED = "int4-packed"
_packed = {}  # (weight device pointer, N, K, block size) -> packed uint8 tensor
_packed_finalizers = {}
_int4_liveness = {LABEL_INT4: 0, LABEL_INT4_PACKED: 0}
_cus = {}  # device index -> compute units


def _plane_enabled() -> bool:
    return os.environ.get("QGEMV_Q4K_DSC", "1") != "0"


def _mmq_min_rows() -> int:
    v = os.environ.get("QGEMV_Q4K_MMQ_MIN_ROWS", "0")
    try:
        return max(0, int(v))
    except ValueError:
        raise ValueError(f"QGEMV_Q4K_MMQ_MIN_ROWS must be an integer, got {v!r}") from None


def _workspace(device: torch.device, stream, nbytes: int) -> torch.Tensor:
    """The prefill workspace of (device, stream), at least ``nbytes`` long.
    Growing it first waits for the work queued on that stream, which may
    still read the old buffer."""
    handle = _q._stream(stream)
    key = (device.index, handle)
    with _lock:
        ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None and device.type == "cuda":
            torch.cuda.ExternalStream(handle, device=device).synchronize()
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        with _lock:
            _workspaces[key] = ws
    return ws


def q4k_shape(w: torch.Tensor) -> Tuple[int, int]:
    """(N, K) of raw q4_K weights stored as uint8 [N, K/256*144]."""
    if w.dim() != 2 or w.shape[1] % 144 != 0:
        raise ValueError("q4_K weights must be a 2-D uint8 tensor [N, K/256*144]")
    return w.shape[0], w.shape[1] // 144 * 256


def _key(w: torch.Tensor):
    N, K = q4k_shape(w)
    return (w.data_ptr(), N, K)


def _forget(key) -> None:
    with _lock:
        _planes.pop(key, None)
        _failed.pop(key, None)
        _finalizers.pop(key, None)


def _track(key, w: torch.Tensor) -> None:
    """Drop the registry entry of ``key`` when the tensor ``w`` is freed."""
    with _lock:
        if key in _finalizers and _finalizers[key].alive:
            return
        _finalizers[key] = weakref.finalize(w, _forget, key)


def register_q4k_plane(w: torch.Tensor, stream=None) -> bool:
    """Build the W_dsc plane of raw q4_K weights ``w`` and register it under
    w's device pointer and shape.  Returns False, and remembers why, when the
    plane cannot be allocated or built; calls on ``w`` then fall back to
    in-kernel decode with the fallback label.  The entry lives as long as the
    tensor ``w``."""
    try:
        N, K = q4k_shape(w)
    except ValueError:
        return False  # not a q4_K weight: no entry, calls on it are refused too
    key = (w.data_ptr(), N, K)
    _track(key, w)
    try:
        nbytes = _q.q4k_dsc_plane_bytes(N, K)
        if nbytes == 0 and N > 0:
            raise ValueError(f"no plane for N={N}, K={K}")
        dsc = torch.empty((nbytes // 8, 2), dtype=torch.float32, device=w.device)
        _q.q4k_build_dsc_plane(w, dsc, N, K, stream)
    except (ValueError, RuntimeError) as e:  # QgemvError and allocation failures included
        with _lock:
            _planes.pop(key, None)
            _failed[key] = str(e)
        return False
    with _lock:
        _planes[key] = dsc
        _failed.pop(key, None)
    return True


def unregister_q4k_plane(w: torch.Tensor) -> None:
    key = _key(w)
    with _lock:
        fin = _finalizers.get(key)
    if fin is not None:
        fin.detach()
    _forget(key)


def q4k_plane_of(w: torch.Tensor) -> Optional[torch.Tensor]:
    with _lock:
        return _planes.get(_key(w))


def _row_groups(M: int):
    for m0 in range(0, M, MAX_ROWS):
        yield m0, min(M, m0 + MAX_ROWS)


def _count(label: str) -> None:
    with _lock:
        _liveness[label] += 1


def q4k_linear(x: torch.Tensor, w: torch.Tensor, y: Optional[torch.Tensor] = None,
               use_plane: bool = True, stream=None,
               prefill_min_rows: Optional[int] = None) -> Tuple[torch.Tensor, str]:
    """y[M, N] = x[M, K] . dequant(w)^T for raw q4_K weights, through the
    registered plane when there is one; with a plane and at least
    ``prefill_min_rows`` rows of x (> 0), through the prefill product.
    Returns (y, liveness label)."""
    global _warned
    N, K = q4k_shape(w)
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    key = (w.data_ptr(), N, K)
    with _lock:
        dsc = _planes.get(key)
        failure = _failed.get(key)
    if not (use_plane and _plane_enabled()):
        label, dsc = LABEL_OFF, None
    elif dsc is not None:
        label = LABEL_PLANE
    elif failure is not None:
        label = LABEL_FALLBACK
        with _lock:
            first = not _warned
            _warned = True
        if first:
            warnings.warn(f"q4_K plane unavailable ({failure}); falling back to in-kernel "
                          f"decode (this warning is shown once per process)", RuntimeWarning,
                          stacklevel=2)
    else:
        label = LABEL_OFF
    min_rows = _mmq_min_rows() if prefill_min_rows is None else prefill_min_rows
    if dsc is not None and min_rows > 0 and M >= min_rows:
        ws = _workspace(x.device, stream, _q.q4k_mmq_workspace_bytes(M, K))
        _q.qgemm_q4k_mmq(x, w, dsc, y, ws, stream)
        _count(LABEL_MMQ)
        return y, LABEL_MMQ
    for m0, m1 in _row_groups(M):
        if dsc is not None:
            _q.qgemv_q4k_dsc(x[m0:m1], w, dsc, y[m0:m1], stream)
        else:
            _q.qgemv_q4k(x[m0:m1], w, y[m0:m1], stream)
    _count(label)
    return y, label


def _int4_key(w: torch.Tensor, block_size: int):
    if w.dim() != 2:
        raise ValueError("int4 weights must be a 2-D uint8 tensor [N, K/2]")
    return (w.data_ptr(), w.shape[0], 2 * w.shape[1], block_size)


def _forget_packed(key) -> None:
    with _lock:
        _packed.pop(key, None)
        _packed_finalizers.pop(key, None)


def register_int4_packed(w: torch.Tensor, scales: torch.Tensor,
                         zero_points: Optional[torch.Tensor], block_size: int,
                         stream=None) -> bool:
    """Write the packed layout of (w, scales, zero_points) once and register it
    under w's device pointer, shape and block size.  Returns False when the
    shape has no packed layout (K not a multiple of 128 or of the block) or the
    repack fails; calls on ``w`` then keep the original layout."""
    key = _int4_key(w, block_size)
    N, K = key[1], key[2]
    try:
        nbytes = _q.int4_packed_bytes(N, K, block_size)
        if nbytes <= 0:
            return False
        packed = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
        _q.int4_repack(w, scales, zero_points, packed, block_size, stream=stream)
    except (ValueError, RuntimeError):
        return False
    with _lock:
        _packed[key] = packed
        if key not in _packed_finalizers or not _packed_finalizers[key].alive:
            _packed_finalizers[key] = weakref.finalize(w, _forget_packed, key)
    return True


def unregister_int4_packed(w: torch.Tensor, block_size: int) -> None:
    key = _int4_key(w, block_size)
    with _lock:
        fin = _packed_finalizers.get(key)
    if fin is not None:
        fin.detach()
    _forget_packed(key)


def int4_packed_of(w: torch.Tensor, block_size: int) -> Optional[torch.Tensor]:
    with _lock:
        return _packed.get(_int4_key(w, block_size))


def _compute_units(device: torch.device) -> int:
    idx = device.index if device.index is not None else torch.cuda.current_device()
    with _lock:
        if idx not in _cus:
            _cus[idx] = torch.cuda.get_device_properties(idx).multi_processor_count
        return _cus[idx]


def int4_linear(x: torch.Tensor, w: torch.Tensor, scales: torch.Tensor,
                zero_points: Optional[torch.Tensor], block_size: int,
                y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """MatMulNBits int4 for any M >= 1 (row groups of at most 8); fp16 y
    unless ``y`` is given.  A registered packed copy serves row groups of at
    least 2 rows on matrices of at least as many 16-row tiles as CUs."""
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, w.shape[0]), dtype=torch.float16, device=x.device)
    packed = int4_packed_of(w, block_size)
    tall = packed is not None and (w.shape[0] + 15) // 16 >= _compute_units(x.device)
    for m0, m1 in _row_groups(M):
        if tall and m1 - m0 >= 2:
            _q.qgemv_int4_packed(x[m0:m1], packed, y[m0:m1], block_size, stream=stream)
            label = LABEL_INT4_PACKED
        else:
            _q.qgemv_int4_blockwise(x[m0:m1], w, scales, zero_points, y[m0:m1], block_size, stream)
            label = LABEL_INT4
        with _lock:
            _int4_liveness[label] += 1
    return y


def bf16_linear(x: torch.Tensor, w: torch.Tensor, y: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """bf16 GEMV for any M >= 1 (row groups of at most 8); bf16 y unless
    ``y`` is given."""
    M = x.shape[0]
    if y is None:
        y = torch.empty((M, w.shape[0]), dtype=torch.bfloat16, device=x.device)
    for m0, m1 in _row_groups(M):
        _q.gemv_bf16(x[m0:m1], w, y[m0:m1], stream)
    return y


def liveness() -> dict:
    """Calls per q4_K liveness label since the last reset."""
    with _lock:
        return dict(_liveness)


def int4_liveness() -> dict:
    """Row groups of int4 calls per layout (original, packed) since the last reset."""
    with _lock:
        return dict(_int4_liveness)


def reset_liveness() -> None:
    global _warned
    with _lock:
        for k in _liveness:
            _liveness[k] = 0
        for k in _int4_liveness:
            _int4_liveness[k] = 0
        _warned = False


def explain() -> str:
    """The kernels the calling thread's last library call enqueued."""
    return _q.last_launch()

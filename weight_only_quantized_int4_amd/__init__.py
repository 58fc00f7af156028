"""MI355X-native weight-only quantized decode GEMV (int4 MatMulNBits, q4_K, bf16)
and the q4_K prefill product with 8-bit activations.

The compute lives in ``libqgemv.so`` (hand-written HIP kernels for gfx950 behind
a C ABI, see ``include/qgemv.h``).  ``qgemv`` is the thin ctypes binding with
the same entry-point names; PyTorch only supplies device memory and streams.
"""
from .qgemv import (  # noqa: F401
    QG_BF16, QG_F16, QG_F32, QgemvError, gemv_bf16, last_launch, library_path, load_library,
    path_launches, path_names, q4k_build_dsc_plane, q4k_dsc_plane_bytes, qgemv_int4_blockwise,
    qgemv_q4k, qgemv_q4k_dsc, q4k_mmq_workspace_bytes, q8_quantize_rows, qgemm_q4k_mmq,
    qgemm_q4k_mmq_noalloc, MMQ_NOALLOC_SCRATCH_BYTES, INT4_LAYOUT_TILE16_V1, int4_packed_bytes,
    int4_repack, qgemv_int4_packed,
)
from . import dispatch  # noqa: F401

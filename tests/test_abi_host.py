"""Host-side checks of libqgemv.so: it loads, exports exactly the C ABI that
include/qgemv.h declares, and its argument validation rejects bad calls before
anything reaches the GPU.  CPU only: every call here fails validation, so no
kernel is launched and no pointer is dereferenced.
"""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import weight_only_quantized_int4_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")

QG_OK, QG_ERR_NULL_POINTER, QG_ERR_BAD_SHAPE, QG_ERR_UNSUPPORTED = 0, 1, 2, 3
QG_ERR_MISALIGNED, QG_ERR_ALIAS, QG_ERR_HIP = 4, 5, 6


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) -
                  {"if", "sizeof", "defined"})


def test_header_declares_the_entry_points():
    names = _declared_functions()
    assert names == sorted(["qgemv_int4_blockwise", "qgemv_q4k", "qgemv_q4k_dsc", "gemv_bf16",
                            "q4k_dsc_plane_bytes", "q4k_build_dsc_plane", "qg_status_string",
                            "qg_last_error", "qg_last_launch", "qg_path_count", "qg_path_name",
                            "qg_path_launches", "q4k_mmq_workspace_bytes", "q8_quantize_rows",
                            "qgemm_q4k_mmq", "qgemm_q4k_mmq_noalloc", "int4_packed_bytes",
                            "int4_repack", "qgemv_int4_packed"])


def test_library_exports_exactly_the_header():
    L = q.load_library()
    for name in _declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", q.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(line.split()[-1] for line in out.splitlines() if " T " in line)
    assert exported == _declared_functions()


def test_library_has_gfx950_code_object():
    """The offload bundle of the library holds device code for gfx950 and for
    no other target (bundle entry ids name the target)."""
    with open(q.library_path(), "rb") as f:
        data = f.read()
    targets = set(re.findall(rb"hipv4-amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", data))
    assert targets == {b"gfx950"}, targets


def test_status_strings():
    L = q.load_library()
    names = ["QG_OK", "QG_ERR_NULL_POINTER", "QG_ERR_BAD_SHAPE", "QG_ERR_UNSUPPORTED",
             "QG_ERR_MISALIGNED", "QG_ERR_ALIAS", "QG_ERR_HIP"]
    for i, n in enumerate(names):
        assert L.qg_status_string(i).decode() == n
    assert L.qg_status_string(99).decode() == "QG_ERR_UNKNOWN"


def test_plane_bytes():
    assert q.q4k_dsc_plane_bytes(4096, 4096) == 4096 * 4096 // 4
    assert q.q4k_dsc_plane_bytes(11008, 4096) == 11008 * 4096 // 4
    assert q.q4k_dsc_plane_bytes(0, 256) == 0
    assert q.q4k_dsc_plane_bytes(3, 100) == 0
    assert q.q4k_dsc_plane_bytes(-1, 256) == 0


# Fake, never-dereferenced device addresses (16-byte aligned, far apart).
A = 0x7F0000000000
B = 0x7F0100000000
C = 0x7F0200000000
D = 0x7F0300000000
E = 0x7F0400000000


def _int4(L, x=A, ldx=64, w=B, s=C, zp=D, y=E, ldy=16, yt=0, M=1, N=16, K=64, bs=32, xt=0):
    return L.qgemv_int4_blockwise(x, ldx, xt, w, s, zp, y, ldy, yt, M, N, K, bs, None)


def test_int4_validation():
    L = q.load_library()
    assert _int4(L, x=None) == QG_ERR_NULL_POINTER
    assert _int4(L, s=None) == QG_ERR_NULL_POINTER
    assert _int4(L, y=None) == QG_ERR_NULL_POINTER
    for M in (0, 9, -1):
        assert _int4(L, M=M) == QG_ERR_BAD_SHAPE
        assert f"M = {M}" in L.qg_last_error().decode()
    assert _int4(L, N=-1) == QG_ERR_BAD_SHAPE
    assert _int4(L, K=0) == QG_ERR_BAD_SHAPE
    assert _int4(L, K=96, bs=64) == QG_ERR_BAD_SHAPE       # K % bs != 0
    assert _int4(L, bs=16) == QG_ERR_UNSUPPORTED
    assert _int4(L, bs=48) == QG_ERR_UNSUPPORTED
    assert _int4(L, yt=7) == QG_ERR_UNSUPPORTED
    # activations: fp16 only; bf16 (and anything else) is refused, not converted
    assert _int4(L, xt=1) == QG_ERR_UNSUPPORTED
    assert "x_type" in L.qg_last_error().decode()
    assert _int4(L, xt=2) == QG_ERR_UNSUPPORTED
    assert _int4(L, ldx=32) == QG_ERR_BAD_SHAPE
    assert _int4(L, ldy=8) == QG_ERR_BAD_SHAPE
    assert _int4(L, w=B + 8) == QG_ERR_MISALIGNED
    assert _int4(L, x=A + 1) == QG_ERR_MISALIGNED
    assert _int4(L, y=E + 2, yt=2) == QG_ERR_MISALIGNED
    assert _int4(L, y=B + 16) == QG_ERR_ALIAS               # y inside w
    assert _int4(L, y=A + 64) == QG_ERR_ALIAS               # y inside x (x spans 128 B)
    assert _int4(L, zp=E + 8) == QG_ERR_ALIAS               # zero points overlap y
    # N == 0 is an empty problem: OK, nothing enqueued (no GPU needed)
    assert _int4(L, N=0) == QG_OK
    assert L.qg_last_error().decode() == ""
    # a huge w is refused up front (kernels address with 32-bit offsets)
    assert _int4(L, N=1 << 20, K=1 << 13, ldx=1 << 13, ldy=1 << 20) == QG_ERR_UNSUPPORTED


def test_int4_packed_bytes():
    """Records of 16 rows x 128 weights: 1024 code bytes + 32 scale bytes per
    block of the item + 16 (32 for 4 blocks) zero-point bytes."""
    L = q.load_library()
    V1 = q.INT4_LAYOUT_TILE16_V1
    assert L.int4_packed_bytes(16, 128, 32, V1) == 1184
    assert L.int4_packed_bytes(16, 128, 64, V1) == 1104
    assert L.int4_packed_bytes(16, 128, 128, V1) == 1072
    assert L.int4_packed_bytes(16, 256, 256, V1) == 2 * 1072
    assert L.int4_packed_bytes(17, 256, 32, V1) == 2 * 2 * 1184   # 2 tiles x 2 items
    assert L.int4_packed_bytes(0, 4096, 32, V1) == 0
    assert L.int4_packed_bytes(151936, 4096, 32, V1) == 9496 * 32 * 1184
    for args in ((16, 100, 32, V1), (16, 64, 32, V1), (16, 128, 256, V1), (16, 128, 16, V1),
                 (16, 128, 32, 2), (16, 128, 32, 0), (-1, 128, 32, V1)):
        assert L.int4_packed_bytes(*args) == 0, args


def _repack(L, w=B, s=C, zp=D, out=E, nbytes=1 << 20, N=16, K=256, bs=32, layout=1):
    return L.int4_repack(w, s, zp, out, nbytes, N, K, bs, layout, None)


def _packed(L, x=A, ldx=256, xt=0, wp=B, nbytes=1 << 20, layout=1, y=E, ldy=16, yt=0, M=1, N=16,
            K=256, bs=32):
    return L.qgemv_int4_packed(x, ldx, xt, wp, nbytes, layout, y, ldy, yt, M, N, K, bs, None)


def test_int4_repack_and_packed_validation():
    L = q.load_library()
    assert _repack(L, w=None) == QG_ERR_NULL_POINTER
    assert _repack(L, out=None) == QG_ERR_NULL_POINTER
    assert _repack(L, layout=2) == QG_ERR_UNSUPPORTED
    assert "layout" in L.qg_last_error().decode()
    assert _repack(L, bs=16) == QG_ERR_UNSUPPORTED
    assert _repack(L, K=96) == QG_ERR_BAD_SHAPE
    assert _repack(L, K=128, bs=256) == QG_ERR_BAD_SHAPE
    assert _repack(L, nbytes=2 * 1184 - 1) == QG_ERR_BAD_SHAPE
    assert _repack(L, w=B + 2) == QG_ERR_MISALIGNED
    assert _repack(L, out=E + 8) == QG_ERR_MISALIGNED
    assert _repack(L, out=B + 64) == QG_ERR_ALIAS
    assert _repack(L, N=0) == QG_OK
    assert _packed(L, x=None) == QG_ERR_NULL_POINTER
    assert _packed(L, wp=None) == QG_ERR_NULL_POINTER
    assert _packed(L, layout=0) == QG_ERR_UNSUPPORTED
    assert _packed(L, xt=1) == QG_ERR_UNSUPPORTED
    assert _packed(L, M=9) == QG_ERR_BAD_SHAPE
    assert _packed(L, K=192, ldx=192) == QG_ERR_BAD_SHAPE
    assert _packed(L, nbytes=100) == QG_ERR_BAD_SHAPE
    assert _packed(L, ldx=128) == QG_ERR_BAD_SHAPE
    assert _packed(L, ldy=8) == QG_ERR_BAD_SHAPE
    assert _packed(L, yt=5) == QG_ERR_UNSUPPORTED
    assert _packed(L, wp=B + 8) == QG_ERR_MISALIGNED
    assert _packed(L, y=E + 2, yt=2) == QG_ERR_MISALIGNED
    assert _packed(L, y=B + 64) == QG_ERR_ALIAS
    assert _packed(L, K=1 << 17, ldx=1 << 17, nbytes=1 << 24) == QG_ERR_UNSUPPORTED  # x beyond LDS
    assert _packed(L, N=0) == QG_OK


def _q4k(L, x=A, ldx=256, w=B, y=E, ldy=16, M=1, N=16, K=256, dsc=None, use_dsc=False):
    if use_dsc:
        return L.qgemv_q4k_dsc(x, ldx, w, dsc, y, ldy, M, N, K, None)
    return L.qgemv_q4k(x, ldx, w, y, ldy, M, N, K, None)


def test_q4k_validation():
    L = q.load_library()
    assert _q4k(L, w=None) == QG_ERR_NULL_POINTER
    assert _q4k(L, K=300, ldx=300) == QG_ERR_BAD_SHAPE
    assert _q4k(L, K=128, ldx=128) == QG_ERR_BAD_SHAPE
    assert _q4k(L, M=9) == QG_ERR_BAD_SHAPE
    assert _q4k(L, w=B + 4) == QG_ERR_MISALIGNED
    assert _q4k(L, x=A + 2) == QG_ERR_MISALIGNED
    assert _q4k(L, y=B + 64) == QG_ERR_ALIAS
    assert _q4k(L, N=0) == QG_OK
    # the plane entry point never falls back silently
    assert _q4k(L, use_dsc=True, dsc=None) == QG_ERR_NULL_POINTER
    assert "NULL" in L.qg_last_error().decode()
    assert _q4k(L, use_dsc=True, dsc=C + 8) == QG_ERR_MISALIGNED
    assert _q4k(L, use_dsc=True, dsc=E) == QG_ERR_ALIAS


def test_mmq_workspace_bytes():
    # codes T*K (a multiple of 256 since K is), then T*(K/32) float2
    assert q.q4k_mmq_workspace_bytes(1, 256) == 256 + 8 * 8
    assert q.q4k_mmq_workspace_bytes(3, 512) == 1536 + 3 * 16 * 8
    assert q.q4k_mmq_workspace_bytes(5, 256) == 1280 + 5 * 8 * 8
    assert q.q4k_mmq_workspace_bytes(7, 256) == 1792 + 7 * 8 * 8
    assert q.q4k_mmq_workspace_bytes(0, 256) == 0
    assert q.q4k_mmq_workspace_bytes(4, 100) == 0
    assert q.q4k_mmq_workspace_bytes(4, 128) == 0


def _mmq(L, x=A, ldx=256, w=B, dsc=C, y=E, ldy=16, T=4, N=16, K=256, ws=D, wsb=None):
    wsb = L.q4k_mmq_workspace_bytes(T, K) if wsb is None else wsb
    return L.qgemm_q4k_mmq(x, ldx, w, dsc, y, ldy, T, N, K, ws, wsb, None)


def test_mmq_validation():
    L = q.load_library()
    assert _mmq(L, x=None) == QG_ERR_NULL_POINTER
    assert _mmq(L, dsc=None) == QG_ERR_NULL_POINTER
    assert "no silent fallback" in L.qg_last_error().decode()
    assert _mmq(L, ws=None) == QG_ERR_NULL_POINTER
    assert _mmq(L, K=300, ldx=300) == QG_ERR_BAD_SHAPE
    assert _mmq(L, K=128, ldx=128) == QG_ERR_BAD_SHAPE
    assert _mmq(L, T=-1) == QG_ERR_BAD_SHAPE
    assert _mmq(L, ldx=128) == QG_ERR_BAD_SHAPE
    assert _mmq(L, ldy=8) == QG_ERR_BAD_SHAPE
    assert _mmq(L, wsb=100) == QG_ERR_BAD_SHAPE
    assert "workspace" in L.qg_last_error().decode()
    assert _mmq(L, w=B + 8) == QG_ERR_MISALIGNED
    assert _mmq(L, dsc=C + 8) == QG_ERR_MISALIGNED
    assert _mmq(L, ws=D + 16) == QG_ERR_MISALIGNED
    assert _mmq(L, x=A + 2) == QG_ERR_MISALIGNED
    assert _mmq(L, y=B + 64) == QG_ERR_ALIAS          # y inside w
    assert _mmq(L, ws=B) == QG_ERR_ALIAS              # workspace over w
    assert _mmq(L, ws=E) == QG_ERR_ALIAS              # workspace over y
    # empty problems enqueue nothing (no GPU needed)
    assert _mmq(L, T=0) == QG_OK and _mmq(L, N=0) == QG_OK
    assert L.qg_last_error().decode() == ""
    # the prepass alone
    assert L.q8_quantize_rows(None, 64, B, C, 2, 64, None) == QG_ERR_NULL_POINTER
    assert L.q8_quantize_rows(A, 64, B, C, 2, 48, None) == QG_ERR_BAD_SHAPE
    assert L.q8_quantize_rows(A, 32, B, C, 2, 64, None) == QG_ERR_BAD_SHAPE
    assert L.q8_quantize_rows(A, 64, B, C + 4, 2, 64, None) == QG_ERR_MISALIGNED
    assert L.q8_quantize_rows(A, 64, A + 16, C, 2, 64, None) == QG_ERR_ALIAS
    assert L.q8_quantize_rows(A, 64, B, C, 0, 64, None) == QG_OK


def test_plane_builder_validation():
    L = q.load_library()
    assert L.q4k_build_dsc_plane(None, C, 4, 256, None) == QG_ERR_NULL_POINTER
    assert L.q4k_build_dsc_plane(B, C, 4, 100, None) == QG_ERR_BAD_SHAPE
    assert L.q4k_build_dsc_plane(B, C, -1, 256, None) == QG_ERR_BAD_SHAPE
    assert L.q4k_build_dsc_plane(B + 1, C, 4, 256, None) == QG_ERR_MISALIGNED
    assert L.q4k_build_dsc_plane(B, B + 32, 4, 256, None) == QG_ERR_ALIAS
    assert L.q4k_build_dsc_plane(B, C, 0, 256, None) == QG_OK


def _bf16(L, x=A, ldx=64, w=B, ldw=64, y=E, ldy=16, yt=1, M=1, N=16, K=64):
    return L.gemv_bf16(x, ldx, w, ldw, y, ldy, yt, M, N, K, None)


def test_bf16_validation():
    L = q.load_library()
    assert _bf16(L, w=None) == QG_ERR_NULL_POINTER
    assert _bf16(L, M=9) == QG_ERR_BAD_SHAPE
    assert _bf16(L, K=0) == QG_ERR_BAD_SHAPE
    assert _bf16(L, ldw=63) == QG_ERR_BAD_SHAPE
    assert _bf16(L, x=A + 1) == QG_ERR_MISALIGNED
    assert _bf16(L, w=B + 1) == QG_ERR_MISALIGNED
    assert _bf16(L, y=B + 2) == QG_ERR_ALIAS
    assert _bf16(L, yt=5) == QG_ERR_UNSUPPORTED
    assert _bf16(L, N=0) == QG_OK


def test_binding_raises_with_library_message():
    x = torch.zeros(9, 64, dtype=torch.float16)
    w = torch.zeros(4, 32, dtype=torch.uint8)
    s = torch.zeros(4, 2, dtype=torch.float16)
    y = torch.zeros(9, 4, dtype=torch.float16)
    with pytest.raises(q.QgemvError) as ei:
        q.qgemv_int4_blockwise(x, w, s, None, y, 32, stream=0)
    assert ei.value.status == QG_ERR_BAD_SHAPE
    assert "M = 9" in str(ei.value)
    with pytest.raises(q.QgemvError) as ei:
        q.qgemv_q4k_dsc(torch.zeros(1, 256), torch.zeros(4, 144, dtype=torch.uint8), None,
                        torch.zeros(1, 4), stream=0)
    assert ei.value.status == QG_ERR_NULL_POINTER


def test_binding_refuses_wrong_dtypes_before_the_call():
    w = torch.zeros(4, 144, dtype=torch.uint8)
    with pytest.raises(TypeError, match="x: expected torch.float32"):
        q.qgemv_q4k(torch.zeros(1, 256, dtype=torch.float16), w, torch.zeros(1, 4), stream=0)
    with pytest.raises(TypeError, match="w: expected torch.uint8"):
        q.qgemv_q4k(torch.zeros(1, 256), w.view(torch.int8), torch.zeros(1, 4), stream=0)
    with pytest.raises(TypeError, match="y: expected"):
        q.gemv_bf16(torch.zeros(1, 8, dtype=torch.bfloat16), torch.zeros(4, 8, dtype=torch.bfloat16),
                    torch.zeros(1, 4, dtype=torch.float64), stream=0)
    with pytest.raises(TypeError, match="scales: expected torch.float16"):
        q.qgemv_int4_blockwise(torch.zeros(1, 64, dtype=torch.float16), torch.zeros(4, 32, dtype=torch.uint8),
                               torch.zeros(4, 2), None, torch.zeros(1, 4, dtype=torch.float16), 32,
                               stream=0)


def test_product_package_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "weight_only_quantized_int4_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f


def test_liveness_exports_on_the_host():
    # host-only functions: no GPU needed
    names = q.path_names()
    assert len(names) == q.load_library().qg_path_count() == 19
    assert names[0] == "int4_dot2_persistent" and "q4k_persistent_plane" in names
    assert q.load_library().qg_path_name(-1) is None
    assert q.load_library().qg_path_name(len(names)) is None
    assert q.load_library().qg_path_launches(len(names)) == 0
    counts = q.path_launches()
    assert set(counts) == set(names) and all(v >= 0 for v in counts.values())
    assert isinstance(q.last_launch(), str)


def test_binding_refuses_mismatched_shapes_before_the_call():
    """Sizes come from x and w; every other tensor must match them, or the
    library would read or write past its end.  These raise before any call
    (host tensors, no GPU needed)."""
    f16, u8 = torch.float16, torch.uint8
    x = torch.zeros(1, 64, dtype=f16)
    w = torch.zeros(4, 32, dtype=u8)
    s = torch.zeros(4, 2, dtype=f16)
    zp = torch.zeros(4, 1, dtype=u8)
    y = torch.zeros(1, 4, dtype=f16)
    bad = {
        "y": dict(y=torch.zeros(4, 4, dtype=f16)),          # x [1,K] with y [4,N]
        "w": dict(w=torch.zeros(4, 16, dtype=u8)),
        "scales": dict(s=torch.zeros(4, 1, dtype=f16)),
        "zero_points": dict(zp=torch.zeros(4, 2, dtype=u8)),
    }
    for name, kw in bad.items():
        args = dict(x=x, w=w, s=s, zp=zp, y=y)
        args.update(kw)
        with pytest.raises(ValueError, match=name):
            q.qgemv_int4_blockwise(args["x"], args["w"], args["s"], args["zp"], args["y"], 32,
                                   stream=0)
    with pytest.raises(ValueError, match="contiguous"):
        q.qgemv_int4_blockwise(x, torch.zeros(32, 4, dtype=u8).t(), s, zp, y, 32, stream=0)
    # q4_K: y, w and the plane
    xq, wq = torch.zeros(2, 256), torch.zeros(4, 144, dtype=u8)
    with pytest.raises(ValueError, match="y"):
        q.qgemv_q4k(xq, wq, torch.zeros(1, 4), stream=0)
    with pytest.raises(ValueError, match="w"):
        q.qgemv_q4k(xq, torch.zeros(4, 288, dtype=u8), torch.zeros(2, 4), stream=0)
    with pytest.raises(ValueError, match="dsc"):
        q.qgemv_q4k_dsc(xq, wq, torch.zeros(8 * 4 - 1, 2), torch.zeros(2, 4), stream=0)
    with pytest.raises(ValueError, match="dsc_out"):
        q.q4k_build_dsc_plane(wq, torch.zeros(16, 2), 4, 256, stream=0)
    # bf16: w rows of another length
    with pytest.raises(ValueError, match="w"):
        q.gemv_bf16(torch.zeros(1, 8, dtype=torch.bfloat16), torch.zeros(4, 16, dtype=torch.bfloat16),
                    torch.zeros(1, 4, dtype=torch.bfloat16), stream=0)
    # prefill: codes, scales, y
    xt = torch.zeros(3, 256)
    with pytest.raises(ValueError, match="qa"):
        q.q8_quantize_rows(xt, torch.zeros(2, 256, dtype=torch.int8), torch.zeros(3, 8, 2), stream=0)
    with pytest.raises(ValueError, match="sda"):
        q.q8_quantize_rows(xt, torch.zeros(3, 256, dtype=torch.int8), torch.zeros(3, 4, 2), stream=0)
    with pytest.raises(ValueError, match="y"):
        q.qgemm_q4k_mmq(xt, wq, torch.zeros(32, 2), torch.zeros(3, 5), torch.zeros(4096, dtype=u8),
                        stream=0)


def test_noalloc_prefill_validation_on_the_host():
    """The allocation-free prefill entry point refuses, before touching the
    GPU, problems whose workspace exceeds its static array, and shares the
    other checks of qgemm_q4k_mmq."""
    L = q.load_library()
    text = open(HEADER).read()
    m = re.search(r"#define QG_MMQ_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == q.MMQ_NOALLOC_SCRATCH_BYTES

    def call(x=A, ldx=4096, w=B, dsc=C, y=E, ldy=16, T=4, N=16, K=4096):
        return L.qgemm_q4k_mmq_noalloc(x, ldx, w, dsc, y, ldy, T, N, K, None)

    # 8192 rows of 4096: 40 MiB of codes and scales > the 32 MiB array
    T_big = 8192
    assert q.q4k_mmq_workspace_bytes(T_big, 4096) > q.MMQ_NOALLOC_SCRATCH_BYTES
    assert call(T=T_big, ldy=16) == QG_ERR_UNSUPPORTED
    assert "static scratch" in L.qg_last_error().decode()
    assert call(dsc=None) == QG_ERR_NULL_POINTER
    assert call(K=300, ldx=300) == QG_ERR_BAD_SHAPE
    assert call(T=0) == QG_OK and call(N=0) == QG_OK

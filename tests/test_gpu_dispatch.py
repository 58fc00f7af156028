"""GPU behaviour of the dispatch layer and the liveness record (MI355X):
the registered q4_K plane is used and agrees bitwise with in-kernel decode, a
failed registration falls back with its label, qg_last_launch names the
kernels of the last call, the per-path counters move, row groups beyond 8
rows of x match the oracle, and the opt-in prefill arm gives the prefill
product's result."""
import warnings

import numpy as np
import pytest
import torch

import datagen
import oracle
import weight_only_quantized_int4_amd as q
from weight_only_quantized_int4_amd import dispatch
from gpu_cases import (DEV, assert_accept, bf16_case, bf16_dev, f16_dev, int4_case, int4_ref,
                       q4k_case, q4k_ref, say, to_dev, y_host)

pytestmark = pytest.mark.gpu


def test_q4k_plane_registry_and_liveness():
    N, K = 512, 1024
    p = q4k_case(N, K, 430)
    wd = to_dev(p.w)
    x = to_dev(p.x[:3])
    say("dispatch q4k plane registry")
    dispatch.reset_liveness()
    before = q.path_launches()
    _, label = dispatch.q4k_linear(x, wd)
    assert label == dispatch.LABEL_OFF
    assert q.last_launch().startswith("q4k_persistent M=3")
    assert dispatch.register_q4k_plane(wd)
    assert q.last_launch().startswith("q4k_plane_build")
    y_plane, label = dispatch.q4k_linear(x, wd)
    assert label == dispatch.LABEL_PLANE
    assert dispatch.explain().startswith("q4k_persistent_plane M=3")
    y_direct, label = dispatch.q4k_linear(x, wd, use_plane=False)
    assert label == dispatch.LABEL_OFF
    torch.cuda.synchronize()
    assert torch.equal(y_plane, y_direct)
    after = q.path_launches()
    assert after["q4k_persistent"] - before["q4k_persistent"] == 2
    assert after["q4k_persistent_plane"] - before["q4k_persistent_plane"] == 1
    assert after["q4k_plane_build"] - before["q4k_plane_build"] == 1
    yr, S = q4k_ref(N, K, 430)
    assert_accept(y_host(y_plane), yr[:3], S[:3], "f32", "dispatch q4k plane")
    assert dispatch.liveness() == {dispatch.LABEL_PLANE: 1, dispatch.LABEL_OFF: 2,
                                   dispatch.LABEL_FALLBACK: 0, dispatch.LABEL_MMQ: 0}
    dispatch.unregister_q4k_plane(wd)


def test_q4k_failed_registration_falls_back(monkeypatch):
    N, K = 256, 512
    p = q4k_case(N, K, 431)
    wd = to_dev(p.w)
    say("dispatch q4k fallback")
    dispatch.reset_liveness()

    # a plane that cannot be built (as when its allocation fails)
    def failing_build(w, dsc, N, K, stream=None):
        raise q.QgemvError("q4k_build_dsc_plane", 6, "QG_ERR_HIP", "simulated failure")

    monkeypatch.setattr(q.qgemv, "q4k_build_dsc_plane", failing_build)
    assert not dispatch.register_q4k_plane(wd)
    with warnings.catch_warnings(record=True) as got:
        warnings.simplefilter("always")
        y, label = dispatch.q4k_linear(to_dev(p.x[:1]), wd)
    assert label == dispatch.LABEL_FALLBACK
    assert dispatch.explain().startswith("q4k_persistent M=1")
    assert any(issubclass(g.category, RuntimeWarning) for g in got)
    yr, S = q4k_ref(N, K, 431)
    assert_accept(y_host(y), yr[:1], S[:1], "f32", "dispatch q4k fallback")
    dispatch.unregister_q4k_plane(wd)


def test_explain_names_each_path():
    say("dispatch explain strings")
    p = int4_case(4096, 1024, 32, True, 432)
    wd, sd, zd = to_dev(p.w), f16_dev(p.scales), to_dev(p.zp)
    y = torch.empty((8, 4096), dtype=torch.float16, device=DEV)
    q.qgemv_int4_blockwise(f16_dev(p.x[:1]), wd, sd, zd, y[:1], 32)
    assert q.last_launch().startswith("int4_dot2_persistent M=1 ")
    q.qgemv_int4_blockwise(f16_dev(p.x[:4]), wd, sd, zd, y[:4], 32)
    assert q.last_launch().startswith("int4_mfma_")
    b = bf16_case(256, 1536, 433)
    yb = torch.empty((3, 256), dtype=torch.bfloat16, device=DEV)
    q.gemv_bf16(bf16_dev(b.x[:3]), bf16_dev(b.w), yb)
    assert q.last_launch().startswith("bf16_mfma_")
    b2 = bf16_case(256, 100, 434)
    q.gemv_bf16(bf16_dev(b2.x[:3]), bf16_dev(b2.w), yb)
    assert q.last_launch().startswith("bf16_general M=3 ")
    # a call that enqueues nothing (N = 0) leaves an empty record
    xb2, wb2 = bf16_dev(b2.x[:3]), bf16_dev(b2.w)
    L = q.load_library()
    assert L.gemv_bf16(xb2.data_ptr(), 100, wb2.data_ptr(), 100, yb.data_ptr(), 256, 1, 3, 0, 100,
                       torch.cuda.current_stream().cuda_stream) == 0
    assert q.last_launch() == ""
    # q4_K rows of x beyond what LDS holds: one launch per row group
    qp = q4k_case(300, 11008, 421)
    yq = torch.empty((8, 300), device=DEV)
    q.qgemv_q4k(to_dev(qp.x[:8]), to_dev(qp.w), yq)
    launches = q.last_launch().split("; ")
    assert [l.split()[:2] for l in launches] == [["q4k_persistent", "M=3"],
                                                 ["q4k_persistent", "M=3"],
                                                 ["q4k_persistent", "M=2"]]
    torch.cuda.synchronize()


@pytest.mark.parametrize("M", [9, 13])
def test_row_groups_match_the_oracle(M):
    say(f"dispatch row groups M={M}")
    p = int4_case(1536, 1536, 128, False, 201)
    # x with more than 8 rows: reuse the 8 seeded rows, negated for rows 8..
    xr = np.concatenate([p.x, p.x ^ np.uint16(0x8000)])[:M]
    y = dispatch.int4_linear(f16_dev(xr), to_dev(p.w), f16_dev(p.scales), None, 128,
                             torch.empty((M, 1536), dtype=torch.float32, device=DEV))
    yr, S = int4_ref(1536, 1536, 128, False, 201)
    yref = np.concatenate([yr, -yr])[:M]
    Sref = np.concatenate([S, S])[:M]
    assert_accept(y_host(y), yref, Sref, "f32", f"int4 row groups M={M}")
    b = bf16_case(1536, 1536, 301)
    xb = np.concatenate([b.x, b.x ^ np.uint16(0x8000)])[:M]
    yb = dispatch.bf16_linear(bf16_dev(xb), bf16_dev(b.w),
                              torch.empty((M, 1536), dtype=torch.float32, device=DEV))
    ybr, Sb = oracle.bf16_gemv(np.ascontiguousarray(xb), b.w, M, 1536, 1536, 1536, 1536)
    assert_accept(y_host(yb), ybr, Sb, "f32", f"bf16 row groups M={M}")


def test_prefill_arm_is_the_prefill_product():
    N, K, T = 300, 1024, 40
    p = q4k_case(N, K, 435)
    wd = to_dev(p.w)
    x = to_dev(datagen.prefill_x(T, K, 436))
    say(f"dispatch q4k prefill arm T={T} N={N} K={K}")
    dispatch.reset_liveness()
    assert dispatch.register_q4k_plane(wd)
    y_rows, label = dispatch.q4k_linear(x, wd)  # default: no prefill arm
    assert label == dispatch.LABEL_PLANE
    y_mmq, label = dispatch.q4k_linear(x, wd, prefill_min_rows=32)
    assert label == dispatch.LABEL_MMQ
    launches = q.last_launch()
    assert "q8_quantize" in launches and "q4k_mmq" in launches
    ws = torch.empty(q.q4k_mmq_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    y_direct = q.qgemm_q4k_mmq(x, wd, dispatch.q4k_plane_of(wd), torch.empty((T, N), device=DEV), ws)
    torch.cuda.synchronize()
    assert torch.equal(y_mmq, y_direct)
    _, label = dispatch.q4k_linear(x[:20], wd, prefill_min_rows=32)  # fewer rows: row groups
    assert label == dispatch.LABEL_PLANE
    assert dispatch.liveness()[dispatch.LABEL_MMQ] == 1
    yr, S = oracle.q4k_mmq(datagen.prefill_x(T, K, 436), p.w, T, N, K)
    ok, worst = oracle.accept(y_host(y_mmq), yr, S, "f32", rtol=oracle.RTOL_MMQ)
    assert ok, worst
    # the default (row groups) is the GEMV, within the GEMV tolerance
    yg, Sg = oracle.q4k_gemv(datagen.prefill_x(T, K, 436), p.w, T, N, K)
    assert_accept(y_host(y_rows), yg, Sg, "f32", "dispatch q4k rows T=40")
    dispatch.unregister_q4k_plane(wd)


def test_int4_packed_copy_serves_tall_matrices():
    """A registered packed copy of a matrix of more 16-row tiles than CUs
    serves the row groups of >= 2 rows (8 + 3 here) and the single row stays on
    the original layout; all within the bound of the oracle.  A short matrix
    keeps the original layout although its copy is registered."""
    N, K, bs = 4100, 1024, 64
    say("dispatch int4 packed copy")
    p = int4_case(N, K, bs, True, 433)
    wd, sd, zd = to_dev(p.w), f16_dev(p.scales), to_dev(p.zp)
    assert dispatch.register_int4_packed(wd, sd, zd, bs)
    assert dispatch.int4_packed_of(wd, bs) is not None
    dispatch.reset_liveness()
    M = 11
    xr = np.concatenate([p.x, p.x ^ np.uint16(0x8000)])[:M]
    y = dispatch.int4_linear(f16_dev(xr), wd, sd, zd, bs,
                             torch.empty((M, N), dtype=torch.float32, device=DEV))
    assert dispatch.explain().startswith("int4_packed M=3"), dispatch.explain()
    y1 = dispatch.int4_linear(f16_dev(p.x[:1]), wd, sd, zd, bs,
                              torch.empty((1, N), dtype=torch.float32, device=DEV))
    assert dispatch.explain().startswith("int4_span M=1") or \
        dispatch.explain().startswith("int4_dot2"), dispatch.explain()
    assert dispatch.int4_liveness() == {dispatch.LABEL_INT4: 1, dispatch.LABEL_INT4_PACKED: 2}
    yr, S = int4_ref(N, K, bs, True, 433)
    yref = np.concatenate([yr, -yr])[:M]
    Sref = np.concatenate([S, S])[:M]
    assert_accept(y_host(y), yref, Sref, "f32", "int4 packed copy M=11")
    assert_accept(y_host(y1), yr[:1], S[:1], "f32", "int4 packed copy M=1")
    # short matrix: the original layout's k-part kernel
    ps = int4_case(1536, 1536, 128, False, 201)
    ws, ss = to_dev(ps.w), f16_dev(ps.scales)
    assert dispatch.register_int4_packed(ws, ss, None, 128)
    dispatch.int4_linear(f16_dev(ps.x[:4]), ws, ss, None, 128,
                         torch.empty((4, 1536), dtype=torch.float32, device=DEV))
    assert dispatch.explain().startswith("int4_mfma_split M=4"), dispatch.explain()
    dispatch.unregister_int4_packed(wd, bs)
    dispatch.unregister_int4_packed(ws, 128)
    assert dispatch.int4_packed_of(wd, bs) is None

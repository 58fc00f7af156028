"""Host-side logic of the dispatch layer (no GPU): plane registry, liveness
labels, the once-per-process fallback warning, the QGEMV_Q4K_DSC switch and
row groups.  The C-ABI calls are replaced by recorders; the GPU behaviour is
covered by tests/test_gpu_dispatch.py."""
import warnings

import pytest
import torch

from weight_only_quantized_int4_amd import dispatch, qgemv


@pytest.fixture
def fake_abi(monkeypatch):
    calls = []

    def q4k(x, w, y, stream=None):
        calls.append(("q4k", x.shape[0]))
        return y

    def q4k_dsc(x, w, dsc, y, stream=None):
        assert dsc is not None
        calls.append(("q4k_dsc", x.shape[0]))
        return y

    def build(w, dsc, N, K, stream=None):
        calls.append(("build", N, K))
        return dsc

    def int4(x, w, s, z, y, bs, stream=None):
        calls.append(("int4", x.shape[0], y.shape[0]))
        return y

    def bf16(x, w, y, stream=None):
        calls.append(("bf16", x.shape[0], y.shape[0]))
        return y

    monkeypatch.setattr(qgemv, "qgemv_q4k", q4k)
    monkeypatch.setattr(qgemv, "qgemv_q4k_dsc", q4k_dsc)
    monkeypatch.setattr(qgemv, "q4k_build_dsc_plane", build)
    monkeypatch.setattr(qgemv, "q4k_dsc_plane_bytes", lambda N, K: N * K // 4)
    monkeypatch.setattr(qgemv, "qgemv_int4_blockwise", int4)
    monkeypatch.setattr(qgemv, "gemv_bf16", bf16)

    def mmq(x, w, dsc, y, workspace, stream=None):
        assert dsc is not None and workspace.numel() >= x.shape[0] * 10
        calls.append(("mmq", x.shape[0], workspace.numel()))
        return y

    monkeypatch.setattr(qgemv, "qgemm_q4k_mmq", mmq)
    monkeypatch.setattr(qgemv, "q4k_mmq_workspace_bytes", lambda T, K: T * 10)
    monkeypatch.setattr(qgemv, "_stream", lambda stream: 0 if stream is None else int(stream))
    monkeypatch.delenv("QGEMV_Q4K_DSC", raising=False)
    monkeypatch.delenv("QGEMV_Q4K_MMQ_MIN_ROWS", raising=False)
    dispatch.reset_liveness()
    yield calls
    dispatch.reset_liveness()


def _q4k_weights(N=16, K=512):
    return torch.zeros((N, K // 256 * 144), dtype=torch.uint8)


def test_plane_label_and_row_groups(fake_abi):
    w = _q4k_weights()
    assert dispatch.register_q4k_plane(w)
    assert fake_abi[-1] == ("build", 16, 512)
    assert dispatch.q4k_plane_of(w).shape == (16 * 512 // 4 // 8, 2)
    x = torch.zeros((19, 512))
    y, label = dispatch.q4k_linear(x, w)
    assert label == dispatch.LABEL_PLANE and y.shape == (19, 16)
    assert fake_abi[-3:] == [("q4k_dsc", 8), ("q4k_dsc", 8), ("q4k_dsc", 3)]
    assert dispatch.liveness()[dispatch.LABEL_PLANE] == 1
    dispatch.unregister_q4k_plane(w)
    _, label = dispatch.q4k_linear(x[:1], w)
    assert label == dispatch.LABEL_OFF and fake_abi[-1] == ("q4k", 1)


def test_switched_off_plane(fake_abi, monkeypatch):
    w = _q4k_weights()
    assert dispatch.register_q4k_plane(w)
    monkeypatch.setenv("QGEMV_Q4K_DSC", "0")
    _, label = dispatch.q4k_linear(torch.zeros((2, 512)), w)
    assert label == dispatch.LABEL_OFF and fake_abi[-1] == ("q4k", 2)
    monkeypatch.delenv("QGEMV_Q4K_DSC")
    _, label = dispatch.q4k_linear(torch.zeros((2, 512)), w, use_plane=False)
    assert label == dispatch.LABEL_OFF
    _, label = dispatch.q4k_linear(torch.zeros((2, 512)), w)
    assert label == dispatch.LABEL_PLANE


def test_failed_registration_falls_back_loudly_once(fake_abi, monkeypatch):
    w = _q4k_weights()

    def failing_build(w, dsc, N, K, stream=None):
        raise qgemv.QgemvError("q4k_build_dsc_plane", 6, "QG_ERR_HIP", "simulated")

    monkeypatch.setattr(qgemv, "q4k_build_dsc_plane", failing_build)
    assert not dispatch.register_q4k_plane(w)
    assert dispatch.q4k_plane_of(w) is None
    x = torch.zeros((1, 512))
    with warnings.catch_warnings(record=True) as got:
        warnings.simplefilter("always")
        _, l1 = dispatch.q4k_linear(x, w)
        _, l2 = dispatch.q4k_linear(x, w)
    assert l1 == l2 == dispatch.LABEL_FALLBACK
    assert len([g for g in got if issubclass(g.category, RuntimeWarning)]) == 1
    assert dispatch.liveness()[dispatch.LABEL_FALLBACK] == 2
    assert fake_abi[-2:] == [("q4k", 1), ("q4k", 1)]


def test_bad_weight_shape_is_a_failed_registration(fake_abi):
    w = torch.zeros((4, 100), dtype=torch.uint8)  # not a multiple of 144 bytes per row
    assert not dispatch.register_q4k_plane(w)


@pytest.mark.parametrize("M,groups", [(1, [1]), (8, [8]), (9, [8, 1]), (20, [8, 8, 4])])
def test_int4_and_bf16_row_groups(fake_abi, M, groups):
    x = torch.zeros((M, 64), dtype=torch.float16)
    w = torch.zeros((32, 32), dtype=torch.uint8)
    y = dispatch.int4_linear(x, w, torch.zeros((32, 2), dtype=torch.float16), None, 32)
    assert y.shape == (M, 32) and y.dtype == torch.float16
    assert [c[1] for c in fake_abi if c[0] == "int4"] == groups
    assert all(c[1] == c[2] for c in fake_abi if c[0] == "int4")
    xb = torch.zeros((M, 64), dtype=torch.bfloat16)
    yb = dispatch.bf16_linear(xb, torch.zeros((32, 64), dtype=torch.bfloat16))
    assert yb.shape == (M, 32) and yb.dtype == torch.bfloat16
    assert [c[1] for c in fake_abi if c[0] == "bf16"] == groups


def test_prefill_arm_is_opt_in(fake_abi, monkeypatch):
    w = _q4k_weights()
    x = torch.zeros((40, 512))
    # without a plane the arm is never taken
    _, label = dispatch.q4k_linear(x, w, prefill_min_rows=32)
    assert label == dispatch.LABEL_OFF and fake_abi[-1] == ("q4k", 8)
    assert dispatch.register_q4k_plane(w)
    _, label = dispatch.q4k_linear(x, w)  # default: off
    assert label == dispatch.LABEL_PLANE and fake_abi[-1] == ("q4k_dsc", 8)
    monkeypatch.setenv("QGEMV_Q4K_MMQ_MIN_ROWS", "32")
    _, label = dispatch.q4k_linear(x, w)
    assert label == dispatch.LABEL_MMQ and fake_abi[-1] == ("mmq", 40, 400)
    _, label = dispatch.q4k_linear(x[:31], w)  # below the threshold: row groups
    assert label == dispatch.LABEL_PLANE
    _, label = dispatch.q4k_linear(x, w, prefill_min_rows=0)  # the argument wins
    assert label == dispatch.LABEL_PLANE
    _, label = dispatch.q4k_linear(x, w, use_plane=False)  # no plane, no arm
    assert label == dispatch.LABEL_OFF
    assert dispatch.liveness()[dispatch.LABEL_MMQ] == 1
    monkeypatch.setenv("QGEMV_Q4K_MMQ_MIN_ROWS", "many")
    with pytest.raises(ValueError):
        dispatch.q4k_linear(x, w)
    dispatch.unregister_q4k_plane(w)


def test_prefill_workspace_grows_per_stream(fake_abi):
    w = _q4k_weights()
    assert dispatch.register_q4k_plane(w)
    dispatch.q4k_linear(torch.zeros((40, 512)), w, prefill_min_rows=16)
    ws40 = dispatch._workspaces[(None, 0)]
    dispatch.q4k_linear(torch.zeros((20, 512)), w, prefill_min_rows=16)
    assert dispatch._workspaces[(None, 0)] is ws40  # large enough: reused
    dispatch.q4k_linear(torch.zeros((64, 512)), w, prefill_min_rows=16)
    assert dispatch._workspaces[(None, 0)].numel() == 640  # grown
    dispatch.q4k_linear(torch.zeros((16, 512)), w, prefill_min_rows=16, stream=7)
    assert dispatch._workspaces[(None, 7)].numel() == 160  # its own stream, its own buffer
    assert [c[2] for c in fake_abi if c[0] == "mmq"] == [400, 400, 640, 160]
    dispatch._workspaces.clear()
    dispatch.unregister_q4k_plane(w)


def test_plane_entry_is_keyed_on_shape_and_dropped_with_the_weight(fake_abi):
    import gc

    w = _q4k_weights(16, 512)
    assert dispatch.register_q4k_plane(w)
    # another view of the same bytes with another shape finds no plane
    w2 = w.view(32, 144)
    assert dispatch.q4k_plane_of(w2) is None
    _, label = dispatch.q4k_linear(torch.zeros((1, 256)), w2)
    assert label == dispatch.LABEL_OFF
    key = (w.data_ptr(), 16, 512)
    del w2
    del w
    gc.collect()
    # the weight is gone: a tensor that later reuses its address must not meet
    # the old plane
    assert key not in dispatch._planes and key not in dispatch._failed


def test_failed_registration_is_dropped_with_the_weight(fake_abi, monkeypatch):
    import gc

    def failing_build(w, dsc, N, K, stream=None):
        raise qgemv.QgemvError("q4k_build_dsc_plane", 6, "QG_ERR_HIP", "simulated")

    monkeypatch.setattr(qgemv, "q4k_build_dsc_plane", failing_build)
    w = _q4k_weights(8, 256)
    key = (w.data_ptr(), 8, 256)
    assert not dispatch.register_q4k_plane(w)
    assert key in dispatch._failed
    del w
    gc.collect()
    assert key not in dispatch._failed


def test_int4_packed_copy_choice_and_lifetime(fake_abi, monkeypatch):
    """A registered packed copy serves row groups of >= 2 rows of x on
    matrices of at least as many 16-row tiles as CUs; single rows, short
    matrices and unregistered weights keep the original layout.  The entry
    is dropped with the weight tensor."""
    import gc

    def repack(w, s, z, packed, bs, layout=1, stream=None):
        fake_abi.append(("repack", w.shape[0], bs))
        return packed

    def packed_gemv(x, packed, y, bs, layout=1, stream=None):
        fake_abi.append(("packed", x.shape[0], y.shape[0]))
        return y

    monkeypatch.setattr(qgemv, "int4_packed_bytes", lambda N, K, bs, layout=1: 0 if K % 128 else N * K)
    monkeypatch.setattr(qgemv, "int4_repack", repack)
    monkeypatch.setattr(qgemv, "qgemv_int4_packed", packed_gemv)
    monkeypatch.setattr(dispatch, "_compute_units", lambda device: 4)
    tall = torch.zeros((64, 128), dtype=torch.uint8)   # 4 tiles of 16 rows = the 4 CUs
    short = torch.zeros((48, 128), dtype=torch.uint8)  # 3 tiles
    s = torch.zeros((64, 8), dtype=torch.float16)
    assert dispatch.register_int4_packed(tall, s, None, 32)
    assert dispatch.register_int4_packed(short, s[:48], None, 32)
    assert not dispatch.register_int4_packed(torch.zeros((64, 100), dtype=torch.uint8), s, None, 40)
    assert fake_abi == [("repack", 64, 32), ("repack", 48, 32)]
    del fake_abi[:]
    x = torch.zeros((11, 256), dtype=torch.float16)
    dispatch.int4_linear(x, tall, s, None, 32)          # groups of 8 and 3 rows
    dispatch.int4_linear(x[:1], tall, s, None, 32)      # one row: original layout
    dispatch.int4_linear(x[:9], tall, s, None, 32)      # 8 + 1
    dispatch.int4_linear(x[:3], short, s[:48], None, 32)  # short matrix
    dispatch.int4_linear(x[:3], tall, s, None, 64)      # no copy for this block size
    assert fake_abi == [("packed", 8, 8), ("packed", 3, 3), ("int4", 1, 1), ("packed", 8, 8),
                        ("int4", 1, 1), ("int4", 3, 3), ("int4", 3, 3)]
    assert dispatch.int4_liveness() == {dispatch.LABEL_INT4: 4, dispatch.LABEL_INT4_PACKED: 3}
    key = dispatch._int4_key(tall, 32)
    assert dispatch.int4_packed_of(tall, 32) is not None
    dispatch.unregister_int4_packed(short, 32)
    assert dispatch.int4_packed_of(short, 32) is None
    del tall
    gc.collect()
    assert key not in dispatch._packed

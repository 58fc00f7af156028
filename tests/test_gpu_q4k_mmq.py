"""GPU parity of the q4_K prefill product (q8_quantize_rows, qgemm_q4k_mmq).

The 8-bit activation prepass is compared bit for bit with the oracle's codes
and scales (the codes are integers decided by a binary32 quotient on both
sides).  The product is compared with the oracle's exact value of
sum_c d_a * (dv * sum q_w q_a + mv * sum q_a) within RTOL_MMQ * S + 1 ulp
(the oracle derives RTOL_MMQ from the fp32 steps of the rescale), on full
small shapes (several tiles and ragged edges in both T and N) and on sampled
columns of the 7B layer shapes at prompt lengths 512 and 200; integer-valued
inputs must come out exactly.
"""
import numpy as np
import pytest
import torch

import datagen
import oracle
import weight_only_quantized_int4_amd as q
from gpu_cases import DEV, q4k_case, say, to_dev, y_host

pytestmark = pytest.mark.gpu


def _plane(wd, N, K):
    dsc = torch.empty((q.q4k_dsc_plane_bytes(N, K) // 8, 2), dtype=torch.float32, device=DEV)
    q.q4k_build_dsc_plane(wd, dsc, N, K)
    return dsc


def _mmq(x, w, N, K, ldy=None, xd=None):
    T = x.shape[0]
    wd = to_dev(w)
    dsc = _plane(wd, N, K)
    xd = to_dev(x) if xd is None else xd
    ws = torch.empty(q.q4k_mmq_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    ybuf = torch.full((T, N if ldy is None else ldy), float("nan"), dtype=torch.float32, device=DEV)
    y = ybuf[:, :N]
    q.qgemm_q4k_mmq(xd, wd, dsc, y, ws)
    return y_host(y), y_host(ybuf)


def _accept(y, yr, S, what):
    ok, worst = oracle.accept(y, yr, S, "f32", rtol=oracle.RTOL_MMQ)
    assert ok, f"{what}: max |err|/(RTOL_MMQ*S+ulp) = {worst:.3g}"


@pytest.mark.parametrize("T,K,ldx,offset", [(1, 256, 256, 0), (37, 512, 512, 0), (300, 4096, 4096, 0),
                                            (5, 1024, 1030, 1)])
def test_prepass_bit_exact(T, K, ldx, offset):
    x = datagen.prefill_x(T, K, 900 + T)
    say(f"q8 prepass T={T} K={K} ldx={ldx} offset={offset}")
    buf = np.zeros(offset + T * ldx, dtype=np.float32)
    for t in range(T):
        buf[offset + t * ldx:offset + t * ldx + K] = x[t]
    xd = to_dev(buf)[offset:].as_strided((T, K), (ldx, 1)) if offset or ldx != K else to_dev(x)
    qa = torch.empty((T, K), dtype=torch.int8, device=DEV)
    sda = torch.empty((T, K // 32, 2), dtype=torch.float32, device=DEV)
    q.q8_quantize_rows(xd, qa, sda)
    torch.cuda.synchronize()
    want_q, want_d = oracle.q8_quantize(x, T, K)
    got_q, got = qa.cpu().numpy(), sda.cpu().numpy()
    assert np.array_equal(got_q, want_q)
    assert np.array_equal(got[..., 0].view(np.uint32), want_d.view(np.uint32))
    sums = want_q.reshape(T, K // 32, 32).astype(np.int64).sum(axis=2).astype(np.float32)
    assert np.array_equal(got[..., 1].view(np.uint32), (want_d * sums).astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("T,N,K", [(1, 64, 256), (37, 300, 512), (130, 1000, 1024), (64, 129, 2048),
                                   (257, 256, 256), (1, 1, 256), (65, 1, 512), (2048, 130, 256)])
def test_full_shapes(T, N, K):
    p = q4k_case(N, K, 910 + N)
    x = datagen.prefill_x(T, K, 911 + T)
    say(f"q4k mmq full T={T} N={N} K={K}")
    y, _ = _mmq(x, p.w, N, K)
    assert "q8_quantize" in q.last_launch() and "q4k_mmq" in q.last_launch()
    yr, S = oracle.q4k_mmq(x, p.w, T, N, K)
    _accept(y, yr, S, f"mmq {T}x{N}x{K}")


@pytest.mark.parametrize("T,N,K", [(512, 4096, 4096), (512, 11008, 4096), (200, 4096, 11008)])
def test_layer_shapes_sampled(T, N, K):
    p = q4k_case(N, K, 920 + K)
    x = datagen.prefill_x(T, K, 921)
    say(f"q4k mmq layer T={T} N={N} K={K}")
    y, _ = _mmq(x, p.w, N, K)
    cols = sorted(set(np.random.default_rng(7).integers(0, N, 40).tolist()) | {0, 127, 128, N - 1})
    yr, S = oracle.q4k_mmq(x, p.w, T, N, K, cols=cols)
    _accept(y[:, cols], yr, S, f"mmq layer {T}x{N}x{K}")


def test_integer_inputs_are_exact():
    """d = dmin = 1 and activation blocks with amax 127 (d_a = 1): every term is
    an integer below 2^24, so the fp32 result is the exact integer matmul."""
    rng = np.random.default_rng(77)
    N, K, T = 200, 512, 70
    nsb = K // 256
    blocks = []
    for _ in range(N * nsb):
        blocks.append(datagen.q4k_header(0x3C00, 0x3C00, rng.integers(0, 256, 12, dtype=np.uint8).tobytes(),
                                         rng.integers(0, 256, 128, dtype=np.uint8).tobytes()))
    w = np.frombuffer(b"".join(blocks), dtype=np.uint8).reshape(N, nsb * 144).copy()
    x_int = rng.integers(-127, 128, (T, K))
    x_int.reshape(T, K // 32, 32)[:, :, 3] = 127 * rng.choice([-1, 1], (T, K // 32))
    x = x_int.astype(np.float32)
    say(f"q4k mmq integer T={T} N={N} K={K}")
    y, _ = _mmq(x, w, N, K)
    yr, _ = oracle.q4k_mmq(x, w, T, N, K)
    assert np.all(np.abs(yr) < 2 ** 24)
    assert np.array_equal(y, yr)


def test_strided_x_and_y():
    N, K, T = 300, 512, 45
    p = q4k_case(N, K, 930)
    x = datagen.prefill_x(T, K, 931)
    ldx = K + 4
    buf = torch.zeros((T, ldx), dtype=torch.float32, device=DEV)
    buf[:, :K] = torch.from_numpy(x).to(DEV)
    say(f"q4k mmq strided T={T} N={N} K={K} ldx={ldx} ldy={N + 20}")
    y, ybuf = _mmq(x, p.w, N, K, ldy=N + 20, xd=buf[:, :K])
    yr, S = oracle.q4k_mmq(x, p.w, T, N, K)
    _accept(y, yr, S, "mmq strided")
    assert np.all(np.isnan(ybuf[:, N:]))  # padding of y untouched


def test_rejected_calls_on_device():
    N, K, T = 64, 256, 4
    p = q4k_case(N, K, 940)
    wd = to_dev(p.w)
    xd = to_dev(datagen.prefill_x(T, K, 941))
    y = torch.empty((T, N), device=DEV)
    ws = torch.empty(q.q4k_mmq_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    with pytest.raises(q.QgemvError) as e:
        q.qgemm_q4k_mmq(xd, wd, None, y, ws)
    assert e.value.status_name == "QG_ERR_NULL_POINTER"
    with pytest.raises(q.QgemvError) as e:
        q.qgemm_q4k_mmq(xd, wd, _plane(wd, N, K), y, ws[:100])
    assert e.value.status_name == "QG_ERR_BAD_SHAPE"

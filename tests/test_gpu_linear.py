"""GPU parity of linear_fp8_dynamic, per-token quantization followed by the
scaled FP8 GEMM in one call ("FP8 dynamic quantization" of "Helion in vLLM:
A Unified Route to Tunable Linear Kernels", "What the integration changes").

Bars: the codes and scales it returns are bit-exact to the oracle's
quantizer; its output is bitwise the output of the two separate calls
(quantize_per_token_fp8 then gemm_fp8_scaled with the same configuration)
and within the floating-point rule of tests/gpu_util.py of the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import check_fp, dev_bf16, dev_e4m3, dev, host_codes, host_f64  # noqa: E402


@pytest.fixture(scope="module")
def qll():
    import quantized_linear_layer_scaled_amd as q
    q.load_library()
    q.init()
    return q


@pytest.mark.parametrize("N,K", [(4096, 2048), (2048, 6144), (520, 1040)])
def test_linear_equals_two_calls_and_oracle(qll, N, K):
    w = workloads.weights_bf16(N, K, key=(workloads.W_TEST, 40))
    B, sb = oracle.quantize_fp8(w)
    dB, dsb = dev_e4m3(B), dev(sb[:, 0].copy())
    x_all = workloads.fp8_activations(64, K, key=(workloads.W_TEST, 41))
    for M in (1, 5, 16, 17, 33, 64):
        x = x_all[:M].copy()
        qr, sr = oracle.quantize_fp8(x)
        ref, absref = oracle.gemm_fp8(qr, B, sr[:, 0].copy(), sb[:, 0].copy(), with_abs=True)
        dx = dev_bf16(x)
        for cfg in (None, ("k16x16_w8", 1), ("k16x16_w16", 1), ("k16x32_w8", 1),
                    ("k16x64_w8", 1), ("k16x16_w8", 2), ("p64x128_w2x2_k128_s4", 1)):
            for od in ("bf16", "fp32"):
                y, q, sa = qll.linear_fp8_dynamic(dx, dB, dsb, out_dtype=od, cfg=cfg)
                q2, sa2 = qll.quantize_per_token_fp8(dx)
                y2 = qll.gemm_fp8_scaled(q2, dB, sa2, dsb, out_dtype=od, cfg=cfg)
                torch.cuda.synchronize()
                assert np.array_equal(host_codes(q), qr), (M, cfg)
                assert np.array_equal(sa.cpu().numpy().view(np.uint32), sr.view(np.uint32))
                iv = torch.int16 if od == "bf16" else torch.int32
                assert torch.equal(y.view(iv), y2.view(iv)), (M, cfg, od)
                check_fp(host_f64(y), ref, absref, K, od, f"linear {cfg} M={M} {od}")


def test_linear_large_m_sampled(qll):
    N, K = 4096, 2048
    w = workloads.weights_bf16(N, K, key=(workloads.W_TEST, 42))
    B, sb = oracle.quantize_fp8(w)
    x = workloads.fp8_activations(512, K, key=(workloads.W_TEST, 43))
    qr, sr = oracle.quantize_fp8(x)
    rows = [0, 200, 511]
    ref, absref = oracle.gemm_fp8(qr, B, sr[:, 0].copy(), sb[:, 0].copy(), rows=rows,
                                  with_abs=True)
    y, q, sa = qll.linear_fp8_dynamic(dev_bf16(x), dev_e4m3(B), dev(sb[:, 0].copy()))
    torch.cuda.synchronize()
    assert np.array_equal(host_codes(q), qr)
    check_fp(host_f64(y)[rows], ref, absref, K, "bf16", "linear M=512")


"""GPU parity of the INT4 weight-only (W4A16) quantizer and GEMM against the
oracle.

INT4 is among the formats "Helion in vLLM: A Unified Route to Tunable Linear
Kernels" lists for vLLM (introduction); the symmetric per-group reading is
stated in the oracle.

Bars: codes and scales bit-exact (the quantizer's integer decision is taken
on the same correctly rounded fp32 quotient on both sides); GEMM outputs
within the rule of tests/gpu_util.py (per-group promotion: K/128 extra
roundings, covered by its K/128 term), and bit-exact when every partial sum
is an exactly representable integer (unit scales, integer activations);
every variant, with and without Split-K, on shapes with ragged M, N and K
tails; the sweep shapes at full size on sampled rows through the shipped
dispatch.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import check_fp, dev, dev_bf16, host_f64, sample_rows  # noqa: E402


@pytest.fixture(scope="module")
def qll():
    import quantized_linear_layer_scaled_amd as q
    q.load_library()
    q.init()
    return q


def names(qll):
    return [v["name"] for v in qll.variants("w4a16")]


def corner_rows(K):
    """bf16 weight rows that hit the rule's corner cases."""
    rows = []
    t = 2.0 ** -3
    r = np.zeros(K, np.float32)     # exact halves after division by s = 2^-3
    vals = [7, 0.5, 1.5, 2.5, 3.5, 6.5, -0.5, -1.5, -2.5, -6.5, -7, 0.25, 0.75]
    r[:len(vals)] = np.array(vals, np.float32) * np.float32(t)
    rows.append(r)
    r = np.zeros(K, np.float32)     # an all-zero group (and negative zeros)
    r[3] = -0.0
    rows.append(r)
    r = np.full(K, 2.0 ** -130, np.float32)   # subnormal bf16 group
    r[1] = -(2.0 ** -128)
    rows.append(r)
    r = np.ones(K, np.float32)      # near the bf16 maximum
    r[0] = 3.3895313892515355e38
    r[2] = -1.0e38
    rows.append(r)
    return workloads.to_bf16_bits(np.stack(rows))


@pytest.mark.parametrize("N,K", [(1, 128), (3, 256), (64, 2048), (300, 1152), (2048, 6144)])
def test_quantizer_bit_exact(qll, N, K):
    w = workloads.w4_weights(N, K, key=(workloads.W_TEST, 80, N, K))
    q_ref, s_ref = oracle.quantize_int4(w)
    q, s = qll.quantize_int4_weights(dev_bf16(w))
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "scales"
    assert np.array_equal(q.cpu().numpy(), q_ref), "codes"


@pytest.mark.parametrize("K", [128, 384])
def test_quantizer_corner_cases(qll, K):
    w = corner_rows(K)
    q_ref, s_ref = oracle.quantize_int4(w)
    q, s = qll.quantize_int4_weights(dev_bf16(w))
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32)), "scales"
    assert np.array_equal(q.cpu().numpy(), q_ref), "codes"


GEMM_SHAPES = [(1, 520, 1024), (37, 300, 2048), (130, 264, 512), (300, 648, 1152)]


@pytest.fixture(scope="module")
def w4_cases():
    out = {}
    for (M, N, K) in GEMM_SHAPES:
        key = (workloads.W_TEST, 81, M, N, K)
        A = workloads.w4_activations(M, K, key=key)
        B = workloads.mx_codes(N, K, (*key, 1))
        s = workloads.scales_uniform(N * (K // 128), (*key, 2)).reshape(N, K // 128)
        ref, absref = oracle.gemm_w4a16(A, B, s, with_abs=True)
        out[(M, N, K)] = (A, B, s, ref, absref)
    return out


@pytest.mark.parametrize("shape", GEMM_SHAPES)
@pytest.mark.parametrize("splits", [1, 3])
def test_gemm_all_variants(qll, w4_cases, shape, splits):
    A, B, s, ref, absref = w4_cases[shape]
    K = shape[2]
    dA, dB, ds = dev_bf16(A), dev(B), dev(s)
    for name in names(qll):
        for od in ("fp32", "bf16"):
            y = qll.gemm_w4a16(dA, dB, ds, out_dtype=od, cfg=(name, splits))
            torch.cuda.synchronize()
            check_fp(host_f64(y), ref, absref, K, od, f"{name} S={splits} {od}", mfma="w4a16")


@pytest.mark.parametrize("M", [1, 40, 333])
def test_gemm_integer_inputs_exact(qll, M):
    """Unit scales and small integer activations: every partial sum is an
    integer below 2^24, so every variant must return the oracle's value."""
    N, K = 200, 2048
    key = (workloads.W_TEST, 82, M)
    Ai = workloads.rng(*key, 0).integers(-64, 65, size=(M, K)).astype(np.float32)
    A = workloads.to_bf16_bits(Ai)
    B = workloads.mx_codes(N, K, (*key, 1))
    s = np.ones((N, K // 128), np.float32)
    ref = oracle.gemm_w4a16(A, B, s)
    dA, dB, ds = dev_bf16(A), dev(B), dev(s)
    for name in names(qll):
        for splits in (1, 2):
            y = qll.gemm_w4a16(dA, dB, ds, out_dtype="fp32", cfg=(name, splits))
            torch.cuda.synchronize()
            assert np.array_equal(host_f64(y), ref), f"{name} S={splits}"


def test_gemm_empty(qll):
    A = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((3, 128), dtype=torch.uint8, device="cuda")
    s = torch.ones((3, 2), dtype=torch.float32, device="cuda")
    y = qll.gemm_w4a16(A, B, s)
    torch.cuda.synchronize()
    assert y.shape == (0, 3)


@pytest.mark.parametrize("M,N,K", [(16, 1040, 2048), (300, 648, 1152)])
def test_end_to_end(qll, M, N, K):
    x = workloads.w4_activations(M, K, key=(workloads.W_TEST, 83, M, K))
    w = workloads.w4_weights(N, K, key=(workloads.W_TEST, 83, N, K))
    q_ref, s_ref = oracle.quantize_int4(w)
    q, s = qll.quantize_int4_weights(dev_bf16(w))
    y = qll.gemm_w4a16(dev_bf16(x), q, s, out_dtype="bf16")
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    ref, absref = oracle.gemm_w4a16(x, q_ref, s_ref, with_abs=True)
    check_fp(host_f64(y), ref, absref, K, "bf16", f"M={M} N={N} K={K}", mfma="w4a16")


@pytest.fixture(scope="module")
def w4_weights():
    out = {}
    for N, K in workloads.W4_SHAPES:
        w = workloads.w4_weights(N, K)
        out[(N, K)] = (w,) + oracle.quantize_int4(w)
    return out


@pytest.mark.parametrize("N,K", workloads.W4_SHAPES)
def test_w4_sweep_full_size_sampled(qll, w4_weights, N, K):
    w, q_ref, s_ref = w4_weights[(N, K)]
    q, s = qll.quantize_int4_weights(dev_bf16(w))
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    x_all = workloads.w4_activations(workloads.MAX_M, K)
    dx = dev_bf16(x_all)
    for M in workloads.W4_M:
        y = qll.gemm_w4a16(dx[:M].contiguous(), q, s, out_dtype="bf16")
        torch.cuda.synchronize()
        rows = sample_rows(M, 6, seed=K)
        ref, absref = oracle.gemm_w4a16(x_all[:M], q_ref, s_ref, rows=rows, with_abs=True)
        check_fp(host_f64(y[torch.from_numpy(rows).cuda()]), ref, absref, K, "bf16",
                 f"M={M} N={N} K={K}", mfma="w4a16")

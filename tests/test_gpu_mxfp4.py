"""GPU parity of the MXFP4 quantizer and GEMM against the oracle.

MXFP4 is the block-scaled form of the 4-bit formats that "Helion in vLLM: A
Unified Route to Tunable Linear Kernels" lists among vLLM's (introduction);
the encodings and the conversion rule are those of the OCP Microscaling (MX)
v1.0 specification, as the oracle states.

Bars: codes and scale bytes bit-exact (the quantizer decides integers: both
sides take the decision exactly, x / 2^E being exact in any binary format);
GEMM outputs within the rule of tests/gpu_util.py, and bit-exact where every
partial sum is exactly representable (unit scales); every variant, with and
without Split-K, on shapes with ragged M, N and K tails; the sweep shapes at
full size on sampled rows through the shipped dispatch.
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
    return [v["name"] for v in qll.variants("mxfp4")]


def host_u8(t):
    return t.cpu().numpy()


# ------------------------------------------------------------------ quantizer
def special_rows(K):
    """bf16 rows that hit the rule's corner cases, one per row."""
    rows = []
    t = 2.0 ** 5
    # ties of the E2M1 grid (block max 6 * 2^5 fixes E = 5) and their negatives
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.5, 3.0]
    r = np.zeros(K, np.float32)
    for i, v in enumerate(ties):
        r[i] = v * t
        r[i + 16] = -v * t
    rows.append(r)
    # an all-zero block, negative zeros, then a block of values that saturate
    # (max 7.9375 * 2^E after the power-of-two choice)
    r = np.zeros(K, np.float32)
    r[3] = -0.0
    r[17] = -0.0
    if K >= 96:
        r[64:96] = np.linspace(-7.9375, 7.9375, 32, dtype=np.float32)
    rows.append(r)
    # subnormal and tiny-normal bf16 blocks (scale byte clamped at 0)
    r = np.full(K, 2.0 ** -130, np.float32)
    r[5] = -(2.0 ** -128)
    r[7] = 2.0 ** -127
    if K >= 64:
        r[32:64] = 2.0 ** -125
        r[40] = 1.5 * 2.0 ** -124
    rows.append(r)
    # near the bf16 maximum and powers of two exactly at block maxima
    r = np.ones(K, np.float32)
    r[0] = 3.3895313892515355e38
    r[1] = -1.7e38
    if K >= 64:
        r[32:64] = 4.0
        r[50] = 2.0 ** 100
    rows.append(r)
    return workloads.to_bf16_bits(np.stack(rows))


QUANT_SHAPES = [(1, 32), (3, 96), (5, 2048), (64, 4096), (300, 1056), (2, 65536)]


@pytest.mark.parametrize("M,K", QUANT_SHAPES)
def test_quantizer_bit_exact(qll, M, K):
    x = workloads.mx_activations(M, K, key=(workloads.W_TEST, 70, M, K))
    q_ref, s_ref = oracle.quantize_mxfp4(x)
    q, s = qll.quantize_mxfp4(dev_bf16(x))
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(s), s_ref), "scale bytes"
    assert np.array_equal(host_u8(q), q_ref), "codes"


@pytest.mark.parametrize("K", [32, 128, 2048])
def test_quantizer_corner_cases(qll, K):
    x = special_rows(K)
    q_ref, s_ref = oracle.quantize_mxfp4(x)
    q, s = qll.quantize_mxfp4(dev_bf16(x))
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(s), s_ref), "scale bytes"
    assert np.array_equal(host_u8(q), q_ref), "codes"


def test_quantizer_empty(qll):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    q, s = qll.quantize_mxfp4(x)
    torch.cuda.synchronize()
    assert q.shape == (0, 32) and s.shape == (0, 2)


# ------------------------------------------------------------------ GEMM
GEMM_SHAPES = [(1, 520, 1024), (37, 300, 2048), (130, 264, 512), (300, 648, 1152)]


@pytest.fixture(scope="module")
def mx_cases():
    out = {}
    for (M, N, K) in GEMM_SHAPES:
        key = (workloads.W_TEST, 71, M, N, K)
        A = workloads.mx_codes(M, K, (*key, 0))
        B = workloads.mx_codes(N, K, (*key, 1))
        sa = workloads.mx_scale_bytes(M, K, (*key, 2))
        sb = workloads.mx_scale_bytes(N, K, (*key, 3))
        ref, absref = oracle.gemm_mxfp4(A, B, sa, sb, with_abs=True)
        out[(M, N, K)] = (A, B, sa, sb, ref, absref)
    return out


@pytest.mark.parametrize("shape", GEMM_SHAPES)
@pytest.mark.parametrize("splits", [1, 3])
def test_gemm_all_variants(qll, mx_cases, shape, splits):
    A, B, sa, sb, ref, absref = mx_cases[shape]
    K = shape[2]
    dA, dB, dsa, dsb = dev(A), dev(B), dev(sa), dev(sb)
    for name in names(qll):
        for od in ("fp32", "bf16"):
            y = qll.gemm_mxfp4(dA, dB, dsa, dsb, out_dtype=od, cfg=(name, splits))
            torch.cuda.synchronize()
            check_fp(host_f64(y), ref, absref, K, od, f"{name} S={splits} {od}", mfma="fp4")


def test_gemm_sequential_variants_agree_bitwise(qll, mx_cases):
    """Kernels that add the K steps one after the other into one accumulator
    (every pipelined tile, the row-split skinny kernels) give identical bits;
    the wave-split skinny kernels add per-wave partial sums instead."""
    A, B, sa, sb, ref, absref = mx_cases[(37, 300, 2048)]
    dA, dB, dsa, dsb = dev(A), dev(B), dev(sa), dev(sb)
    base = qll.gemm_mxfp4(dA, dB, dsa, dsb, out_dtype="fp32",
                          cfg=("p128x128_w2x2_k128_s2", 1)).cpu().numpy()
    diff = []
    for name in names(qll):
        if name[0] == "k":
            continue
        y = qll.gemm_mxfp4(dA, dB, dsa, dsb, out_dtype="fp32", cfg=(name, 1)).cpu().numpy()
        if not np.array_equal(y.view(np.uint32), base.view(np.uint32)):
            diff.append(name)
    assert not diff, f"variants differing bitwise from p128x128_w2x2_k128_s2: {diff}"


@pytest.mark.parametrize("M", [1, 40, 333])
def test_gemm_unit_scales_exact(qll, M):
    """Unit scales: every product is a multiple of 1/4 below 36 and every
    partial sum an exactly representable fp32 value, so all variants must
    return the oracle's value exactly."""
    N, K = 200, 2048
    key = (workloads.W_TEST, 72, M)
    A = workloads.mx_codes(M, K, (*key, 0))
    B = workloads.mx_codes(N, K, (*key, 1))
    sa = np.full((M, K // 32), 127, np.uint8)
    sb = np.full((N, K // 32), 127, np.uint8)
    ref = oracle.gemm_mxfp4(A, B, sa, sb)
    dA, dB, dsa, dsb = dev(A), dev(B), dev(sa), dev(sb)
    for name in names(qll):
        for splits in (1, 2):
            y = qll.gemm_mxfp4(dA, dB, dsa, dsb, out_dtype="fp32", cfg=(name, splits))
            torch.cuda.synchronize()
            assert np.array_equal(host_f64(y), ref), f"{name} S={splits}"


def test_gemm_empty_and_tiny(qll):
    K = 128
    A = torch.zeros((0, K // 2), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((0, K // 32), dtype=torch.uint8, device="cuda")
    B = torch.zeros((3, K // 2), dtype=torch.uint8, device="cuda")
    sb = torch.full((3, K // 32), 127, dtype=torch.uint8, device="cuda")
    y = qll.gemm_mxfp4(A, B, sa, sb)
    torch.cuda.synchronize()
    assert y.shape == (0, 3)
    # one row, one column, one 128-wide K step: 6 * 6 * 2^(1+2) per element x 128
    A1 = torch.full((1, K // 2), 0x77, dtype=torch.uint8, device="cuda")
    sa1 = torch.full((1, K // 32), 128, dtype=torch.uint8, device="cuda")
    B1 = torch.full((1, K // 2), 0x77, dtype=torch.uint8, device="cuda")
    sb1 = torch.full((1, K // 32), 129, dtype=torch.uint8, device="cuda")
    for name in names(qll):
        y = qll.gemm_mxfp4(A1, B1, sa1, sb1, out_dtype="fp32", cfg=(name, 1))
        torch.cuda.synchronize()
        assert y.item() == 36.0 * 8 * K, name


@pytest.mark.parametrize("M,N,K", [(16, 1040, 2048), (300, 648, 1152)])
def test_end_to_end_quantize_and_gemm(qll, M, N, K):
    """bf16 activations and weights quantized on the device (codes bit-exact),
    then the GEMM through the dispatch."""
    x = workloads.mx_activations(M, K, key=(workloads.W_TEST, 73, M, K))
    w = workloads.mx_weights(N, K, key=(workloads.W_TEST, 73, N, K))
    qa_ref, sa_ref = oracle.quantize_mxfp4(x)
    qb_ref, sb_ref = oracle.quantize_mxfp4(w)
    qa, sa = qll.quantize_mxfp4(dev_bf16(x))
    qb, sb = qll.quantize_mxfp4(dev_bf16(w))
    y = qll.gemm_mxfp4(qa, qb, sa, sb, out_dtype="bf16")
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(qa), qa_ref) and np.array_equal(host_u8(sa), sa_ref)
    assert np.array_equal(host_u8(qb), qb_ref) and np.array_equal(host_u8(sb), sb_ref)
    ref, absref = oracle.gemm_mxfp4(qa_ref, qb_ref, sa_ref, sb_ref, with_abs=True)
    check_fp(host_f64(y), ref, absref, K, "bf16", f"M={M} N={N} K={K}", mfma="fp4")


# ------------------------------------------------------------------ full size
@pytest.fixture(scope="module")
def mx_weights():
    out = {}
    for N, K in workloads.MX_SHAPES:
        w = workloads.mx_weights(N, K)
        out[(N, K)] = (w,) + oracle.quantize_mxfp4(w)
    return out


@pytest.mark.parametrize("N,K", workloads.MX_SHAPES)
def test_mx_sweep_full_size_sampled(qll, mx_weights, N, K):
    """The MXFP4 sweep shapes at full size through the shipped dispatch: the
    device quantizes weights and activations (bit-exact), every M of the
    sweep is checked on sampled rows."""
    w, qb_ref, sb_ref = mx_weights[(N, K)]
    qb, sb = qll.quantize_mxfp4(dev_bf16(w))
    torch.cuda.synchronize()
    assert np.array_equal(host_u8(qb), qb_ref) and np.array_equal(host_u8(sb), sb_ref)
    x_all = workloads.mx_activations(workloads.MAX_M, K)
    qa_all, sa_all = oracle.quantize_mxfp4(x_all)
    for M in workloads.MX_M:
        qa, sa = qll.quantize_mxfp4(dev_bf16(x_all[:M]))
        y = qll.gemm_mxfp4(qa, qb, sa, sb, out_dtype="bf16")
        torch.cuda.synchronize()
        assert np.array_equal(host_u8(qa), qa_all[:M]) and np.array_equal(host_u8(sa), sa_all[:M])
        rows = sample_rows(M, 6, seed=K)
        ref, absref = oracle.gemm_mxfp4(qa_all[:M], qb_ref, sa_all[:M], sb_ref, rows=rows,
                                        with_abs=True)
        check_fp(host_f64(y[torch.from_numpy(rows).cuda()]), ref, absref, K, "bf16",
                 f"M={M} N={N} K={K}", mfma="fp4")

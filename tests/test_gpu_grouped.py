"""GPU parity of gemm_fp8_grouped, the per-expert FP8 GEMM of an FP8
mixture-of-experts layer (built from the scaled FP8 GEMM of "Helion in vLLM:
A Unified Route to Tunable Linear Kernels", "What the integration changes").

Bars: within the floating-point rule of tests/gpu_util.py of the oracle's
grouped product; and bitwise equal to gemm_fp8_scaled run with the same
pipelined variant on each expert's rows alone (the same MFMA sequence per
output element).
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import check_fp, dev, dev_bf16, dev_e4m3, host_f64  # noqa: E402


@pytest.fixture(scope="module")
def qll():
    import quantized_linear_layer_scaled_amd as q
    q.load_library()
    q.init()
    return q


def pipe_names(qll):
    # the pipelined tiles with 128-byte K stages: the grouped GEMM has every
    # one of them
    return [v["name"] for v in qll.variants("fp8") if v["name"].endswith(
        tuple(f"_k128_s{s}" for s in (2, 3, 4)))]


def grouped_case(counts, N, K, key):
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M, E = int(off[-1]), len(counts)
    x = workloads.bf16_normal((M, K), (*key, 0), outlier_frac=0.01)
    w = workloads.bf16_normal((E * N, K), (*key, 1), std=0.02)
    A, sa = oracle.quantize_fp8(x)
    B, sb = oracle.quantize_fp8(w)
    return off, A, B.reshape(E, N, K), sa[:, 0].copy(), sb[:, 0].reshape(E, N).copy()


# uneven experts: empty ones, partial tiles, a single row, more rows than a tile
CASES = [((3, 0, 70, 1, 0, 129, 33, 8), 200, 528),
         ((64,), 96, 256),
         ((0, 0, 5), 130, 1040),
         # more experts than one 64-lane scan of the offsets
         (tuple((7 * i) % 5 for i in range(69)) + (140,), 96, 256)]


@pytest.mark.parametrize("counts,N,K", CASES)
def test_grouped_all_variants(qll, counts, N, K):
    off, A, B, sa, sb = grouped_case(counts, N, K, (workloads.W_TEST, 50, len(counts), N, K))
    ref, absref = oracle.gemm_fp8_grouped(A, B, sa, sb, off, with_abs=True)
    dA, dB, dsa, dsb = dev_e4m3(A), dev_e4m3(B), dev(sa), dev(sb)
    doff = torch.from_numpy(off).cuda()
    for name in [None] + pipe_names(qll):
        for od in ("bf16", "fp32"):
            y = qll.gemm_fp8_grouped(dA, dB, dsa, dsb, doff, out_dtype=od, variant=name)
            torch.cuda.synchronize()
            check_fp(host_f64(y), ref, absref, K, od, f"grouped {name} {counts} {od}")


def test_grouped_equals_per_expert_dense_bitwise(qll):
    counts = (17, 0, 150, 64, 3)
    N, K = 260, 1024
    off, A, B, sa, sb = grouped_case(counts, N, K, (workloads.W_TEST, 51))
    dA, dB, dsa, dsb = dev_e4m3(A), dev_e4m3(B), dev(sa), dev(sb)
    doff = torch.from_numpy(off).cuda()
    for name in ("p64x64_w2x2_k128_s3", "p128x128_w2x2_k128_s2", "p256x128_w4x2_k128_s3"):
        y = qll.gemm_fp8_grouped(dA, dB, dsa, dsb, doff, out_dtype="fp32", variant=name)
        for e in range(len(counts)):
            lo, hi = int(off[e]), int(off[e + 1])
            if lo == hi:
                continue
            ye = qll.gemm_fp8_scaled(dA[lo:hi].contiguous(), dB[e].contiguous(),
                                     dsa[lo:hi].contiguous(), dsb[e].contiguous(),
                                     out_dtype="fp32", cfg=(name, 1))
            torch.cuda.synchronize()
            assert torch.equal(y[lo:hi].view(torch.int32), ye.view(torch.int32)), (name, e)


def test_grouped_offsets_read_as_clamped_running_maximum(qll):
    # Offsets outside [0, M] or out of order are read as their running
    # maximum clamped to [0, M]: here [-7, 60, 25, 200, 90] over M = 140 rows
    # gives the experts the rows [0, 60), [60, 60), [60, 140), [140, 140).
    counts = (40, 30, 50, 20)
    N, K = 96, 256
    _, A, B, sa, sb = grouped_case(counts, N, K, (workloads.W_TEST, 53))
    bad = torch.tensor([-7, 60, 25, 200, 90], dtype=torch.int32).cuda()
    owned = [(0, 0, 60), (2, 60, 140)]
    dA, dB, dsa, dsb = dev_e4m3(A), dev_e4m3(B), dev(sa), dev(sb)
    for name in ("p64x64_w2x2_k128_s3", "p128x128_w2x2_k128_s2", "p256x256_w2x4_k128_s2"):
        y = qll.gemm_fp8_grouped(dA, dB, dsa, dsb, bad, out_dtype="fp32", variant=name)
        torch.cuda.synchronize()
        for e, lo, hi in owned:
            ref, absref = oracle.gemm_fp8(A[lo:hi], B[e], sa[lo:hi], sb[e], with_abs=True)
            check_fp(host_f64(y)[lo:hi], ref, absref, K, "fp32", f"grouped {name} expert {e}")


@pytest.fixture(scope="module")
def moe_weights(qll):
    N, K = workloads.MOE_SHAPE
    E = workloads.MOE_E
    w = workloads.moe_weights(E, N, K).reshape(E * N, K)
    qw, sw = qll.quantize_per_token_fp8(dev_bf16(w))
    B, sb = oracle.quantize_fp8(w)
    torch.cuda.synchronize()
    return qw, sw, B, sb


@pytest.mark.parametrize("T", workloads.MOE_T)
def test_grouped_moe_workload_sampled(qll, moe_weights, T):
    N, K = workloads.MOE_SHAPE
    E = workloads.MOE_E
    qw, sw, B, sb = moe_weights
    off = workloads.moe_routing(T)
    M = int(off[-1])
    x = workloads.moe_activations(M, K)
    # the quantization runs on the device (as in the layer), its codes are
    # checked against the oracle's
    qx, sx = qll.quantize_per_token_fp8(dev_bf16(x))
    torch.cuda.synchronize()
    A, sa = oracle.quantize_fp8(x)
    assert np.array_equal(qx.cpu().view(torch.uint8).numpy(), A)
    y = qll.gemm_fp8_grouped(qx, qw.view(E, N, K), sx.view(M), sw.view(E, N),
                             torch.from_numpy(off).cuda())
    torch.cuda.synchronize()
    g = np.random.default_rng([52, T])
    rows = np.unique(np.concatenate([[0, M - 1], g.integers(0, M, 24)]))
    ref, absref = oracle.gemm_fp8_grouped(A, B.reshape(E, N, K), sa[:, 0],
                                          sb[:, 0].reshape(E, N), off, rows=rows,
                                          with_abs=True)
    check_fp(host_f64(y)[rows], ref, absref, K, "bf16", f"moe T={T}")


def test_grouped_zero_rows_is_noop(qll):
    B = torch.zeros((2, 64, 128), dtype=torch.float8_e4m3fn, device="cuda")
    A = torch.zeros((0, 128), dtype=torch.float8_e4m3fn, device="cuda")
    y = qll.gemm_fp8_grouped(A, B, torch.zeros(0, device="cuda"),
                             torch.zeros((2, 64), device="cuda"),
                             torch.zeros(3, dtype=torch.int32, device="cuda"))
    assert y.shape == (0, 64)

"""The matrix core's own rounding, per instruction kind, against the oracle.

The acceptance rule in gpu_util.py adds a term t_mfma to the fp32
accumulation bound for the e4m3 ops only.  This test measures, for each kind
of matrix-core step the kernels use, the worst elementwise error relative to
absref = sum_k |a_k b_k| (fp32 output, unit scales, so nothing but the sum is
rounded) and pins it below that kind's budget: the fp32 term
(K + K/128 + 4) * 2^-23 plus MFMA_TERM[kind].  For the bf16, MXFP4 and W4A16
steps it also pins the error below 2^-20 of absref, far inside the fp32
term, which is why those ops carry no extra term.

Operations: the scaled products of "Helion in vLLM: A Unified Route to
Tunable Linear Kernels", section "What the integration changes" (FP8,
batch-invariant bf16, MXFP4, W4A16).
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from gpu_util import MFMA_TERM, dev, dev_bf16, dev_e4m3, host_f64  # noqa: E402


@pytest.fixture(scope="module")
def qll():
    import quantized_linear_layer_scaled_amd as q
    q.load_library()
    return q


M, N = 64, 256


def worst(y, ref, absref):
    torch.cuda.synchronize()
    return float(np.max(np.abs(host_f64(y) - ref) / np.maximum(absref, 1e-300)))


def pin(kind, name, r, K):
    acc = (K + K // 128 + 4) * 2.0 ** -23
    print(f"{kind} {name} K={K}: max err/absref = 2^{np.log2(max(r, 1e-300)):.2f} "
          f"(fp32 term 2^{np.log2(acc):.2f})", flush=True)
    assert r <= acc + MFMA_TERM[kind], f"{kind} {name} K={K}: {r:.3e}"
    if MFMA_TERM[kind] == 0.0:
        assert r <= 2.0 ** -20, f"{kind} {name} K={K}: {r:.3e}"


def e4m3_codes(rng, shape):
    c = rng.integers(0, 256, shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0  # NaN codes
    return c


@pytest.mark.parametrize("K", [256, 2048])
def test_e4m3_steps(qll, K):
    # every finite code, both step shapes (16x16x128 and 32x32x64)
    rng = np.random.default_rng(K + 1)
    A, B = e4m3_codes(rng, (M, K)), e4m3_codes(rng, (N, K))
    one_a, one_b = np.ones(M, np.float32), np.ones(N, np.float32)
    ref, absref = oracle.gemm_fp8(A, B, one_a, one_b, with_abs=True)
    for name in ("k16x64_w8", "n64x128_w2x2_k128", "p64x64_w2x2_k128_s2",
                 "p128x128_w2x2_k64_s4", "p64x128_w2x2_k64_s6"):
        y = qll.gemm_fp8_scaled(dev_e4m3(A), dev_e4m3(B), dev(one_a), dev(one_b),
                                out_dtype="fp32", cfg=(name, 1))
        pin("e4m3", name, worst(y, ref, absref), K)


@pytest.mark.parametrize("K", [256, 2048])
def test_bf16_steps(qll, K):
    a = workloads.bf16_normal((M, K), (workloads.W_TEST, 40, K))
    b = workloads.bf16_normal((N, K), (workloads.W_TEST, 41, K))
    ref, absref = oracle.gemm_bf16(a, b, with_abs=True)
    for name in ("k16x64_w8", "n64x128_w2x2_k128", "p64x64_w2x2_k128_s2"):
        y = qll.gemm_bf16_batch_invariant(dev_bf16(a), dev_bf16(b), out_dtype="fp32",
                                          cfg=(name, 1))
        pin("bf16", name, worst(y, ref, absref), K)


@pytest.mark.parametrize("K", [256, 2048])
def test_mxfp4_steps(qll, K):
    # every E2M1 code; scale bytes around 2^0
    rng = np.random.default_rng(K + 2)
    ca = rng.integers(0, 256, (M, K // 2)).astype(np.uint8)
    cb = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    xa = rng.integers(118, 137, (M, K // 32)).astype(np.uint8)
    xb = rng.integers(118, 137, (N, K // 32)).astype(np.uint8)
    ref, absref = oracle.gemm_mxfp4(ca, cb, xa, xb, with_abs=True)
    for name in ("k16x64_w8", "p64x64_w2x2_k128_s2"):
        y = qll.gemm_mxfp4(dev(ca), dev(cb), dev(xa), dev(xb), out_dtype="fp32", cfg=(name, 1))
        pin("fp4", name, worst(y, ref, absref), K)


@pytest.mark.parametrize("K", [256, 2048])
def test_w4a16_steps(qll, K):
    rng = np.random.default_rng(K + 3)
    a = workloads.bf16_normal((M, K), (workloads.W_TEST, 42, K))
    codes = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    sc = rng.uniform(1e-3, 1e-2, (N, K // 128)).astype(np.float32)
    ref, absref = oracle.gemm_w4a16(a, codes, sc, with_abs=True)
    for name in ("k16x64_w8", "p64x64_w2x2_s2", "t64x64_w2x2"):
        y = qll.gemm_w4a16(dev_bf16(a), dev(codes), dev(sc), out_dtype="fp32", cfg=(name, 1))
        pin("w4a16", name, worst(y, ref, absref), K)

"""GPU parity at the full workload sizes, through the shipped dispatch (the
configuration the benchmark times): W8A8 INT8 M=16 N=K=2048 in full; the FP8
dynamic sweep, Block-FP8 and the large-vocabulary shape on sampled rows.

Workloads: the serving shapes of vLLM PR #53446 ("H100 NVL Sweep Results")
run through the three quantized formats of "Helion in vLLM: A Unified Route
to Tunable Linear Kernels" ("What the integration changes").  Quantized bytes
and scales are bit-exact; the GEMMs meet the rule of tests/gpu_util.py.
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import (block_fp8_product, check_all_rows, check_fp, dev,  # noqa: E402
                      dev_bf16, dev_e4m3, fp8_product, host_codes, host_f64, sample_rows)


@pytest.fixture(scope="module")
def qll():
    import quantized_linear_layer_scaled_amd as q
    q.load_library()
    q.init()
    return q


def test_int8_full_bit_exact(qll):
    M, N, K = workloads.INT8_SHAPE
    d = workloads.int8_inputs(M, N, K)
    acc, y = oracle.gemm_w8a8_int8(d["A"], d["B"], d["sa"], d["sb"])
    A, B, sa, sb = dev(d["A"]), dev(d["B"]), dev(d["sa"]), dev(d["sb"])
    o32 = qll.gemm_w8a8_int8(A, B, sa, sb, out_dtype="int32")
    ob = qll.gemm_w8a8_int8(A, B, sa, sb, out_dtype="bf16")
    torch.cuda.synchronize()
    assert np.array_equal(o32.cpu().numpy(), acc)
    assert np.array_equal(ob.view(torch.int16).cpu().numpy().view(np.uint16),
                          oracle.bf16_encode(y))


def test_int8_every_table_bucket_bit_exact(qll):
    # every M bucket of the shipped INT8 table at N = K = 2048 -- the decode
    # kernels, the pipelined tiles, the two-K-group tiles of the mid-size M
    # -- through the dispatch: int32 accumulators and bf16 output bit-exact
    # against the oracle on sampled rows
    N, K = 2048, 2048
    picks = set()
    for M in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048):
        d = workloads.int8_inputs(M, N, K, key=(workloads.W_TEST, 70, M))
        rows = sample_rows(M, 12, seed=M)
        acc, y = oracle.gemm_w8a8_int8(d["A"], d["B"], d["sa"], d["sb"], rows=rows)
        A, B, sa, sb = dev(d["A"]), dev(d["B"]), dev(d["sa"]), dev(d["sb"])
        o32 = qll.gemm_w8a8_int8(A, B, sa, sb, out_dtype="int32")
        ob = qll.gemm_w8a8_int8(A, B, sa, sb, out_dtype="bf16")
        torch.cuda.synchronize()
        picks.add(qll.select("int8", M, N, K)[0])
        assert np.array_equal(o32.cpu().numpy()[rows], acc), M
        assert np.array_equal(ob.view(torch.int16).cpu().numpy().view(np.uint16)[rows],
                              oracle.bf16_encode(y)), M
    assert any(n.endswith("_g2") for n in picks), picks


@pytest.fixture(scope="module")
def fp8_weights():
    out = {}
    for N, K in workloads.FP8_SHAPES:
        w = workloads.weights_bf16(N, K)
        B, sb = oracle.quantize_fp8(w)
        out[(N, K)] = (w, B, sb[:, 0].copy())
    return out


@pytest.mark.parametrize("N,K", workloads.FP8_SHAPES)
def test_fp8_dynamic_sweep(qll, fp8_weights, N, K):
    w, B, sb = fp8_weights[(N, K)]
    # the weights: per-output-channel quantization on the device is bit-exact
    qB, qsb = qll.quantize_per_token_fp8(dev_bf16(w))
    torch.cuda.synchronize()
    assert np.array_equal(host_codes(qB), B)
    assert np.array_equal(qsb.cpu().numpy()[:, 0].view(np.uint32), sb.view(np.uint32))
    x_all = workloads.fp8_activations(workloads.MAX_M, K)
    Aq_all, sa_all = oracle.quantize_fp8(x_all)
    for M in workloads.FP8_M:
        x = dev_bf16(x_all[:M])
        q, sa = qll.quantize_per_token_fp8(x)
        y = qll.gemm_fp8_scaled(q, qB, sa, qsb)
        torch.cuda.synchronize()
        assert np.array_equal(host_codes(q), Aq_all[:M]), f"M={M} codes"
        assert np.array_equal(sa.cpu().numpy().view(np.uint32),
                              sa_all[:M].view(np.uint32)), f"M={M} scales"
        rows = sample_rows(M, 8, seed=M)
        ref, absref = oracle.gemm_fp8(Aq_all[:M], B, sa_all[:M, 0].copy(), sb,
                                      rows=rows, with_abs=True)
        check_fp(host_f64(y)[rows], ref, absref, K, "bf16", f"fp8 N={N} K={K} M={M}")
        check_all_rows(y, fp8_product(q, qB, sa, qsb), "bf16", f"fp8 N={N} K={K} M={M}")


@pytest.mark.parametrize("N,K", workloads.BLOCK_SHAPES)
def test_block_fp8_sweep(qll, N, K):
    w = workloads.weights_bf16(N, K, key=(workloads.W_BLOCK,))
    B, sb = oracle.quantize_fp8_block(w)
    qB, qsb = qll.quantize_weight_block_fp8(dev_bf16(w))
    torch.cuda.synchronize()
    assert np.array_equal(host_codes(qB), B)
    assert np.array_equal(qsb.cpu().numpy().view(np.uint32), sb.view(np.uint32))
    x_all = workloads.block_activations(workloads.MAX_M, K)
    Aq_all, sa_all = oracle.quantize_fp8(x_all, group=128)
    for M in workloads.BLOCK_M:
        q, sa = qll.quantize_per_token_fp8(dev_bf16(x_all[:M]), group=128)
        y = qll.gemm_block_fp8(q, qB, sa, qsb)
        torch.cuda.synchronize()
        assert np.array_equal(host_codes(q), Aq_all[:M])
        assert np.array_equal(sa.cpu().numpy().view(np.uint32), sa_all[:M].view(np.uint32))
        rows = sample_rows(M, 8, seed=M)
        ref, absref = oracle.gemm_block_fp8(Aq_all[:M], B, sa_all[:M].copy(), sb,
                                            rows=rows, with_abs=True)
        check_fp(host_f64(y)[rows], ref, absref, K, "bf16", f"block N={N} K={K} M={M}")
        check_all_rows(y, block_fp8_product(q, qB, sa, qsb), "bf16", f"block N={N} K={K} M={M}")


def test_vocab_projection_both_paths(qll):
    N, K = workloads.VOCAB_SHAPE
    w = workloads.vocab_weights(N, K)
    a_full = workloads.vocab_activations(K)
    B, sb = oracle.quantize_fp8(w)
    dW = dev_bf16(w)
    qB, qsb = qll.quantize_per_token_fp8(dW)
    torch.cuda.synchronize()
    assert np.array_equal(host_codes(qB), B)
    Aq_all, sa_all = oracle.quantize_fp8(a_full)
    dA = dev_bf16(a_full)
    bi_full = qll.gemm_bf16_batch_invariant(dA, dW)
    check_all_rows(bi_full, dA.to(torch.float64) @ dW.to(torch.float64).T, "bf16",
                   "vocab bf16 M=2048 every row")
    for M in workloads.VOCAB_M:
        rows = sample_rows(M, 3, seed=M)
        # bf16 batch-invariant path
        y = qll.gemm_bf16_batch_invariant(dA[:M].contiguous(), dW)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), bi_full[:M].view(torch.int16)), M
        ref, absref = oracle.gemm_bf16(a_full[:M], w, rows=rows, with_abs=True)
        check_fp(host_f64(y)[rows], ref, absref, K, "bf16", f"vocab bf16 M={M}", mfma="bf16")
        # FP8 dynamic path on the same data
        q, sa = qll.quantize_per_token_fp8(dA[:M].contiguous())
        y8 = qll.gemm_fp8_scaled(q, qB, sa, qsb)
        torch.cuda.synchronize()
        assert np.array_equal(host_codes(q), Aq_all[:M])
        ref, absref = oracle.gemm_fp8(Aq_all[:M], B, sa_all[:M, 0].copy(), sb[:, 0].copy(),
                                      rows=rows, with_abs=True)
        check_fp(host_f64(y8)[rows], ref, absref, K, "bf16", f"vocab fp8 M={M}")
        check_all_rows(y8, fp8_product(q, qB, sa, qsb), "bf16", f"vocab fp8 M={M}")

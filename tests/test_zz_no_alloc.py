"""GPU check of gemm_fp8_scaled_noalloc, the FP8 GEMM entry point that
allocates nothing (its Split-K partials live in the library's static device
array): called through the C ABI, its output is bitwise the output of
gemm_fp8_scaled on the same inputs -- on two calls in a row, the second with
fewer rows, on shapes whose configuration splits K -- and within the
floating-point rule of tests/gpu_util.py of the oracle; a configuration whose
partials exceed the array is refused before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
from gpu_util import check_fp, dev, dev_bf16, dev_e4m3, host_f64, sample_rows  # noqa: E402


@pytest.fixture(scope="module")
def qll():
    import quantized_linear_layer_scaled_amd as q
    q.load_library()
    q.init()
    return q


def call_noalloc(qll, q, B, sa, sb, out, M, N, K):
    L = qll.load_library()
    return L.gemm_fp8_scaled_noalloc(
        q.data_ptr(), B.data_ptr(), sa.data_ptr(), sb.data_ptr(), out.data_ptr(), 0,
        M, N, K, torch.cuda.current_stream().cuda_stream)


@pytest.mark.parametrize("N,K,Ms", [(2048, 6144, (256, 200)), (2048, 6144, (64, 40)),
                                    (4096, 2048, (2048, 1500)), (4096, 2048, (16, 3))])
def test_noalloc_equals_gemm_fp8_scaled(qll, N, K, Ms):
    w = workloads.weights_bf16(N, K, key=(workloads.W_TEST, 60))
    B, sb = oracle.quantize_fp8(w)
    dB, dsb = dev_e4m3(B), dev(sb[:, 0].copy())
    x_all = workloads.fp8_activations(max(Ms), K, key=(workloads.W_TEST, 61))
    qr_all, sr_all = oracle.quantize_fp8(x_all)
    splits_seen = []
    for M in Ms:  # two calls in a row, the second with fewer rows
        q, sa = dev_e4m3(qr_all[:M]), dev(sr_all[:M, 0].copy())
        name, splits = qll.select("fp8", M, N, K)
        splits_seen.append(qll.effective_splits("fp8", K, splits))
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        assert call_noalloc(qll, q, dB, sa, dsb, out, M, N, K) == 0
        want = qll.gemm_fp8_scaled(q, dB, sa, dsb)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), (M, name, splits)
        rows = sample_rows(M, 8, seed=M)
        ref, absref = oracle.gemm_fp8(qr_all[:M], B, sr_all[:M, 0].copy(), sb[:, 0].copy(),
                                      rows=rows, with_abs=True)
        check_fp(host_f64(out)[rows], ref, absref, K, "bf16", f"noalloc M={M} {name}/{splits}")
    if N == 2048:
        # these shapes split K in the shipped table: the scratch array is used
        assert max(splits_seen) > 1, splits_seen


def test_noalloc_refuses_partials_beyond_the_array(qll, tmp_path):
    # a table whose entry splits K eight ways at M = 2048, N = 4096: 256 MiB
    # of partials, more than the 16 MiB array -> QLL_ERR_WORKSPACE, nothing
    # enqueued (the output keeps its contents)
    t = tmp_path / "t.tsv"
    t.write_text(f"device {qll.device_signature()}\n"
                 "fp8 4096 2048 2048 p128x128_w2x2_k128_s2 8\n")
    M, N, K = 2048, 4096, 2048
    try:
        assert qll.init(str(t)) == 0 and qll.select("fp8", M, N, K)[1] == 8
        q = torch.zeros((M, K), dtype=torch.float8_e4m3fn, device="cuda")
        B = torch.zeros((N, K), dtype=torch.float8_e4m3fn, device="cuda")
        sa = torch.ones(M, device="cuda")
        sb = torch.ones(N, device="cuda")
        out = torch.full((M, N), 3.0, dtype=torch.bfloat16, device="cuda")
        assert call_noalloc(qll, q, B, sa, sb, out, M, N, K) == 4
        torch.cuda.synchronize()
        assert bool((out == 3.0).all())
    finally:
        qll.init()

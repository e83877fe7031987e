"""GPU parity of the FP8 quantizers: codes and scale bits bit-exact against
the oracle (the codes are an encoding, so exactly one result is correct).

Operation: "FP8 dynamic quantization" / "Block-FP8" of "Helion in vLLM: A
Unified Route to Tunable Linear Kernels", section "What the integration
changes"; rule s = absmax / 448, q = e4m3_rne(clamp(x / s)).
"""
import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def qll():
    import quantized_linear_layer_scaled_amd as q
    q.load_library()
    return q


def run_quant(qll, x_bits, group=None):
    from gpu_util import dev_bf16, host_codes
    q, s = qll.quantize_per_token_fp8(dev_bf16(x_bits), group=group)
    torch.cuda.synchronize()
    return host_codes(q), s.cpu().numpy()


def assert_same(q, s, qr, sr, what):
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32)), f"{what}: scales differ"
    if not np.array_equal(q, qr):
        bad = np.argwhere(q != qr)
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} codes differ, first at {i}: "
                             f"gpu {q[i]:#04x} oracle {qr[i]:#04x}")


# K spans every row-kernel shape: 64, 128 and 256 threads per row, one to
# sixteen 16-byte chunks per thread, and the two-pass kernel past 32768; more
# than 512 rows of 2048..8192 take the row loop (one to four chunks, a ragged
# K tail, workgroups with an odd number of rows); 512 rows and more of up to
# 2048 elements (2048 rows and more of up to 4096) take one wave per row (one
# to eight chunks per lane, ragged K tails, a partial last workgroup)
@pytest.mark.parametrize("M,K", [(1, 16), (4, 608), (9, 1024), (301, 1040), (3, 2048),
                                 (5, 6144), (2048, 2048), (7, 4112), (2, 16400),
                                 (64, 20000), (3, 32768), (2, 40000),
                                 (2048, 6144), (1500, 4112), (513, 8192), (1025, 2064),
                                 (512, 16), (600, 1040), (777, 2048), (2048, 4096),
                                 (2101, 3088), (4096, 2048), (2050, 2576)])
def test_per_token_bit_exact(qll, M, K):
    x = workloads.bf16_normal((M, K), (workloads.W_TEST, 20, M, K), outlier_frac=0.01)
    q, s = run_quant(qll, x)
    qr, sr = oracle.quantize_fp8(x)
    assert_same(q, s, qr, sr, f"per-token M={M} K={K}")


@pytest.mark.parametrize("M,K", [(1, 128), (5, 2048), (2048, 6144), (33, 1152)])
def test_group128_bit_exact(qll, M, K):
    x = workloads.bf16_normal((M, K), (workloads.W_TEST, 21, M, K))
    q, s = run_quant(qll, x, group=128)
    qr, sr = oracle.quantize_fp8(x, group=128)
    assert_same(q, s, qr, sr, f"group128 M={M} K={K}")


def test_golden_examples_on_gpu(qll, golden):
    for x_hex, s_hex, q_hex in golden("quantizer_examples.txt"):
        x = np.array([int(t, 16) for t in x_hex.split()], np.uint16)
        n = x.size
        row = np.zeros((1, 16), np.uint16)  # K must be a multiple of 16
        row[0, :n] = x
        q, s = run_quant(qll, row)
        assert s.view(np.uint32)[0, 0] == int(s_hex, 16), x_hex
        ref = [int(t, 16) for t in q_hex.split()]
        assert q[0, :n].tolist() == ref, (x_hex, q[0, :n])
        assert np.all(q[0, n:] == 0)


# the edge rows repeated over enough rows to take the many-row kernels: one
# wave per row (512+ rows of <= 2048 elements, 2048+ rows of <= 4096) and
# the row loop (513+ rows of 2048..8192 elements)
@pytest.mark.parametrize("M,K", [(600, 256), (520, 1040), (2048, 4096), (530, 6144)])
def test_edge_values_many_rows_bit_exact(qll, M, K):
    from gpu_util import edge_rows
    e = edge_rows(K)
    x = workloads.bf16_normal((M, K), (workloads.W_TEST, 24, M, K))
    x[::3] = e[np.arange(0, M, 3) % len(e)]
    q, s = run_quant(qll, x)
    qr, sr = oracle.quantize_fp8(x)
    assert_same(q, s, qr, sr, f"edge rows M={M} K={K}")


def test_edge_values_bit_exact(qll):
    # zeros, signed zeros, tiny values that round to +-0, subnormal ties,
    # bf16 subnormals, values at the clamp, an all-zero row
    K = 256
    g = np.random.default_rng(22)
    rows = []
    r = np.zeros(K, np.uint16)
    rows.append(r.copy())                            # all zero
    r[:] = 0x8000
    rows.append(r.copy())                            # all -0.0
    big = workloads.to_bf16_bits(np.float32([448.0]))[0]
    # scales on both sides of the reciprocal path's range of s, [2^-64, 2^64]
    for scale in (1.0, 1e-3, 2.0**-55, 2.0**-58, 2.0**-61, 1e-30, 2.0**68, 2.0**71, 1e37):
        v = (g.standard_normal(K) * scale).astype(np.float32)
        v[::7] *= np.float32(1e-6)
        b = workloads.to_bf16_bits(v)
        b[0] = big if scale == 1.0 else b[0]
        rows.append(b)
    sub = np.arange(1, K + 1, dtype=np.uint16) & 0x7F    # bf16 subnormals
    sub[1::2] |= 0x8000
    rows.append(sub)
    x = np.stack(rows)
    q, s = run_quant(qll, x)
    qr, sr = oracle.quantize_fp8(x)
    assert_same(q, s, qr, sr, "edge rows")
    q, s = run_quant(qll, x, group=128)
    qr, sr = oracle.quantize_fp8(x, group=128)
    assert_same(q, s, qr, sr, "edge groups")


@pytest.mark.parametrize("N,K", [(256, 2048), (300, 384), (12288, 2048), (2048, 6144)])
def test_weight_blocks_bit_exact(qll, N, K):
    from gpu_util import dev_bf16, host_codes
    w = workloads.bf16_normal((N, K), (workloads.W_TEST, 23, N, K), std=0.02)
    q, s = qll.quantize_weight_block_fp8(dev_bf16(w))
    torch.cuda.synchronize()
    qr, sr = oracle.quantize_fp8_block(w)
    assert_same(host_codes(q), s.cpu().numpy(), qr, sr, f"weight blocks N={N} K={K}")


def test_zero_rows_is_noop(qll):
    x = torch.empty((0, 2048), dtype=torch.bfloat16, device="cuda")
    q, s = qll.quantize_per_token_fp8(x)
    assert q.shape == (0, 2048) and s.shape == (0, 1)

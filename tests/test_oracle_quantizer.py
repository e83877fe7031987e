"""Pins of the oracle's dynamic FP8 quantizers.

Operation: "FP8 dynamic quantization" and "Block-FP8" of the page "Helion in
vLLM: A Unified Route to Tunable Linear Kernels" (section "What the
integration changes"), with s = absmax / 448 and q = e4m3_rne(clamp(x/s)).

Pins: hand-worked fixtures (tests/golden/quantizer_examples.txt), torch's own
e4m3 cast applied to torch-computed scales, structural identities (a 1x128
group quantizes like a row of its own; a 128x128 weight block like one
flattened row) and invariants (the amax element hits +-448, signs survive,
the rounding error stays inside half an e4m3 step).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads


def parse_hex_list(s, dtype):
    return np.array([int(t, 16) for t in s.split()], dtype=dtype)


def test_golden_examples(golden):
    rows = golden("quantizer_examples.txt")
    assert len(rows) >= 6
    for x_hex, s_hex, q_hex in rows:
        x = parse_hex_list(x_hex, np.uint16)[None, :]
        s_bits = np.uint32(int(s_hex, 16))
        q_ref = parse_hex_list(q_hex, np.uint8)
        q, s = oracle.quantize_fp8(x)
        assert s.shape == (1, 1)
        assert s.view(np.uint32)[0, 0] == s_bits, (x_hex, hex(s.view(np.uint32)[0, 0]))
        assert np.array_equal(q[0], q_ref), (x_hex, q[0])


def torch_quantize_rows(x_bits):
    """Quantize rows with torch CPU ops: fp32 absmax, fp32 division, clamp,
    torch's e4m3fn cast."""
    x = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16)
    x = x.to(torch.float32)
    amax = x.abs().amax(dim=1, keepdim=True)
    s = amax / torch.tensor(448.0, dtype=torch.float32)
    safe = torch.where(s == 0, torch.ones_like(s), s)
    v = torch.clamp(x / safe, -448.0, 448.0)
    q = v.to(torch.float8_e4m3fn).view(torch.uint8)
    q = torch.where(s == 0, torch.zeros_like(q), q)
    return q.numpy(), s[:, 0].numpy()


@pytest.mark.parametrize("M,K", [(7, 2048), (33, 6144), (5, 128), (3, 16)])
def test_per_token_matches_torch_ops(M, K):
    x = workloads.bf16_normal((M, K), (workloads.W_TEST, M, K), outlier_frac=0.01)
    q, s = oracle.quantize_fp8(x)
    q_ref, s_ref = torch_quantize_rows(x)
    assert np.array_equal(s[:, 0].view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)


def test_group_128_equals_rows_of_128():
    M, K = 9, 1024
    x = workloads.bf16_normal((M, K), (workloads.W_TEST, 1), outlier_frac=0.01)
    q, s = oracle.quantize_fp8(x, group=128)
    q2, s2 = oracle.quantize_fp8(x.reshape(M * K // 128, 128))
    assert s.shape == (M, K // 128)
    assert np.array_equal(s.reshape(-1).view(np.uint32), s2[:, 0].view(np.uint32))
    assert np.array_equal(q.reshape(-1), q2.reshape(-1))


@pytest.mark.parametrize("N,K", [(256, 256), (300, 384)])
def test_weight_blocks_equal_flattened_blocks(N, K):
    w = workloads.bf16_normal((N, K), (workloads.W_TEST, 2, N), std=0.02)
    q, s = oracle.quantize_fp8_block(w)
    nb, kb = (N + 127) // 128, K // 128
    assert s.shape == (nb, kb)
    for i in range(nb):
        for j in range(kb):
            blk = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            qb, sb = oracle.quantize_fp8(np.ascontiguousarray(blk).reshape(1, -1))
            assert sb[0, 0].view(np.uint32) == s[i, j].view(np.uint32)
            assert np.array_equal(
                q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128].reshape(-1), qb[0])


def test_invariants_on_outlier_rows():
    M, K = 64, 2048
    x = workloads.bf16_normal((M, K), (workloads.W_TEST, 3), outlier_frac=0.01)
    xf = oracle.bf16_decode(x).astype(np.float64)
    q, s = oracle.quantize_fp8(x)
    dq = oracle.e4m3_decode(q)
    s64 = s.astype(np.float64)
    for m in range(M):
        i = np.argmax(np.abs(xf[m]))
        assert q[m, i] in (0x7E, 0xFE)
    nz = xf != 0
    # the sign bit of every code is the sign of its input (zero keeps its sign)
    assert np.array_equal((q >> 7).astype(bool)[nz], np.signbit(xf[nz]))
    # rounding error: half a step of e4m3 relative to |x/s| (normal range:
    # 2^-4 |v|; subnormal range: 2^-10), plus one fp32 rounding of x/s
    v = xf / s64
    err = np.abs(dq - v)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10) + np.abs(v) * 2.0 ** -23
    assert np.all(err <= bound)


def test_zero_row_and_rejects_nonfinite():
    x = np.zeros((2, 256), dtype=np.uint16)
    x[1, 5] = 0x8000  # -0.0
    q, s = oracle.quantize_fp8(x)
    assert np.all(s == 0) and np.all(q == 0)
    bad = np.zeros((1, 16), dtype=np.uint16)
    bad[0, 3] = 0x7F80  # +inf
    with pytest.raises(ValueError):
        oracle.quantize_fp8(bad)

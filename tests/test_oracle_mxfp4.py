"""Pins of the oracle's MXFP4 functions against things other than the oracle:
the E2M1 value set of the OCP Microscaling (MX) v1.0 specification, torch's
own E8M0 cast, exact brute force with Python Fractions (independent decoding
and nibble unpacking written here), a numpy matmul for the special case of
unit scales, and round trips of values the format holds exactly.

Readings these tests fix (the pages name 4-bit formats but define none):
  * element 2j of a row sits in bits 0-3 of byte j, element 2j+1 in bits 4-7;
  * shared exponent floor(log2(amax)) - 2, clamped to [-127, 127]; an
    all-zero block takes -127;
  * element codes round to nearest, ties to even, and saturate at 6; the sign
    bit follows the input's sign also when the magnitude rounds to zero.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

# E2M1 magnitudes of codes 0..7 (the format's value table: subnormal 0.5,
# normals 1, 1.5, 2, 3, 4, 6); codes 8..15 are their negatives.
E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
        Fraction(3), Fraction(4), Fraction(6)]


def dec(code):
    mag = E2M1[code & 7]
    return -mag if code & 8 else mag


def nearest_code(v: Fraction, negative: bool) -> int:
    """Brute force: the magnitude code nearest to |v| (ties to an even code,
    above 6 -> 6), with the sign bit from `negative`."""
    a = abs(v)
    best = min(range(8), key=lambda c: (abs(E2M1[c] - a), c & 1))
    return best | (8 if negative else 0)


def nibbles(row_bytes):
    out = []
    for b in row_bytes:
        out.append(int(b) & 15)
        out.append(int(b) >> 4)
    return out


def bf16_bits(x):
    """float32 values that are exactly bf16 -> their bit patterns."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all(u & 0xFFFF == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def test_e2m1_value_table():
    got = oracle.e2m1_decode(np.arange(16))
    want = [float(dec(c)) for c in range(16)]
    assert got.tolist() == want
    assert np.signbit(got[8])            # code 8 is -0
    assert not np.signbit(got[0])


def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e8m0_decode(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


def test_e2m1_encode_ties_and_saturation():
    v = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.0, 100.0, 0.0, -0.0, -0.2, -5.5]
    want = [0, 2, 2, 4, 4, 6, 6, 7, 7, 7, 0, 8, 8, 15]
    assert oracle.e2m1_encode(v).tolist() == want


def test_e2m1_encode_brute_force():
    rng = np.random.default_rng(5)
    grid = [j / 64 for j in range(-640, 641)]
    vals = np.array(grid + list(rng.uniform(-9, 9, 2000)), dtype=np.float64)
    got = oracle.e2m1_encode(vals)
    for v, c in zip(vals.tolist(), got.tolist()):
        assert c == nearest_code(Fraction(v), np.signbit(v)), v


def test_quantize_round_trip_exact_values():
    """Blocks built from codes whose largest magnitude is 4 or 6 times 2^t come
    back with the same codes and scale code t + 127."""
    rng = np.random.default_rng(11)
    M, K = 6, 128
    codes = rng.integers(0, 16, size=(M, K))
    t = rng.integers(-120, 121, size=(M, K // 32))
    for m in range(M):
        for b in range(K // 32):
            codes[m, b * 32 + rng.integers(0, 32)] = rng.choice([6, 7, 14, 15])
    x = np.empty((M, K), dtype=np.float32)
    for m in range(M):
        for k in range(K):
            v = float(dec(int(codes[m, k])) * Fraction(2) ** int(t[m, k // 32]))
            x[m, k] = -0.0 if codes[m, k] == 8 else v   # Fraction has no -0
    q, s = oracle.quantize_mxfp4(bf16_bits(x))
    assert s.tolist() == (t + 127).tolist()
    got = np.array([nibbles(r) for r in q])
    # zeros come back with the input's sign: code 8 stays 8, code 0 stays 0
    assert got.tolist() == codes.tolist()


def test_quantize_brute_force_random_rows():
    """Every block: the scale is the power of two X with 4 <= amax / X < 8
    (unless the lower clamp applies), and every code is the nearest E2M1
    value to x / X (brute force, saturating)."""
    rng = np.random.default_rng(3)
    M, K = 5, 96
    x = (rng.standard_normal((M, K)) * np.exp2(rng.integers(-30, 30, (M, 1)))).astype(np.float32)
    x[1, 32:64] = 0.0                       # an all-zero block
    x[2, 0:32] = np.float32(2.0 ** -130)    # subnormal bf16 block
    x[2, 5] = -np.float32(2.0 ** -128)
    xb = bf16_bits((x.view(np.uint32) & 0xFFFF0000).view(np.float32))
    xv = (xb.astype(np.uint32) << 16).view(np.float32)
    q, s = oracle.quantize_mxfp4(xb)
    assert q.shape == (M, K // 2) and s.shape == (M, K // 32)
    for m in range(M):
        codes = nibbles(q[m])
        for b in range(K // 32):
            blk = [Fraction(float(v)) for v in xv[m, b * 32:(b + 1) * 32]]
            amax = max(abs(v) for v in blk)
            X = Fraction(2) ** (int(s[m, b]) - 127)
            if amax == 0:
                assert s[m, b] == 0
            elif s[m, b] > 0:
                assert 4 <= amax / X < 8
            else:
                assert amax / X < 8
            for i, v in enumerate(blk):
                neg = bool(np.signbit(xv[m, b * 32 + i]))
                assert codes[b * 32 + i] == nearest_code(v / X, neg), (m, b, i)
    assert s[2, 0] == 0 and s[1, 1] == 0


def test_quantize_error_bound():
    """|x - dequant| stays below twice the block's scale (half the widest
    spacing, 2 between 4 and 6, below 6; saturation above it costs < 2)."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    xb = bf16_bits((x.view(np.uint32) & 0xFFFF0000).view(np.float32))
    xv = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    q, s = oracle.quantize_mxfp4(xb)
    deq = oracle.e2m1_decode(oracle.unpack_fp4(q)) * np.repeat(
        oracle.e8m0_decode(s), 32, axis=1)
    X = np.repeat(oracle.e8m0_decode(s), 32, axis=1)
    assert np.all(np.abs(xv - deq) < 2 * X)


def test_gemm_brute_force_fractions():
    rng = np.random.default_rng(17)
    M, N, K = 3, 5, 96
    A = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    B = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sa = rng.integers(118, 137, size=(M, K // 32), dtype=np.uint8)
    sb = rng.integers(118, 137, size=(N, K // 32), dtype=np.uint8)
    ref, absref = oracle.gemm_mxfp4(A, B, sa, sb, with_abs=True)
    for m in range(M):
        a = nibbles(A[m])
        for n in range(N):
            b = nibbles(B[n])
            tot = Fraction(0)
            atot = Fraction(0)
            for k in range(K):
                p = (dec(a[k]) * Fraction(2) ** (int(sa[m, k // 32]) - 127) *
                     dec(b[k]) * Fraction(2) ** (int(sb[n, k // 32]) - 127))
                tot += p
                atot += abs(p)
            assert ref[m, n] == float(tot)
            assert absref[m, n] == float(atot)


def test_gemm_unit_scales_is_a_plain_matmul():
    rng = np.random.default_rng(21)
    M, N, K = 7, 9, 256
    A = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    B = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    ones_a = np.full((M, K // 32), 127, dtype=np.uint8)
    ones_b = np.full((N, K // 32), 127, dtype=np.uint8)
    table = np.array([float(dec(c)) for c in range(16)])
    Ad = table[np.array([nibbles(r) for r in A])]
    Bd = table[np.array([nibbles(r) for r in B])]
    assert np.array_equal(oracle.gemm_mxfp4(A, B, ones_a, ones_b), Ad @ Bd.T)
    # one block's scale code + 1 doubles exactly that block's contribution
    sa = ones_a.copy()
    sa[:, 1] = 128
    want = Ad @ Bd.T + Ad[:, 32:64] @ Bd[:, 32:64].T
    assert np.array_equal(oracle.gemm_mxfp4(A, B, sa, ones_b), want)


def test_gemm_rows_subset():
    rng = np.random.default_rng(2)
    M, N, K = 10, 4, 128
    A = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    B = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    sa = rng.integers(120, 130, size=(M, K // 32), dtype=np.uint8)
    sb = rng.integers(120, 130, size=(N, K // 32), dtype=np.uint8)
    full = oracle.gemm_mxfp4(A, B, sa, sb)
    rows = [9, 0, 4]
    assert np.array_equal(oracle.gemm_mxfp4(A, B, sa, sb, rows=rows), full[rows])


def test_quantize_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.quantize_mxfp4(np.zeros((2, 48), dtype=np.uint16))

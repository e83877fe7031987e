"""Pins of the oracle's INT4 weight-only functions against things other than
the oracle: the two's complement closed form, numpy's IEEE float32 division
plus a brute-force nearest-integer search, exact round trips, the half-step
error bound, Fraction brute force of the GEMM (own nibble unpacking and bf16
decoding written here), and numpy matmuls for the unit-scale case.

Readings these tests fix (the pages name INT4 without defining it):
  * signed 4-bit two's complement codes, element 2j of a row in bits 0-3 of
    byte j, element 2j+1 in bits 4-7;
  * one fp32 scale per output channel and 128-element K group,
    s = amax / 7 (fp32), q = clamp(rne(fl32(w / s)), -8, 7), s = 0 and zero
    codes for an all-zero group;
  * out = sum over groups of s * (exact group partial sum), bf16 activations.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def i4(c):
    c = int(c) & 15
    return c - 16 if c >= 8 else c


def nibbles(row_bytes):
    out = []
    for b in row_bytes:
        out.append(int(b) & 15)
        out.append(int(b) >> 4)
    return out


def bf16_value(bits):
    return float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0])


def bf16_bits(x):
    u = np.asarray(x, dtype=np.float32).view(np.uint32)
    assert np.all(u & 0xFFFF == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def test_int4_decode_twos_complement():
    got = oracle.int4_decode(np.arange(16)).tolist()
    assert got == [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]


def test_quantize_round_trip():
    """Groups holding q * 2^t with some |q| = 7 come back exactly."""
    rng = np.random.default_rng(4)
    N, K = 5, 256
    q = rng.integers(-7, 8, size=(N, K))
    t = rng.integers(-20, 20, size=(N, K // 128))
    for n in range(N):
        for g in range(K // 128):
            q[n, g * 128 + rng.integers(0, 128)] = rng.choice([-7, 7])
    w = (q * np.exp2(np.repeat(t, 128, axis=1))).astype(np.float32)
    codes, s = oracle.quantize_int4(bf16_bits(w))
    assert np.array_equal(s, np.exp2(t).astype(np.float32))
    got = np.array([[i4(c) for c in nibbles(r)] for r in codes])
    assert np.array_equal(got, q)


def test_quantize_ties_to_even():
    """A group with amax = 7 * 2^-3 makes w / s exact: halves round to the
    even neighbour (0.5 -> 0, 1.5 -> 2, 2.5 -> 2, 6.5 -> 6, and negatives)."""
    K = 128
    t = 2.0 ** -3
    vals = [7, 0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5, -0.5, -1.5, -2.5, -6.5, -7, 0.25, 0.75]
    want = [7, 0, 2, 2, 4, 4, 6, 6, 0, -2, -2, -6, -7, 0, 1]
    w = np.zeros((1, K), np.float32)
    w[0, :len(vals)] = np.array(vals, np.float32) * np.float32(t)
    codes, s = oracle.quantize_int4(bf16_bits(w))
    assert s[0, 0] == np.float32(t)
    got = [i4(c) for c in nibbles(codes[0])][:len(vals)]
    assert got == want


def test_quantize_brute_force():
    """s equals numpy's float32 amax / 7; every code is the integer in
    [-8, 7] nearest to numpy's float32 quotient w / s (ties to even); an
    all-zero group has s = 0 and zero codes; |w - q s| <= s / 2."""
    rng = np.random.default_rng(8)
    N, K = 4, 384
    w = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-12, 4, (N, 1)))).astype(np.float32)
    w[2, 128:256] = 0.0
    wb = bf16_bits((w.view(np.uint32) & 0xFFFF0000).view(np.float32))
    wv = (wb.astype(np.uint32) << 16).view(np.float32)
    codes, s = oracle.quantize_int4(wb)
    assert codes.shape == (N, K // 2) and s.shape == (N, K // 128)
    for n in range(N):
        c = nibbles(codes[n])
        for g in range(K // 128):
            blk = wv[n, g * 128:(g + 1) * 128]
            amax = np.max(np.abs(blk))
            sg = np.float32(amax) / np.float32(7.0)
            assert s[n, g] == sg
            for i, x in enumerate(blk):
                code = i4(c[g * 128 + i])
                if sg == 0:
                    assert code == 0
                    continue
                v = Fraction(float(np.float32(x) / sg))
                best = min(range(-8, 8), key=lambda k: (abs(v - k), k & 1))
                assert code == best, (n, g, i)
                assert abs(Fraction(float(x)) - code * Fraction(float(sg))) <= \
                    Fraction(float(sg)) / 2 * (1 + Fraction(1, 1 << 20))
    assert np.all(s[2, 1] == 0)


def test_gemm_brute_force_fractions():
    rng = np.random.default_rng(13)
    M, N, K = 3, 4, 256
    A = bf16_bits((rng.standard_normal((M, K)).astype(np.float32).view(np.uint32)
                   & 0xFFFF0000).view(np.float32))
    B = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = rng.uniform(1e-3, 1e-1, size=(N, K // 128)).astype(np.float32)
    ref, absref = oracle.gemm_w4a16(A, B, s, with_abs=True)
    for m in range(M):
        a = [Fraction(bf16_value(x)) for x in A[m]]
        for n in range(N):
            b = [i4(c) for c in nibbles(B[n])]
            tot = Fraction(0)
            atot = Fraction(0)
            for g in range(K // 128):
                pg = sum(a[k] * b[k] for k in range(g * 128, (g + 1) * 128))
                apg = sum(abs(a[k] * b[k]) for k in range(g * 128, (g + 1) * 128))
                tot += Fraction(float(s[n, g])) * pg
                atot += Fraction(float(s[n, g])) * apg
            assert abs(Fraction(ref[m, n]) - tot) <= abs(tot) * Fraction(1, 1 << 50) + Fraction(1, 1 << 100)
            assert abs(Fraction(absref[m, n]) - atot) <= atot * Fraction(1, 1 << 50)


def test_gemm_unit_scales_is_a_plain_matmul():
    rng = np.random.default_rng(23)
    M, N, K = 6, 5, 384
    Ai = rng.integers(-64, 65, size=(M, K)).astype(np.float32)   # exact in bf16
    A = bf16_bits(Ai)
    B = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    Bi = np.array([[i4(c) for c in nibbles(r)] for r in B], dtype=np.float64)
    ones = np.ones((N, K // 128), dtype=np.float32)
    assert np.array_equal(oracle.gemm_w4a16(A, B, ones), Ai.astype(np.float64) @ Bi.T)
    # doubling one group's scales adds exactly that group's contribution
    s2 = ones.copy()
    s2[:, 2] = 2.0
    want = Ai.astype(np.float64) @ Bi.T + Ai[:, 256:384].astype(np.float64) @ Bi[:, 256:384].T
    assert np.array_equal(oracle.gemm_w4a16(A, B, s2), want)


def test_gemm_rows_subset():
    rng = np.random.default_rng(3)
    M, N, K = 9, 4, 128
    A = bf16_bits(rng.integers(-8, 9, size=(M, K)).astype(np.float32))
    B = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = rng.uniform(0.5, 2.0, size=(N, 1)).astype(np.float32)
    full = oracle.gemm_w4a16(A, B, s)
    rows = [8, 1, 4]
    assert np.array_equal(oracle.gemm_w4a16(A, B, s, rows=rows), full[rows])


def test_quantize_rejects_bad_k():
    with pytest.raises(ValueError):
        oracle.quantize_int4(np.zeros((2, 64), dtype=np.uint16))

"""Pins of the oracle's GEMMs against Python integer / Fraction brute force,
numpy fp64 products of torch-decoded operands, closed forms and the
hand-worked epilogue fixture.

Operations: W8A8 INT8, FP8 dynamic (per-token x per-channel scales) and
Block-FP8 of "Helion in vLLM: A Unified Route to Tunable Linear Kernels"
(section "What the integration changes"); the bf16 product of the
batch-invariant matmul of vLLM PR #53446 ("Summary").  Shapes are never square
so that a transposed operand or a swapped index fails.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads


def torch_dec_e4m3(c):
    return torch.from_numpy(np.asarray(c, np.uint8).copy()).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def torch_dec_bf16(b):
    return torch.from_numpy(np.asarray(b, np.uint16).view(np.int16).copy()).view(
        torch.bfloat16).to(torch.float64).numpy()


def rand_e4m3(shape, g):
    c = g.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    return c


# ---------------------------------------------------------------- INT8
@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (6, 4, 40), (2, 7, 64)])
def test_int8_acc_bruteforce(M, N, K):
    g = np.random.default_rng([M, N, K])
    A = g.integers(-128, 128, size=(M, K), dtype=np.int8)
    B = g.integers(-128, 128, size=(N, K), dtype=np.int8)
    acc = oracle.gemm_int8_acc(A, B)
    for m in range(M):
        for n in range(N):
            assert acc[m, n] == sum(int(A[m, k]) * int(B[n, k]) for k in range(K))


def test_int8_closed_forms():
    K = 2048
    ones = np.ones((3, K), np.int8)
    assert np.all(oracle.gemm_int8_acc(ones, np.ones((5, K), np.int8)) == K)
    A = np.full((2, K), 127, np.int8)
    B = np.full((4, K), -127, np.int8)
    assert np.all(oracle.gemm_int8_acc(A, B) == -16129 * K)
    A = np.full((1, K), -128, np.int8)
    assert np.all(oracle.gemm_int8_acc(A, A) == 16384 * K)
    # B = identity (N = K): acc = A
    Kc = 96
    A = np.random.default_rng(1).integers(-127, 128, (5, Kc), dtype=np.int8)
    acc = oracle.gemm_int8_acc(A, np.eye(Kc, dtype=np.int8))
    assert np.array_equal(acc, A.astype(np.int64))


def test_int8_matches_numpy_and_rows():
    d = workloads.int8_inputs(M=37, N=53, K=304, key=(workloads.W_TEST, 4))
    acc = oracle.gemm_int8_acc(d["A"], d["B"])
    ref = d["A"].astype(np.int64) @ d["B"].astype(np.int64).T
    assert np.array_equal(acc, ref)
    rows = [36, 0, 17]
    assert np.array_equal(oracle.gemm_int8_acc(d["A"], d["B"], rows), ref[rows])


def test_int8_epilogue_golden(golden):
    for lhs, rhs in golden("int8_epilogue_examples.txt"):
        a, sa_h, sb_h = lhs.split()
        y_h, b_h = rhs.split()
        acc = np.array([[int(a)]], np.int64)
        sa = np.array([int(sa_h, 16)], np.uint32).view(np.float32)
        sb = np.array([int(sb_h, 16)], np.uint32).view(np.float32)
        y = oracle.epilogue_int8(acc, sa, sb)
        assert y.view(np.uint32)[0, 0] == int(y_h, 16)
        assert oracle.bf16_encode(y)[0, 0] == int(b_h, 16)


def test_int8_epilogue_order_is_left_to_right():
    # the two fp32 products are rounded separately, sa first
    g = np.random.default_rng(5)
    acc = g.integers(-3_000_000, 3_000_000, size=(64, 48)).astype(np.int64)
    sa = g.uniform(1e-3, 1e-2, 64).astype(np.float32)
    sb = g.uniform(1e-3, 1e-2, 48).astype(np.float32)
    y = oracle.epilogue_int8(acc, sa, sb)
    exact = [[Fraction(int(acc[m, n])) * Fraction(float(sa[m])) for n in range(48)]
             for m in range(64)]
    # fp32(fp32(acc*sa)*sb) via Fraction rounding with numpy's float32 rounding
    t = np.array([[np.float32(float(exact[m][n])) for n in range(48)]
                  for m in range(64)], np.float32)
    assert np.array_equal(y, (t * sb[None, :]).astype(np.float32))


# ---------------------------------------------------------------- FP8
@pytest.mark.parametrize("M,N,K", [(2, 3, 5), (4, 3, 33), (1, 6, 128)])
def test_fp8_fraction_bruteforce(M, N, K):
    g = np.random.default_rng([7, M, N, K])
    A, B = rand_e4m3((M, K), g), rand_e4m3((N, K), g)
    sa = g.uniform(1e-4, 1e-1, M).astype(np.float32)
    sb = g.uniform(1e-4, 1e-1, N).astype(np.float32)
    ref, absref = oracle.gemm_fp8(A, B, sa, sb, with_abs=True)
    da, db = torch_dec_e4m3(A), torch_dec_e4m3(B)
    for m in range(M):
        for n in range(N):
            s = sum(Fraction(da[m, k]) * Fraction(db[n, k]) for k in range(K))
            ex = Fraction(float(sa[m])) * Fraction(float(sb[n])) * s
            assert ref[m, n] == float(ex)
            aex = abs(Fraction(float(sa[m])) * Fraction(float(sb[n]))) * sum(
                abs(Fraction(da[m, k]) * Fraction(db[n, k])) for k in range(K))
            assert absref[m, n] == float(aex)


def test_fp8_grouped_fraction_bruteforce():
    # three experts, one of them empty; rows sorted by expert
    g = np.random.default_rng([17])
    counts = [2, 0, 3]
    off = np.concatenate([[0], np.cumsum(counts)])
    M, N, K, E = int(off[-1]), 4, 24, 3
    A, B = rand_e4m3((M, K), g), rand_e4m3((E, N, K), g)
    sa = g.uniform(1e-3, 1e-1, M).astype(np.float32)
    sb = g.uniform(1e-3, 1e-1, (E, N)).astype(np.float32)
    ref, absref = oracle.gemm_fp8_grouped(A, B, sa, sb, off, with_abs=True)
    da, db = torch_dec_e4m3(A), torch_dec_e4m3(B)
    owner = [0, 0, 2, 2, 2]
    for m in range(M):
        e = owner[m]
        for n in range(N):
            s = sum(Fraction(da[m, k]) * Fraction(db[e, n, k]) for k in range(K))
            assert ref[m, n] == float(Fraction(float(sa[m])) * Fraction(float(sb[e, n])) * s)
            aex = abs(Fraction(float(sa[m])) * Fraction(float(sb[e, n]))) * sum(
                abs(Fraction(da[m, k]) * Fraction(db[e, n, k])) for k in range(K))
            assert absref[m, n] == float(aex)
    # sampled rows give the same values as the full product
    rows = [4, 0, 3]
    assert np.array_equal(oracle.gemm_fp8_grouped(A, B, sa, sb, off, rows=rows), ref[rows])


def test_fp8_grouped_single_expert_is_the_dense_product():
    g = np.random.default_rng([18])
    M, N, K = 7, 5, 40
    A, B = rand_e4m3((M, K), g), rand_e4m3((1, N, K), g)
    sa = g.uniform(1e-3, 1e-1, M).astype(np.float32)
    sb = g.uniform(1e-3, 1e-1, (1, N)).astype(np.float32)
    dense = oracle.gemm_fp8(A, B[0], sa, sb[0])
    assert np.array_equal(oracle.gemm_fp8_grouped(A, B, sa, sb, [0, M]), dense)


def test_fp8_matches_numpy_dequantized():
    g = np.random.default_rng(8)
    M, N, K = 19, 41, 512
    A, B = rand_e4m3((M, K), g), rand_e4m3((N, K), g)
    sa = g.uniform(1e-3, 1e-2, M).astype(np.float32)
    sb = g.uniform(1e-3, 1e-2, N).astype(np.float32)
    ref = oracle.gemm_fp8(A, B, sa, sb)
    npref = (torch_dec_e4m3(A) @ torch_dec_e4m3(B).T) * sa[:, None].astype(
        np.float64) * sb[None, :].astype(np.float64)
    np.testing.assert_allclose(ref, npref, rtol=1e-12, atol=1e-300)
    assert np.array_equal(oracle.gemm_fp8(A, B, sa, sb, rows=[18, 3]), ref[[18, 3]])


def test_fp8_integer_valued_equals_int8():
    # integers in [-16, 16] are exact in e4m3; with unit scales the fp8
    # product must equal the INT8 product of the same integers
    g = np.random.default_rng(9)
    M, N, K = 8, 24, 256
    ia = g.integers(-16, 17, (M, K)).astype(np.int8)
    ib = g.integers(-16, 17, (N, K)).astype(np.int8)
    A = oracle.e4m3_encode(ia.astype(np.float32))
    B = oracle.e4m3_encode(ib.astype(np.float32))
    ref = oracle.gemm_fp8(A, B, np.ones(M, np.float32), np.ones(N, np.float32))
    assert np.array_equal(ref, oracle.gemm_int8_acc(ia, ib).astype(np.float64))


# ---------------------------------------------------------------- Block-FP8
def test_block_fp8_fraction_bruteforce_edge_block():
    g = np.random.default_rng(10)
    M, N, K = 3, 130, 256  # N has a partial last 128-block, K two groups
    A, B = rand_e4m3((M, K), g), rand_e4m3((N, K), g)
    sa = g.uniform(1e-3, 1.0, (M, 2)).astype(np.float32)
    sb = g.uniform(1e-3, 1.0, (2, 2)).astype(np.float32)
    ref = oracle.gemm_block_fp8(A, B, sa, sb)
    da, db = torch_dec_e4m3(A), torch_dec_e4m3(B)
    for m in range(M):
        for n in [0, 1, 64, 127, 128, 129]:
            ex = Fraction(0)
            for gi in range(2):
                pg = sum(Fraction(da[m, k]) * Fraction(db[n, k])
                         for k in range(128 * gi, 128 * gi + 128))
                ex += Fraction(float(sa[m, gi])) * Fraction(float(sb[n // 128, gi])) * pg
            assert abs(ref[m, n] - float(ex)) <= 2.0 ** -50 * abs(float(ex)) + 1e-300


def test_block_fp8_reduces_to_per_channel():
    g = np.random.default_rng(11)
    M, N, K = 5, 384, 512
    A, B = rand_e4m3((M, K), g), rand_e4m3((N, K), g)
    ra = g.uniform(1e-3, 1e-2, M).astype(np.float32)
    rb = g.uniform(1e-3, 1e-2, N // 128).astype(np.float32)
    sa = np.repeat(ra[:, None], K // 128, axis=1)
    sb = np.repeat(rb[:, None], K // 128, axis=1)
    blk = oracle.gemm_block_fp8(A, B, sa, sb)
    chan, absref = oracle.gemm_fp8(A, B, ra, np.repeat(rb, 128), with_abs=True)
    # the per-group sums are exact; only the (K/128 + 1) fp64 roundings of
    # the scaled group sums separate the two
    assert np.all(np.abs(blk - chan) <= (K // 128 + 1) * 2.0 ** -52 * absref)


def test_block_fp8_matches_numpy_expanded_scales():
    g = np.random.default_rng(12)
    M, N, K = 7, 300, 384
    A, B = rand_e4m3((M, K), g), rand_e4m3((N, K), g)
    sa = g.uniform(1e-3, 1e-2, (M, 3)).astype(np.float32)
    sb = g.uniform(1e-3, 1e-2, (3, 3)).astype(np.float32)
    ref = oracle.gemm_block_fp8(A, B, sa, sb)
    da, db = torch_dec_e4m3(A), torch_dec_e4m3(B)
    out = np.zeros((M, N))
    for gi in range(3):
        ks = slice(128 * gi, 128 * gi + 128)
        out += (da[:, ks] @ db[:, ks].T) * sa[:, gi:gi + 1].astype(np.float64) * \
            np.repeat(sb[:, gi], 128)[:N][None, :].astype(np.float64)
    np.testing.assert_allclose(ref, out, rtol=1e-12, atol=1e-300)


# ---------------------------------------------------------------- bf16
@pytest.mark.parametrize("M,N,K", [(2, 3, 9), (3, 2, 40)])
def test_bf16_fraction_bruteforce(M, N, K):
    g = np.random.default_rng([13, M, N, K])
    A = workloads.to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    B = workloads.to_bf16_bits(g.standard_normal((N, K)).astype(np.float32))
    ref = oracle.gemm_bf16(A, B)
    da, db = torch_dec_bf16(A), torch_dec_bf16(B)
    for m in range(M):
        for n in range(N):
            ex = sum(Fraction(da[m, k]) * Fraction(db[n, k]) for k in range(K))
            assert ref[m, n] == float(ex)  # short sums are exact in fp64


def test_bf16_matches_numpy():
    d = workloads.bi_inputs(160, 256, key=(workloads.W_TEST, 14))
    A = d["A_full"][:33]
    ref = oracle.gemm_bf16(A, d["B"])
    np.testing.assert_allclose(ref, torch_dec_bf16(A) @ torch_dec_bf16(d["B"]).T,
                               rtol=1e-12, atol=1e-14)
